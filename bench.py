"""Benchmark of the shared Q8_1 activation-image path on one MI355X.

A step is one component graph: the fused producer writes the f32 output and the Q8_1 image,
then the Q4_0 readers consume the image. Default workload: T=8 tokens, K=8192, RMSNorm x gamma,
three readers N=8192/1024/1024 (the ordinary K8192/T8 component graph).

Timing: a HIP graph holds R instances of the step, each with its own copy of every tensor,
with R x weights >= 1 GiB so replays stream weights from HBM rather than from the 256 MB
Infinity Cache (the instances repeat in order until the graph holds at least 32 steps). W
warmup steps, then exactly K timed steps, bracketed by synchronisation. The reader kernel is
also timed alone (a graph of reader launches over the same instances) for the roofline line,
beside a plain streaming read of the same byte count (the measured ceiling). The GLU workload's
graph includes its extra f32 reader of the kept output, also timed alone.
--moe times the whole routed MoE FFN of the routed workloads the same way.
The CPU baseline is the plain oracle on the host on a bounded sample, on all the threads this
process may use (at most 16; each reader's output rows split over them) and on one thread.
--pmc-probe and --pmc-summarize take and summarise the reader's HBM counters (rocprofv3).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 matrix-core rate, published (no sparsity)
ROT_BYTES = 1 << 30


def _t():
    import torch
    return torch


class Instance:
    """Device tensors of one copy of a workload's component graph."""

    def __init__(self, wl, host_dev_cache=None):
        from q8_activation_quant_amd import qimg
        torch = _t()
        self.wl = wl
        T, K = wl.T, wl.K
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
        if wl.producer == "rmsnorm":
            self.x = dev(wl.x)
            self.gamma = dev(wl.gamma)
        else:
            self.gu = dev(wl.gu)
        self.y = torch.empty(T, K, dtype=torch.float32, device="cuda")
        self.img = torch.empty(qimg.image_bytes(T, K), dtype=torch.uint8, device="cuda")
        self.live = torch.tensor([wl.live if wl.live is not None else T], dtype=torch.int32, device="cuda")
        self.specs = []
        for r in wl.readers:
            N = r.d.shape[-2]
            out = torch.empty(*((T, wl.top_k, N) if wl.routed else (T, N)), dtype=torch.float32, device="cuda")
            tiles = qimg.tile_weights(dev(r.qs.view(np.uint8)), dev(r.d), K, fmt=r.fmt,
                                      w_m=None if r.m is None else dev(r.m))
            self.specs.append((tiles, N, out))
        if wl.routed:
            self.ids = dev(wl.ids)
            self.ws = torch.empty(qimg.workspace_bytes(T, wl.top_k, wl.E) // 4, dtype=torch.int32, device="cuda")
        self.v = dev(wl.extra_v.reshape(1, K)) if wl.extra_v is not None else None
        self.fo = torch.empty(T, 1, dtype=torch.float32, device="cuda") if self.v is not None else None
        self.ceil_buf = None

    def extra(self):
        """The extra f32 reader of the kept producer output (the GLU workload)."""
        from q8_activation_quant_amd import qimg
        live = self.live if self.wl.live is not None else None
        qimg.f32_reader(self.y, self.v, self.fo, live)

    def ceiling(self):
        """A plain streaming read of as many bytes as the reader launch moves (its own buffer)."""
        from q8_activation_quant_amd import qimg
        qimg.read_ceiling(self.ceil_buf, self.ceil_sink)

    def produce(self, with_img=True):
        from q8_activation_quant_amd import qimg
        wl = self.wl
        img = self.img if with_img else None
        live = self.live if wl.routed or wl.live is not None else None
        if wl.producer == "rmsnorm":
            qimg.emit_rmsnorm(self.x, self.gamma, 1e-6, self.y, img, live)
        else:
            K = wl.K
            qimg.emit_glu_ex(wl.producer, self.gu[:, :K], self.gu[:, K:], self.y, img, live)

    def quantize(self):
        from q8_activation_quant_amd import qimg
        live = self.live if self.wl.routed or self.wl.live is not None else None
        qimg.quantize_q8_1(self.y, self.img, live)

    def read(self):
        from q8_activation_quant_amd import qimg
        wl = self.wl
        if wl.routed:
            qimg.mmvq_id(self.specs, wl.E, self.img, self.ids, self.live, wl.K, self.ws)
        else:
            qimg.mmvq(self.specs, self.img, wl.T, wl.K, fmt=wl.readers[0].fmt)

    def step(self, arm="fused"):
        if arm == "fused":
            self.produce(True)
        else:  # control: producer keeps only f32, then the separate quantizer launch
            self.produce(False)
            self.quantize()
        self.read()
        if self.v is not None:
            self.extra()


def algorithmic_bytes(wl):
    """Bytes the method must move per component graph: producer inputs read, f32 output
    written, image written once and read once, the distinct weights read once (routed: only
    the experts some live pair selects), ids read, outputs written."""
    from q8_activation_quant_amd import qimg
    T, K = wl.T, wl.K
    L = wl.live if wl.live is not None else T
    Kb = K // 32
    prod = (2 * L * K * 4) if wl.producer != "rmsnorm" else (L * K * 4 + K * 4)
    prod += L * K * 4                      # f32 output
    img = L * Kb * 36                      # image bytes written (= read) for live rows
    if wl.routed:
        used = np.unique(wl.ids[:L].reshape(-1))
        w = sum(len(used) * r.d.shape[-2] * Kb * 18 for r in wl.readers)
        out = sum(L * wl.top_k * r.d.shape[-2] * 4 for r in wl.readers)
        ids = L * wl.top_k * 4
    else:
        per_block = {"q4_0": 18, "q8_0": 34, "q4_1": 20}
        w = sum(r.d.shape[-2] * Kb * per_block[r.fmt] for r in wl.readers)
        out = sum(L * r.d.shape[-2] * 4 for r in wl.readers)
        ids = 0
    # the GLU workload's extra f32 reader: the kept output and the vector read, one f32 per row
    extra = (L * K * 4 + K * 4 + L * 4) if wl.extra_v is not None else 0
    return {"producer": prod, "image_write": img, "image_read": img, "weights": w, "outputs": out,
            "ids": ids, "extra_f32_reader": extra, "total": prod + 2 * img + w + out + ids + extra,
            "reader_kernel": img + w + out + ids}


class MoeInstance:
    """Device tensors of one routed MoE FFN: RMS producer + image -> device router (reading the
    kept f32 output) and top-k -> gate/up experts -> per-slot SwiGLU + image -> per-slot down
    experts -> combine with the routing weights."""

    def __init__(self, wl):
        from q8_activation_quant_amd import qimg
        torch = _t()
        self.wl = wl
        B, k, K, F = wl.T, wl.top_k, wl.K, wl.n_ff
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
        self.x, self.gamma = dev(wl.x), dev(wl.gamma)
        self.ids, self.w = dev(wl.ids), dev(wl.route_w)
        self.live = torch.tensor([wl.live if wl.live is not None else B], dtype=torch.int32, device="cuda")
        f32 = lambda *sh: torch.empty(*sh, dtype=torch.float32, device="cuda")
        self.y, self.img = f32(B, K), torch.empty(qimg.image_bytes(B, K), dtype=torch.uint8, device="cuda")
        self.gate, self.up, self.h = f32(B, k, F), f32(B, k, F), f32(B, k, F)
        self.himg = torch.empty(qimg.image_bytes(B * k, F), dtype=torch.uint8, device="cuda")
        self.down, self.out = f32(B, k, K), f32(B, K)
        ws = qimg.workspace_bytes(B, k, wl.E) // 4
        self.ws1 = torch.empty(ws, dtype=torch.int32, device="cuda")
        self.ws2 = torch.empty(ws, dtype=torch.int32, device="cuda")
        self.wg = qimg.tile_q4_0(dev(wl.readers[0].qs), dev(wl.readers[0].d), K)
        self.wu = qimg.tile_q4_0(dev(wl.readers[1].qs), dev(wl.readers[1].d), K)
        self.wd = qimg.tile_q4_0(dev(wl.down.qs), dev(wl.down.d), F)
        # device routing: router weights, logits; the top-k rewrites ids and routing weights
        self.rw = dev(wl.router_w)
        self.logits = f32(B, wl.E)

    def produce(self):
        from q8_activation_quant_amd import qimg
        qimg.emit_rmsnorm(self.x, self.gamma, 1e-6, self.y, self.img, self.live)

    def route(self):
        from q8_activation_quant_amd import qimg
        qimg.moe_router(self.y, self.rw, self.logits, self.live)
        qimg.moe_topk(self.logits, self.ids, self.w, self.live)

    def gate_up(self):
        from q8_activation_quant_amd import qimg
        wl = self.wl
        qimg.mmvq_id([(self.wg, wl.n_ff, self.gate), (self.wu, wl.n_ff, self.up)], wl.E, self.img, self.ids,
                     self.live, wl.K, self.ws1)

    def glu(self):
        from q8_activation_quant_amd import qimg
        qimg.emit_glu_per_slot("swiglu", self.gate, self.up, self.h, self.himg, self.live)

    def down_proj(self):
        from q8_activation_quant_amd import qimg
        wl = self.wl
        qimg.mmvq_id_per_slot([(self.wd, wl.K, self.down)], wl.E, self.himg, self.ids, self.live, wl.n_ff,
                              self.ws2)

    def combine(self):
        from q8_activation_quant_amd import qimg
        qimg.moe_combine(self.down, self.w, self.ids, self.wl.E, self.out, self.live)

    def step(self):
        self.produce()
        self.route()
        self.gate_up()
        self.glu()
        self.down_proj()
        self.combine()


def moe_bytes(wl, ids):
    """Algorithmic bytes of one MoE FFN (live rows L, pairs P = L top_k, distinct experts U):
    x, gamma read, y written, token image written and read; the router reading y and its f32
    weights and writing the logits, the top-k reading them and writing ids and routing
    weights; gate/up weights of U experts; ids
    read by both routed launches; gate/up outputs written and read by the GLU; h written; the
    per-slot image written and read; down weights of U experts; down outputs written and read
    by the combine; routing weights and ids read by the combine; the output written."""
    B, k, K, F = wl.T, wl.top_k, wl.K, wl.n_ff
    L = wl.live if wl.live is not None else B
    P = L * k
    U = len(np.unique(ids[:L].reshape(-1)))  # the experts the device router picked
    img_tok = L * (K // 32) * 36
    img_pair = P * (F // 32) * 36
    E = wl.E
    parts = {
        "producer": L * K * 4 + K * 4 + L * K * 4 + img_tok,
        "route": L * K * 4 + E * K * 4 + 2 * L * E * 4 + 2 * P * 4,
        "gate_up": img_tok + U * 2 * F * (K // 32) * 18 + P * 4 + 2 * P * F * 4,
        "glu": 2 * P * F * 4 + P * F * 4 + img_pair,
        "down": img_pair + U * K * (F // 32) * 18 + P * 4 + P * K * 4,
        "combine": P * K * 4 + 2 * P * 4 + L * K * 4,
    }
    parts["total"] = sum(parts.values())
    return parts


def run_moe(config, steps, warmup, live=None):
    torch = _t()
    from q8_activation_quant_amd import workloads as W
    wl = W.make(config, live=live, moe=True)
    wbytes = sum(r.nbytes for r in wl.readers) + wl.down.nbytes
    R = max(1, int(np.ceil(ROT_BYTES / wbytes)))
    insts = [MoeInstance(wl) for _ in range(R)]
    insts[0].step()
    torch.cuda.synchronize()
    res = {"wl": wl, "R": R, "bytes": moe_bytes(wl, insts[0].ids.cpu().numpy())}
    res["us"] = time_graph([i.step for i in insts], steps, warmup)
    for part in ("produce", "route", "gate_up", "glu", "down_proj", "combine"):
        res[part] = float(np.median(time_graph([getattr(i, part) for i in insts], steps, warmup)))
    del insts
    torch.cuda.empty_cache()
    return res


def weight_bytes(wl):
    return sum(r.qs.nbytes + r.d.nbytes for r in wl.readers)


def make_instances(wl, rot_bytes=ROT_BYTES):
    R = max(1, int(np.ceil(rot_bytes / max(weight_bytes(wl), 1))))
    return [Instance(wl) for _ in range(R)]


MIN_GRAPH_CALLS = 32


def time_graph(fns, steps, warmup, runs=3):
    """Capture fns (one call per instance, repeated in order until the graph holds at least
    MIN_GRAPH_CALLS calls, so a replay's fixed launch cost is spread over many calls) in one
    graph; replay to cover `warmup` then exactly `steps` calls (a remainder graph covers steps
    not divisible by the graph's call count). Returns the per-call microseconds of each run."""
    torch = _t()
    fns = list(fns) * max(1, -(-MIN_GRAPH_CALLS // len(fns)))
    R = len(fns)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    rem = steps % R
    g_rem = None
    if rem:
        g_rem = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_rem):
            for f in fns[:rem]:
                f()
    for _ in range(max(1, int(np.ceil(warmup / R)))):
        g.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(runs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps // R):
            g.replay()
        if g_rem is not None:
            g_rem.replay()
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) * 1e3 / steps)
    return res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Host threads for the all-cores oracle run: the CPUs this process may use, at most 16 (a
    one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, budget_s=10.0, threads=1):
    """The plain oracle over the same component graph on `threads` host threads: the producer,
    the quantizer (and the routing plan) on one, each reader's output rows split into `threads`
    contiguous slices run in parallel (the oracle's C readers run with the interpreter lock
    released; slices are cut before timing). Returns (us per graph, median; graphs timed)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as O
    T, K = wl.T, wl.K
    L = wl.live if wl.live is not None else T
    jobs = []
    for r in wl.readers:
        N = r.d.shape[-2]
        bounds = np.linspace(0, N, threads + 1).astype(int)
        for a, b in zip(bounds[:-1], bounds[1:]):
            if b <= a:
                continue
            if wl.routed:
                jobs.append(("id", np.ascontiguousarray(r.qs[:, a:b]), np.ascontiguousarray(r.d[:, a:b]), None))
            else:
                jobs.append((r.fmt, r.qs[a:b], r.d[a:b], None if r.m is None else r.m[a:b]))

    def run_job(job, img):
        kind, qs, d, m = job
        if kind == "id":
            O.mmvq_id(qs, d, wl.E, K, img, T, wl.ids, L)
        elif kind == "q4_0":
            O.mmvq(qs, d, K, img, T, L)
        else:
            O.mmvq_fmt(kind, qs, d, m, K, img, T, L)

    pool = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None
    times = []
    t_end = time.perf_counter() + budget_s
    try:
        while True:
            t0 = time.perf_counter()
            if wl.producer == "rmsnorm":
                y = O.rmsnorm(wl.x[:L], wl.gamma, 1e-6)
            else:
                y = O.glu_ex(wl.gu[:L, :K], wl.gu[:L, K:], wl.producer)
            img = O.quantize(y, img_rows=T)
            if wl.routed:
                O.plan(wl.ids, L, wl.E)
            if pool is not None:
                list(pool.map(lambda j: run_job(j, img), jobs))
            else:
                for j in jobs:
                    run_job(j, img)
            if wl.extra_v is not None:
                O.moe_router(y, wl.extra_v.reshape(1, K), L)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() + times[-1] > t_end or len(times) >= 24:
                break
    finally:
        if pool is not None:
            pool.shutdown()
    return float(np.median(times)) * 1e6, len(times)


def kernel_source_hash():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "q8_activation_quant_amd", "csrc", "qimg.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def pmc_file(config, live=None, wfmt="q4_0"):
    """Name (under profiles/) of the counter summary of a workload's reader kernel, or None."""
    if wfmt != "q4_0":
        return None
    names = {1: "mmvq_t1_k2560", 2: "mmvq_k8192_t8", 3: "mmvq_glu_t8_k14336_n4096",
             4: "mmvq_routed_t8_k2560_e128_gate_up", 6: "mmq_prefill_t3325_k3584"}
    if config == 5:
        return "mmvq_routed_bucket128_k2048_e256_live%d_pmc" % (live if live is not None else 128)
    return names[config] + "_pmc" if config in names and live is None else None


def pmc_traffic(config, live=None, wfmt="q4_0"):
    """HBM bytes per reader launch from the committed rocprofv3 --pmc summary of the workload,
    or None when there is none or the kernel source changed since the counters were taken."""
    name = pmc_file(config, live, wfmt)
    path = os.path.join(ROOT, "profiles", name + ".json") if name else None
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_rows(path):
    """(dispatch id, kernel name, counter, value) rows of a rocprofv3 counter_collection CSV
    (a file, or the directory rocprofv3 wrote it under)."""
    import csv
    import glob
    if os.path.isdir(path):
        hits = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
        if not hits:
            raise SystemExit("no counter_collection.csv under %s" % path)
        path = hits[-1]
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def pmc_summarize(config, live, fetch_path, write_path, out_dir=None):
    """Write profiles/<name>.json and .md from the two counter runs of --pmc-probe: HBM bytes
    per reader launch = counter KiB x 1024 x the scale that makes the plain copy's counters
    equal its known bytes."""
    from q8_activation_quant_amd import workloads as W
    wl = W.make(config, live=live)
    algo = algorithmic_bytes(wl)["reader_kernel"]
    name = pmc_file(config, live)
    res = {}
    for cname, path in (("FETCH_SIZE", fetch_path), ("WRITE_SIZE", write_path)):
        per = {}
        for disp, kname, c, v in _counter_rows(path):
            if c == cname:
                per.setdefault(disp, [kname, 0.0])[1] += v
        reader = [v for k, v in per.values() if "mmvq_" in k or "mmq_kernel" in k]
        copy = [v for k, v in per.values() if "copyBuffer" in k]
        kn = sorted({k for k, v in per.values() if "mmvq_" in k or "mmq_kernel" in k})
        if not reader or not copy:
            raise SystemExit("%s: reader or calibration dispatches missing" % cname)
        res[cname] = {"reader_kib_avg": float(np.mean(reader)), "dispatches": len(reader),
                      "copy_kib": float(copy[-1]), "kernel": kn[0] if kn else None}
    copy_bytes = 256 << 20
    rs = copy_bytes / (res["FETCH_SIZE"]["copy_kib"] * 1024)
    ws = copy_bytes / (res["WRITE_SIZE"]["copy_kib"] * 1024)
    rd = res["FETCH_SIZE"]["reader_kib_avg"] * 1024 * rs
    wr = res["WRITE_SIZE"]["reader_kib_avg"] * 1024 * ws
    probe = "python3 bench.py --pmc-probe --config %d%s" % (config, "" if live is None else " --live %d" % live)
    d = {"kernel_name_in_trace": res["FETCH_SIZE"]["kernel"], "workload": WORKLOAD_NAMES[config],
         "live_rows": live, "kernel_source_sha256_16": kernel_source_hash(),
         "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_f -o fetch -- " + probe,
                      "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_w -o write -- " + probe],
         "calibration": {"kernel": "__amd_rocclr_copyBuffer, %d-byte device copy" % copy_bytes,
                         "FETCH_SIZE_KiB": res["FETCH_SIZE"]["copy_kib"], "WRITE_SIZE_KiB": res["WRITE_SIZE"]["copy_kib"],
                         "read_scale": round(rs, 5), "write_scale": round(ws, 5)},
         "reader_dispatches": res["FETCH_SIZE"]["dispatches"],
         "reader_FETCH_SIZE_KiB_avg": round(res["FETCH_SIZE"]["reader_kib_avg"], 1),
         "reader_WRITE_SIZE_KiB_avg": round(res["WRITE_SIZE"]["reader_kib_avg"], 1),
         "hbm_read_bytes_per_launch": int(round(rd)), "hbm_write_bytes_per_launch": int(round(wr)),
         "hbm_bytes_per_launch": int(round(rd + wr)), "algorithmic_bytes_per_launch": int(algo)}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, name + ".json"), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    md = ["# HBM traffic of the reader kernel: %s%s" % (WORKLOAD_NAMES[config],
                                                        "" if live is None else ", live rows %d" % live),
          "", "Commands (one counter per run; `--pmc-probe` launches the reader once per rotated",
          "instance, then a plain 256 MiB device copy that calibrates the counters):", ""]
    md += ["    " + c for c in d["commands"]]
    md += ["", "| kernel | FETCH_SIZE KiB / dispatch | WRITE_SIZE KiB / dispatch |", "|---|---|---|",
           "| __amd_rocclr_copyBuffer (%d B copy) | %.1f | %.1f |" % (copy_bytes, res["FETCH_SIZE"]["copy_kib"],
                                                                   res["WRITE_SIZE"]["copy_kib"]),
           "| %s (avg of %d) | %.1f | %.1f |" % (d["kernel_name_in_trace"], d["reader_dispatches"],
                                                d["reader_FETCH_SIZE_KiB_avg"], d["reader_WRITE_SIZE_KiB_avg"]),
           "", "Scales from the copy: read %.5f, write %.5f." % (rs, ws),
           "Reader per launch: %.3f MB read + %.3f MB written = %.3f MB against %d algorithmic bytes "
           "(%+.1f%%)." % (rd / 1e6, wr / 1e6, (rd + wr) / 1e6, algo, 100 * ((rd + wr) / algo - 1)),
           "Kernel source hash (first 16 hex of SHA-256 of qimg.hip): %s." % d["kernel_source_sha256_16"], ""]
    with open(os.path.join(out_dir, name + ".md"), "w") as f:
        f.write("\n".join(md))
    return d


WORKLOAD_NAMES = {
    1: "tiny ordinary: T1 K2560 RMSNorm x gamma -> Q8_1 image -> 2 Q4_0 readers N2560",
    2: "ordinary K8192/T8: RMSNorm x gamma -> Q8_1 image -> 3 Q4_0 readers N8192/1024/1024",
    3: "GLU T8: SwiGLU over packed gate|up [8, 2x14336] -> Q8_1 image -> Q4_0 down reader N4096",
    4: "routed T8 K2560 E128 top8: RMSNorm x gamma -> image -> gate+up Q4_0 experts [128,768,2560]",
    5: "padded bucket 128 K2048 E256 top9: RMSNorm x gamma -> image -> Q4_0 experts [256,512,2048]",
    6: "prefill T3325 K3584: RMSNorm x gamma -> Q8_1 image -> 3 Q4_0 readers N3584/512/512 (matrix-core prefill reader)",
}


def run(config, steps, warmup, live=None, glu_op="swiglu", want_cpu=True, arms=("fused", "control"),
        wfmt="q4_0", want_ceiling=True):
    torch = _t()
    from q8_activation_quant_amd import workloads as W
    wl = W.make(config, live=live, glu_op=glu_op, wfmt=wfmt)
    insts = make_instances(wl)
    nb = algorithmic_bytes(wl)
    per_arm = {}
    # ABBA over the two arms
    order = list(arms) + list(reversed(arms)) if len(arms) > 1 else list(arms)
    for arm in order:
        us = time_graph([(lambda i=i, a=arm: i.step(a)) for i in insts], steps, warmup)
        per_arm.setdefault(arm, []).extend(us)
    kern = time_graph([i.read for i in insts], steps, warmup)
    prod = time_graph([(lambda i=i: i.produce(True)) for i in insts], steps, warmup)
    res = {
        "wl": wl, "R": len(insts), "bytes": nb,
        "us": {a: float(np.median(v)) for a, v in per_arm.items()},
        "us_range": {a: [float(min(v)), float(max(v))] for a, v in per_arm.items()},
        "reader_us": float(np.median(kern)), "producer_us": float(np.median(prod)),
    }
    if wl.extra_v is not None:
        res["extra_us"] = float(np.median(time_graph([i.extra for i in insts], steps, warmup)))
    del insts
    torch.cuda.empty_cache()
    if want_ceiling:
        res["ceiling_us"], res["ceiling_bytes"] = time_ceiling(nb["reader_kernel"], steps, warmup)
    if want_cpu:
        res["cpu_us"], res["cpu_reps"] = cpu_baseline(wl, threads=1)
        res["cpu_threads"] = cpu_threads()
        res["cpu_all_us"], res["cpu_all_reps"] = cpu_baseline(wl, threads=res["cpu_threads"])
    return res


def time_ceiling(nbytes, steps, warmup):
    """Per-launch microseconds of the plain streaming read of nbytes (rounded up to 1 KB) over
    rotated buffers of at least ROT_BYTES in all, so every launch reads HBM."""
    torch = _t()
    from q8_activation_quant_amd import qimg
    nb = -(-int(nbytes) // 1024) * 1024
    R = max(2, -(-ROT_BYTES // nb))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.empty(qimg.CEILING_SINK_WORDS, dtype=torch.int32, device="cuda")
    us = time_graph([(lambda b=b: qimg.read_ceiling(b, sink)) for b in bufs], steps, warmup)
    del bufs
    torch.cuda.empty_cache()
    return float(np.median(us)), nb


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4600)
    ap.add_argument("--warmup", type=int, default=460)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--live", type=int, default=None)
    ap.add_argument("--glu", default="swiglu", choices=["swiglu", "geglu_erf", "reglu", "geglu", "geglu_quick",
                                                        "swiglu_oai", "swiglu_clamp"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--all", action="store_true", help="also print one extra line per workload")
    ap.add_argument("--wfmt", default="q4_0", choices=["q4_0", "q8_0", "q4_1"],
                    help="weight format of the ordinary readers")
    ap.add_argument("--moe", action="store_true",
                    help="time the whole routed MoE FFN of workload 4 (or 5 with --config 5) instead")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="counter-collection run: one reader launch per rotated instance of the "
                         "workload, then a plain 256 MiB device copy (the calibration kernel)")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH", "WRITE"),
                    help="write the workload's counter summary under profiles/ from the rocprofv3 "
                         "output (CSV file or directory) of the FETCH_SIZE and WRITE_SIZE runs")
    args = ap.parse_args()
    if args.pmc_summarize:
        print(json.dumps(pmc_summarize(args.config, args.live if args.config == 5 else None,
                                       *args.pmc_summarize)), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see the design notes "
              "for how it would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch = _t()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from q8_activation_quant_amd import qimg
    qimg.lib()

    if args.moe:
        cfg = args.config if args.config in (4, 5) else 4
        r = run_moe(cfg, args.steps, args.warmup, live=args.live)
        wl, nb = r["wl"], r["bytes"]
        us = float(np.median(r["us"]))
        down_gbs = nb["down"] / (r["down_proj"] * 1e-6) / 1e9
        print(json.dumps({
            "metric": "us per routed MoE FFN + achieved HBM GB/s (% of peak), 1 MI355X",
            "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": "int8xu4->int32 dots, f32 producers, accumulation and combine",
            "data": "synthetic (seeded numpy PCG64; shapes/distributions of the workload)",
            "config": {"workload": wl.name, "T": wl.T, "K": wl.K, "E": wl.E, "top_k": wl.top_k,
                       "n_ff": wl.n_ff, "live_rows": wl.live, "graph_instances": r["R"]},
            "us_range": [round(min(r["us"]), 3), round(max(r["us"]), 3)],
            "algorithmic_bytes": nb,
            "achieved_GBs": round(nb["total"] / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * nb["total"] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
            "launch_us": {p: round(r[p], 3) for p in ("produce", "route", "gate_up", "glu", "down_proj", "combine")},
            "roofline": {"bound": "hbm", "kernel": "mmvq_routed_kernel (per-slot down projection)",
                         "achieved": round(down_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(down_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "bytes_per_launch": nb["down"], "avg_launch_us": round(r["down_proj"], 3)},
        }), flush=True)
        return
    if args.pmc_probe:
        from q8_activation_quant_amd import workloads as W
        wl = W.make(args.config, live=args.live, glu_op=args.glu)
        insts = make_instances(wl)
        for i in insts:
            i.produce(True)
        torch.cuda.synchronize()
        for i in insts:
            i.read()
        torch.cuda.synchronize()
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": WORKLOAD_NAMES[args.config], "reader_launches": len(insts),
                          "reader_algorithmic_bytes": algorithmic_bytes(wl)["reader_kernel"],
                          "calibration_copy_bytes": src.numel()}), flush=True)
        return
    r = run(args.config, args.steps, args.warmup, live=args.live, glu_op=args.glu, want_cpu=not args.no_cpu,
            wfmt=args.wfmt)
    wl, nb = r["wl"], r["bytes"]
    us = r["us"]["fused"]
    reader_gbs = nb["reader_kernel"] / (r["reader_us"] * 1e-6) / 1e9
    traffic = pmc_traffic(args.config, wl.live if args.config == 5 else args.live, args.wfmt)
    ceil_gbs = r["ceiling_bytes"] / (r["ceiling_us"] * 1e-6) / 1e9
    line = {
        "metric": "us per component graph + achieved HBM GB/s (% of peak), 1 MI355X",
        "value": round(us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xu4->int32 dots, f32 producer and accumulation",
        "data": "synthetic (seeded numpy PCG64; shapes/distributions of the workload)",
        "config": {"workload": WORKLOAD_NAMES[args.config] + ("" if wl.producer in ("rmsnorm", "swiglu")
                                                              else " (producer %s)" % wl.producer)
                               + ("" if args.wfmt == "q4_0" else " (weights %s)" % args.wfmt),
                   "T": wl.T, "K": wl.K,
                   "readers_N": wl.reader_rows, "producer": wl.producer, "arm": "fused",
                   "graph_instances": r["R"], "live_rows": wl.live},
        "achieved_GBs": round(nb["total"] / (us * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * nb["total"] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
        "algorithmic_bytes": nb["total"],
        "control_us": round(r["us"].get("control", float("nan")), 3),
        "less_gpu_time_vs_control_pct": round(100 * (1 - us / r["us"]["control"]), 2) if "control" in r["us"] else None,
        "us_range": r["us_range"],
        "producer_us": round(r["producer_us"], 3),
        "roofline": {
            "bound": "hbm",
            "kernel": ("mmq_kernel (Q4_0 x Q8_1 prefill readers)" if args.config == 6 else
                       "mmvq_tiled_kernel (%s x Q8_1 readers)" % args.wfmt.upper()),
            "achieved": round(reader_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(reader_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": nb["reader_kernel"],
            "avg_launch_us": round(r["reader_us"], 3),
            # the plain streaming read of the same byte count (read_ceiling_kernel, one launch
            # per rotated buffer): what this GPU reaches on a contiguous read of that size
            "measured_ceiling": {"achieved": round(ceil_gbs, 1), "unit": "GB/s",
                                 "frac_of_peak": round(ceil_gbs / PEAK_HBM_GBS, 4),
                                 "reader_frac_of_ceiling": round(reader_gbs / ceil_gbs, 4),
                                 "avg_launch_us": round(r["ceiling_us"], 3), "bytes_per_launch": r["ceiling_bytes"]},
        },
    }
    if "extra_us" in r:
        line["extra_f32_reader"] = {"avg_launch_us": round(r["extra_us"], 3),
                                    "bytes_per_launch": nb["extra_f32_reader"],
                                    "GBs": round(nb["extra_f32_reader"] / (r["extra_us"] * 1e-6) / 1e9, 1)}
    if args.config == 6:
        # the prefill reader is bound by its per-block scaling on the vector ALUs: 2 operations
        # (convert the block's int32 dot, one fused multiply-add by d_w d_a, which the matrix
        # cores supply) per (image row, weight row, block), against the unpacked f32 vector
        # rate of 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
        ops = 2.0 * wl.T * sum(wl.reader_rows) * (wl.K // 32)
        peak = 256 * 4 * 16 * 2.4e9 / 1e12
        ach = ops / (r["reader_us"] * 1e-6) / 1e12
        # its int8 products: 2 T K N operations against the dense int8 matrix-core peak
        i8 = 2.0 * wl.T * sum(wl.reader_rows) * wl.K / (r["reader_us"] * 1e-6) / 1e12
        # the vector-ALU roofline is the one that bounds it; its HBM view is kept beside it
        hbm = line["roofline"]
        line["roofline"] = {"bound": "alu", "kernel": hbm["kernel"], "achieved": round(ach, 2),
                            "peak": round(peak, 2), "unit": "Tops/s", "frac": round(ach / peak, 4),
                            "traffic": hbm["traffic"], "ops_per_launch": ops,
                            "avg_launch_us": round(r["reader_us"], 3),
                            "int8_mfma": {"achieved": round(i8, 1), "peak": PEAK_INT8_TOPS,
                                          "unit": "Tops/s", "frac": round(i8 / PEAK_INT8_TOPS, 4)},
                            "hbm": {k: v for k, v in hbm.items() if k not in ("kernel", "traffic")}}
    if "cpu_us" in r:
        line["cpu_baseline"] = {"value": round(r["cpu_all_us"], 1), "unit": "us", "cores": r["cpu_threads"],
                                "kind": "oracle",
                                "sample": "%d full component graph(s) of the same workload (median); readers' "
                                          "output rows split over the threads" % r["cpu_all_reps"],
                                "single_thread": {"value": round(r["cpu_us"], 1), "cores": 1,
                                                  "sample": "%d full component graph(s) (median)" % r["cpu_reps"]},
                                "nproc": os.cpu_count(), "cpu_model": cpu_model()}
    print(json.dumps(line), flush=True)
    if args.all:
        for c, live in [(1, None), (3, None), (4, None), (5, 1), (5, 9), (5, 113), (5, 114), (5, 128)]:
            rr = run(c, args.steps, args.warmup, live=live, want_cpu=False)
            nb2 = rr["bytes"]
            u2 = rr["us"]["fused"]
            print(json.dumps({"workload": WORKLOAD_NAMES[c], "live": live, "fused_us": round(u2, 3),
                              "control_us": round(rr["us"]["control"], 3),
                              "reader_us": round(rr["reader_us"], 3), "producer_us": round(rr["producer_us"], 3),
                              "algorithmic_bytes": nb2["total"],
                              "GBs": round(nb2["total"] / (u2 * 1e-6) / 1e9, 1),
                              "pct_hbm": round(100 * nb2["total"] / (u2 * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
                              "reader_GBs": round(nb2["reader_kernel"] / (rr["reader_us"] * 1e-6) / 1e9, 1)}),
                  flush=True)


if __name__ == "__main__":
    main()
