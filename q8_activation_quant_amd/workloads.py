"""Seeded synthetic inputs for the five workloads of the shared Q8_1 activation-image path.

This module only draws random inputs (numpy PCG64 streams). It holds none of the method's
arithmetic, so the HIP path's tests and benchmark and the CPU oracle can both take their
inputs from it. Every stream is ``default_rng([1000 + config, tensor_id])``.

Workloads (sizes and distributions of the pages' component graphs, chosen per workload):
  1 tiny ordinary   T=1, K=2560, RMSNorm x gamma, two Q4_0 readers N=2560, 2560
  2 ordinary        T=8, K=8192, RMSNorm x gamma, x ~ N(0,1) with 1% of positions x20,
                    three Q4_0 readers N=8192, 1024, 1024 (q/k/v shaped)
  3 glu             T=8, packed gate|up f32 [8, 2*14336] ~ N(0,1), SwiGLU or GeGLU-erf,
                    one Q4_0 down-projection reader K=14336, N=4096
  4 routed          T=8, K=2560, E=128, top-8 distinct experts per token, gate and up
                    Q4_0 expert weights [128, 768, 2560]
  5 padded bucket   bucket 128 rows, live rows in {1, 9, 113, 114, 128}, K=2048, E=256,
                    top-9, Q4_0 expert weights [256, 512, 2048]; padding rows poisoned
  6 prefill         T=3325 prompt tokens, K=3584, RMSNorm x gamma, three Q4_0 readers
                    N=3584, 512, 512 (the q/k/v projections of a d=3584 model sharing one image)
Q4_0 weights: 4-bit codes uniform on 0..15 (uniform random bytes), fp16 block scales uniform
on [1e-3, 1e-2]. Gamma ~ N(1, 0.1), eps = 1e-6.

MoE FFN extension of the routed workloads (moe=True): the per-slot SwiGLU over the gate/up
outputs, a Q4_0 down projection per (token, slot) with expert weights [E, K, n_ff] (workload
4: n_ff 768; workload 5: n_ff 512), then the combine with the routing weights. Stage inputs
for checking each step on its own: pair_gu ~ N(0,1) [T*top_k][2*n_ff] (packed gate|up per
pair) and pair_x ~ N(0,1) [T][top_k][K] (expert outputs for the combine); router weights
~ N(0, 0.05^2) [E][K] for the device router.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids of the seeded streams
T_X, T_GAMMA, T_OUTLIER, T_GU, T_LOGITS, T_STALE_IDS, T_EXTRA = 0, 1, 2, 3, 4, 5, 6
T_PAIR_GU, T_PAIR_X, T_ROUTER = 7, 8, 9
T_READER0 = 10  # reader r uses T_READER0 + r
T_DOWN = 20     # MoE down projection

EPS = 1e-6


def rng(config: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([1000 + config, tensor_id])


@dataclass
class Q4Weights:
    """Block-quantized weights. fmt "q4_0": qs uint8 [..., N, K/32, 16], d uint16 (fp16 bits)
    [..., N, K/32]; "q8_0": qs int8 [..., N, K/32, 32], d; "q4_1": qs as q4_0, d and m."""
    qs: np.ndarray
    d: np.ndarray
    fmt: str = "q4_0"
    m: np.ndarray | None = None

    @property
    def nbytes(self) -> int:
        return self.qs.nbytes + self.d.nbytes + (0 if self.m is None else self.m.nbytes)


def q4_0_weights(g: np.random.Generator, shape_rows: tuple, K: int) -> Q4Weights:
    assert K % 32 == 0
    Kb = K // 32
    qs = g.integers(0, 256, size=(*shape_rows, Kb, 16), dtype=np.uint8)
    scales = g.uniform(1e-3, 1e-2, size=(*shape_rows, Kb)).astype(np.float16)
    return Q4Weights(qs=qs, d=scales.view(np.uint16))


def q8_0_weights(g: np.random.Generator, shape_rows: tuple, K: int) -> Q4Weights:
    """Q8_0: codes uniform on -127..127, fp16 scales uniform on [1e-4, 1e-3] (weights of the
    same spread as the Q4_0 ones)."""
    Kb = K // 32
    qs = g.integers(-127, 128, size=(*shape_rows, Kb, 32), dtype=np.int8)
    scales = g.uniform(1e-4, 1e-3, size=(*shape_rows, Kb)).astype(np.float16)
    return Q4Weights(qs=qs, d=scales.view(np.uint16), fmt="q8_0")


def q4_1_weights(g: np.random.Generator, shape_rows: tuple, K: int) -> Q4Weights:
    """Q4_1: codes uniform on 0..15, fp16 d uniform on [1e-3, 1e-2], fp16 m = -8 d (1 + u),
    u uniform on [-0.1, 0.1] (block minima near the Q4_0 offset)."""
    w = q4_0_weights(g, shape_rows, K)
    d = w.d.view(np.float16).astype(np.float64)
    m = (-8.0 * d * (1.0 + g.uniform(-0.1, 0.1, size=d.shape))).astype(np.float16)
    return Q4Weights(qs=w.qs, d=w.d, fmt="q4_1", m=m.view(np.uint16))


WEIGHT_MAKERS = {"q4_0": q4_0_weights, "q8_0": q8_0_weights, "q4_1": q4_1_weights}


def topk_ids(g: np.random.Generator, rows: int, E: int, k: int):
    """Top-k experts of N(0,1) logits per row (descending; a tie goes to the lower id) and
    softmax routing weights over the selected logits (kept for a later combine step)."""
    logits = g.standard_normal((rows, E))
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), w


@dataclass
class Workload:
    config: int
    name: str
    T: int                       # producer rows (tokens, or bucket rows)
    K: int
    producer: str                # "rmsnorm" | "swiglu" | "geglu_erf"
    x: np.ndarray | None = None  # rmsnorm input [T][K]
    gamma: np.ndarray | None = None
    gu: np.ndarray | None = None  # packed gate|up [T][2K]
    readers: list = field(default_factory=list)  # list[Q4Weights]
    E: int = 0
    top_k: int = 0
    ids: np.ndarray | None = None       # [T][top_k]
    route_w: np.ndarray | None = None   # [T][top_k]
    live: int | None = None
    extra_v: np.ndarray | None = None   # f32 vector for the extra f32 reader of workload 3
    n_ff: int = 0                       # MoE: expert hidden width (gate/up rows, down K)
    down: Q4Weights | None = None       # MoE: down projection [E, K, n_ff]
    pair_gu: np.ndarray | None = None   # MoE stage input [T*top_k][2*n_ff]
    pair_x: np.ndarray | None = None    # MoE stage input [T][top_k][K]
    router_w: np.ndarray | None = None  # MoE: router weights [E][K] f32

    @property
    def routed(self) -> bool:
        return self.E > 0

    @property
    def reader_rows(self) -> list:
        return [w.d.shape[-2] for w in self.readers]


def make(config: int, *, live: int | None = None, glu_op: str = "swiglu", small: bool = False,
         moe: bool = False, wfmt: str = "q4_0") -> Workload:
    """Build workload `config` (1..6). `small=True` shrinks the weight row counts (not K or T)
    so the CPU oracle can check every output of a GPU run in well under a second. `moe=True`
    (workloads 4 and 5) adds the down projection and the MoE stage inputs."""
    wl = _make(config, live, glu_op, small, moe)
    if wfmt != "q4_0":  # ordinary readers in another weight format (same seeds, same shapes)
        if wl.routed:
            raise ValueError("other weight formats are built for the ordinary readers")
        wl.readers = [WEIGHT_MAKERS[wfmt](rng(config, T_READER0 + r), (w.d.shape[-2],), wl.K)
                      for r, w in enumerate(wl.readers)]
        wl.name += " " + wfmt
    if moe:
        if not wl.routed:
            raise ValueError("the MoE extension needs a routed workload (4 or 5)")
        c = wl.config
        wl.down = q4_0_weights(rng(c, T_DOWN), (wl.E, wl.K if not small else 80), wl.n_ff)
        wl.pair_gu = rng(c, T_PAIR_GU).standard_normal((wl.T * wl.top_k, 2 * wl.n_ff)).astype(np.float32)
        wl.pair_x = rng(c, T_PAIR_X).standard_normal((wl.T, wl.top_k, wl.K)).astype(np.float32)
        wl.router_w = (rng(c, T_ROUTER).standard_normal((wl.E, wl.K)) * 0.05).astype(np.float32)
        wl.name += " moe-ffn n_ff%d" % wl.n_ff
    return wl


def _make(config, live, glu_op, small, moe):
    if config == 1:
        K, T = 2560, 1
        x = rng(1, T_X).standard_normal((T, K)).astype(np.float32)
        gamma = rng(1, T_GAMMA).normal(1.0, 0.1, K).astype(np.float32)
        Ns = [2560, 2560] if not small else [160, 96]
        readers = [q4_0_weights(rng(1, T_READER0 + r), (N,), K) for r, N in enumerate(Ns)]
        return Workload(1, "tiny ordinary T1 K2560", T, K, "rmsnorm", x=x, gamma=gamma, readers=readers)
    if config == 2:
        K, T = 8192, 8
        x = rng(2, T_X).standard_normal((T, K)).astype(np.float32)
        n_out = int(round(0.01 * T * K))
        pos = rng(2, T_OUTLIER).choice(T * K, size=n_out, replace=False)
        x.reshape(-1)[pos] *= np.float32(20.0)
        gamma = rng(2, T_GAMMA).normal(1.0, 0.1, K).astype(np.float32)
        Ns = [8192, 1024, 1024] if not small else [256, 64, 40]
        readers = [q4_0_weights(rng(2, T_READER0 + r), (N,), K) for r, N in enumerate(Ns)]
        return Workload(2, "ordinary K8192 T8", T, K, "rmsnorm", x=x, gamma=gamma, readers=readers)
    if config == 3:
        K, T = 14336, 8
        gu = rng(3, T_GU).standard_normal((T, 2 * K)).astype(np.float32)
        N = 4096 if not small else 96
        readers = [q4_0_weights(rng(3, T_READER0), (N,), K)]
        v = rng(3, T_EXTRA).standard_normal(K).astype(np.float32)
        return Workload(3, "glu T8 K14336 N4096 " + glu_op, T, K, glu_op, gu=gu, readers=readers,
                        extra_v=v)
    if config == 4:
        K, T, E, k = 2560, 8, 128, 8
        x = rng(4, T_X).standard_normal((T, K)).astype(np.float32)
        gamma = rng(4, T_GAMMA).normal(1.0, 0.1, K).astype(np.float32)
        N = 768 if not small else (64 if moe else 48)
        readers = [q4_0_weights(rng(4, T_READER0 + r), (E, N), K) for r in range(2)]
        ids, w = topk_ids(rng(4, T_LOGITS), T, E, k)
        return Workload(4, "routed T8 K2560 E128 top8", T, K, "rmsnorm", x=x, gamma=gamma,
                        readers=readers, E=E, top_k=k, ids=ids, route_w=w, n_ff=N)
    if config == 5:
        K, B, E, k = 2048, 128, 256, 9
        live = 128 if live is None else live
        x = rng(5, T_X).standard_normal((B, K)).astype(np.float32)
        gamma = rng(5, T_GAMMA).normal(1.0, 0.1, K).astype(np.float32)
        N = 512 if not small else (64 if moe else 40)
        readers = [q4_0_weights(rng(5, T_READER0), (E, N), K)]
        if moe:  # gate and up experts, as in workload 4
            readers.append(q4_0_weights(rng(5, T_READER0 + 1), (E, N), K))
        ids, w = topk_ids(rng(5, T_LOGITS), B, E, k)
        stale, _ = topk_ids(rng(5, T_STALE_IDS), B, E, k)
        ids[live:] = stale[live:]
        poison_rows(x, live)
        return Workload(5, "padded bucket B128 K2048 E256 top9 live%d" % live, B, K, "rmsnorm",
                        x=x, gamma=gamma, readers=readers, E=E, top_k=k, ids=ids, route_w=w,
                        live=live, n_ff=N)
    if config == 6:
        K, T = 3584, 3325
        x = rng(6, T_X).standard_normal((T, K)).astype(np.float32)
        gamma = rng(6, T_GAMMA).normal(1.0, 0.1, K).astype(np.float32)
        Ns = [3584, 512, 512] if not small else [96, 32, 40]
        readers = [q4_0_weights(rng(6, T_READER0 + r), (N,), K) for r, N in enumerate(Ns)]
        return Workload(6, "prefill T3325 K3584", T, K, "rmsnorm", x=x, gamma=gamma, readers=readers)
    raise ValueError("config must be 1..6")


POISON = (np.float32(np.nan), np.float32(1e30), np.float32(-1e30))


def poison_rows(x: np.ndarray, live: int, phase: int = 0) -> None:
    """Fill rows >= live with NaN, +1e30 and -1e30 in turn (rows cycle through the three)."""
    for i in range(live, x.shape[0]):
        x[i, :] = POISON[(i + phase) % 3]
