"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bars: f32 producer outputs, Q8_1 image bytes (codes, half scales/sums, padding), per-block
int32 dots and routed plans bit-exact; reader outputs within normwise relative error 1e-5 of
the float64 oracle and within the per-element rounding bound; NMSE against the unquantized
float64 activation <= 5e-4. Rows past the live count are never written (sentinel bytes stay).
"""
import numpy as np
import pytest

import helpers as H
from oracle import oracle as O
from q8_activation_quant_amd import qimg
from q8_activation_quant_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = H.torch()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qimg.lib()  # raises when the HIP library is missing
    yield
    torch.cuda.synchronize()


def sync():
    H.torch().cuda.synchronize()


def split_image(img, rows, K):
    RB = qimg.row_blocks(K)
    return img[: rows * RB * 32].reshape(rows, RB * 32), img[rows * RB * 32: rows * RB * 36].reshape(rows, RB * 4)


def run_producer(wl, live=None, with_img=True, pass_live=False, x=None, gu=None):
    """Run the fused producer on sentinel-filled outputs; returns host (y, img)."""
    T, K = wl.T, wl.K
    y = H.sentinel_f32(T, K)
    img = H.sentinel_u8(qimg.image_bytes(T, K)) if with_img else None
    lt = H.live_tensor(live) if (pass_live or live is not None) else None
    if wl.producer == "rmsnorm":
        xd = H.dev(wl.x if x is None else x)
        qimg.emit_rmsnorm(xd, H.dev(wl.gamma), W.EPS, y, img, lt)
    else:
        gd = H.dev(wl.gu if gu is None else gu)
        qimg.emit_glu(wl.producer, gd[:, :K], gd[:, K:], y, img, lt)
    sync()
    return H.host(y), (None if img is None else H.host(img))


def check_producer(wl, y, img, live=None):
    live = wl.T if live is None else live
    y_o, img_o = H.oracle_producer(wl, live)
    assert np.array_equal(y[:live].view(np.uint32), y_o.view(np.uint32)), "f32 producer output differs"
    assert (y[live:].view(np.uint8) == H.SENTINEL_BYTE).all(), "padding rows of y were written"
    if img is not None:
        c, d = split_image(img, wl.T, wl.K)
        co, do = split_image(img_o, wl.T, wl.K)
        assert np.array_equal(c[:live], co[:live]), "image codes differ"
        assert np.array_equal(d[:live], do[:live]), "image scales/sums differ"
        assert (c[live:] == H.SENTINEL_BYTE).all() and (d[live:] == H.SENTINEL_BYTE).all(), \
            "padding rows of the image were written"
    return y_o, img_o


# ---- producers ---------------------------------------------------------------------------------
@pytest.mark.parametrize("config", [1, 2, 4])
def test_emit_rmsnorm_bit_exact(config):
    wl = W.make(config, small=True)
    print("emit_rmsnorm config", config, flush=True)
    y, img = run_producer(wl)
    check_producer(wl, y, img)


@pytest.mark.parametrize("op", ["swiglu", "geglu_erf"])
def test_emit_glu_bit_exact(op):
    wl = W.make(3, glu_op=op, small=True)
    print("emit_glu", op, flush=True)
    y, img = run_producer(wl)
    check_producer(wl, y, img)


@pytest.mark.parametrize("op", ["swiglu", "geglu_erf"])
def test_emit_glu_extreme_gates_bit_exact(op):
    # gates over the saturation paths of exp/erfc: far negative, large positive, zero, tiny
    K = 2048
    g = np.random.default_rng(11)
    gate = np.concatenate([np.linspace(-120, 120, K // 2), g.standard_normal(K // 2) * 30]).astype(np.float32)
    gate[:8] = [0.0, -0.0, 1e-30, -1e-30, 88.7, -88.7, 87.0, -87.0]
    gu = np.stack([np.concatenate([gate, g.standard_normal(K).astype(np.float32)]),
                   np.concatenate([-gate, np.ones(K, np.float32)])])
    wl = W.Workload(0, "extreme", 2, K, op, gu=gu)
    y, img = run_producer(wl)
    check_producer(wl, y, img)


@pytest.mark.parametrize("K", [32, 256, 2592, 14336, 32768])
def test_emit_rmsnorm_shapes(K):
    g = np.random.default_rng(K)
    x = (g.standard_normal((3, K)) * np.array([1.0, 1e3, 1e-3])[:, None]).astype(np.float32)
    wl = W.Workload(0, "K%d" % K, 3, K, "rmsnorm", x=x, gamma=g.normal(1, 0.1, K).astype(np.float32))
    y, img = run_producer(wl)
    check_producer(wl, y, img)


def test_emit_rmsnorm_without_gamma_and_zero_row():
    K = 2560
    x = np.random.default_rng(3).standard_normal((2, K)).astype(np.float32)
    x[1] = 0
    T = H.torch()
    y = H.sentinel_f32(2, K)
    img = H.sentinel_u8(qimg.image_bytes(2, K))
    qimg.emit_rmsnorm(H.dev(x), None, W.EPS, y, img)
    sync()
    y_o = O.rmsnorm(x, None, W.EPS)
    assert np.array_equal(H.host(y).view(np.uint32), y_o.view(np.uint32))
    assert np.array_equal(H.host(img), O.quantize(y_o))
    assert not H.host(img)[: 2 * qimg.row_blocks(K) * 36].reshape(-1)[qimg.row_blocks(K) * 32: 2 * qimg.row_blocks(K) * 32].any()


def test_fused_image_equals_separate_quantizer():
    # the emitted image must be the bytes of the original separate quantizer applied to the
    # stored f32 output (control arm == candidate arm)
    for config in (2, 3):
        wl = W.make(config, small=True)
        y, img = run_producer(wl)
        y_only, none = run_producer(wl, with_img=False)
        assert none is None and np.array_equal(y.view(np.uint32), y_only.view(np.uint32))
        img2 = H.sentinel_u8(qimg.image_bytes(wl.T, wl.K))
        qimg.quantize_q8_1(H.dev(y_only), img2)
        sync()
        assert np.array_equal(H.host(img2), img)


def test_quantizer_golden_and_special_blocks():
    K = 64
    y = np.zeros((3, K), np.float32)
    y[0, :6] = [127, 2.5, -2.5, 0.5, -0.5, 1.5]           # ties: half away from zero
    y[1, :32] = np.arange(-16, 16) / 8.0                   # exact multiples of d
    y[1, 0] = -127 / 8.0
    y[2, 32:] = 1e-38                                      # 1/d overflows: zero block
    img = H.sentinel_u8(qimg.image_bytes(3, K))
    qimg.quantize_q8_1(H.dev(y), img)
    sync()
    assert np.array_equal(H.host(img), O.quantize(y))


def fp16_double_rounding_blocks(y):
    """Blocks whose stored sum s16 = fp16(f32(sum * d)) differs from a single rounding of the
    exact product to fp16: the f32 product is an exact fp16 tie and the exact product is not.
    Found from the oracle's image (codes and d of each block)."""
    rows, K = y.shape
    img = O.quantize(y)
    codes, d16, s16 = O.image_planes(img, rows, K)
    Kb = K // 32
    blocks = y.reshape(rows, Kb, 32)
    d = (np.abs(blocks).max(-1) / np.float32(127.0)).astype(np.float32)
    csum = codes[:, :Kb].astype(np.int64).sum(-1)
    p32 = (csum.astype(np.float32) * d).astype(np.float32)
    bits = p32.view(np.uint32)
    tie = ((bits & 0x1FFF) == 0x1000) & (np.abs(p32) >= 2.0 ** -14) & (np.abs(p32) < 65504)
    inexact = csum.astype(np.float64) * d.astype(np.float64) != p32.astype(np.float64)
    return img, np.argwhere(tie & inexact)


def test_quantizer_sum_is_rounded_to_f32_then_fp16():
    # regression: fp16(a * b) must not become one mixed-precision multiply-add (a single rounding)
    g = np.random.default_rng(17)
    y = g.standard_normal((4096, 512)).astype(np.float32)
    img_o, ties = fp16_double_rounding_blocks(y)
    assert len(ties) >= 3, "the sample should hold a few fp16 double-rounding blocks"
    img = H.sentinel_u8(qimg.image_bytes(4096, 512))
    qimg.quantize_q8_1(H.dev(y), img)
    sync()
    assert np.array_equal(H.host(img), img_o)


# ---- block dots ----------------------------------------------------------------------------------
@pytest.mark.parametrize("K,T", [(32, 3), (2592, 13), (8192, 8), (14336, 5)])
def test_blockdots_bit_exact(K, T):
    # the per-block int32 dots of the reader kernel (matrix cores), bit for bit
    g = np.random.default_rng(K + T + 1)
    N = 37
    y = g.standard_normal((T, K)).astype(np.float32)
    img = O.quantize(y)
    w = W.q4_0_weights(g, (N,), K)
    wt = qimg.tile_q4_0(H.dev(w.qs), H.dev(w.d), K)
    ref = O.blockdots(w.qs, K, img, T, T)
    # repeated: a staged image read before its copies land differs only now and then
    for _ in range(4 if K <= 2592 else 1):
        sumi = H.torch().full((T, N, K // 32), -1, dtype=H.torch().int32, device="cuda")
        qimg.blockdots(wt, N, H.dev(img), T, K, sumi)
        sync()
        assert np.array_equal(H.host(sumi), ref)


@pytest.mark.parametrize("N,K,E", [(37, 2592, 1), (768, 2560, 3), (16, 32, 2)])
def test_tiled_weight_order(N, K, E):
    # reader tiles hold the same blocks as the standard order (layout check of the reorder)
    g = np.random.default_rng(N + K)
    w = W.q4_0_weights(g, (E, N), K)
    wt = H.host(qimg.tile_q4_0(H.dev(w.qs), H.dev(w.d), K))
    Kb, TL, KC = K // 32, (N + 15) // 16, (K // 32 + 3) // 4
    assert wt.size == E * TL * KC * 1152
    qs_t = wt[: E * TL * KC * 1024].reshape(E, TL, KC, 4, 16, 16)   # [e][tile][s][g][n][16 B]
    d_t = wt[E * TL * KC * 1024:].view(np.uint16).reshape(E, TL, KC, 4, 16)
    qpad = np.zeros((E, TL * 16, KC * 4, 16), np.uint8)
    qpad[:, :N, :Kb] = w.qs
    dpad = np.zeros((E, TL * 16, KC * 4), np.uint16)
    dpad[:, :N, :Kb] = w.d
    ref_q = qpad.reshape(E, TL, 16, KC, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    ref_d = dpad.reshape(E, TL, 16, KC, 4).transpose(0, 1, 3, 4, 2)
    assert np.array_equal(qs_t, ref_q) and np.array_equal(d_t, ref_d)


# ---- ordinary readers ----------------------------------------------------------------------------
def run_readers(wl, img_host, rows=None, live=None):
    T = wl.T if rows is None else rows
    torch = H.torch()
    img = H.dev(img_host)
    outs, specs = [], []
    for r in wl.readers:
        N = r.d.shape[-2]
        out = H.sentinel_f32(T, N)
        specs.append((qimg.tile_q4_0(H.dev(r.qs), H.dev(r.d), wl.K), N, out))
        outs.append(out)
    qimg.mmvq(specs, img, T, wl.K, H.live_tensor(live) if live is not None else None)
    sync()
    return [H.host(o) for o in outs]


def check_ordinary(wl, img_o, outs, live=None, nmse=True):
    live = wl.T if live is None else live
    for i, (r, out) in enumerate(zip(wl.readers, outs)):
        o64 = O.mmvq(r.qs, r.d, wl.K, img_o, wl.T, live)
        A = H.reader_abs_sum(r.qs, r.d, wl.K, img_o, wl.T, live)
        H.check_reader(out[:live], o64, A, wl.K, "reader %d" % i)
        assert (out[live:].view(np.uint8) == H.SENTINEL_BYTE).all(), "padding rows of out written"
        if nmse:
            ref = H.unquantized_ref(wl, r.qs, r.d, live)
            e = H.nmse(out[:live], ref)
            assert e <= 5e-4, "reader %d NMSE %.3g" % (i, e)


@pytest.mark.parametrize("config", [1, 2, 3])
def test_ordinary_small(config):
    wl = W.make(config, small=True)
    print("ordinary small config", config, flush=True)
    y, img = run_producer(wl)
    _, img_o = check_producer(wl, y, img)
    check_ordinary(wl, img_o, run_readers(wl, img))


@pytest.mark.parametrize("config", [1, 2])
def test_ordinary_full_size(config):
    wl = W.make(config)
    print("ordinary full config", config, flush=True)
    y, img = run_producer(wl)
    _, img_o = check_producer(wl, y, img)
    check_ordinary(wl, img_o, run_readers(wl, img))


@pytest.mark.parametrize("op", ["swiglu", "geglu_erf"])
def test_glu_workload_full_size_with_extra_f32_reader(op):
    # the GLU workload at full size: producer, the Q4_0 down reader (NMSE against the float64
    # activation included), then the kept f32 output is still the oracle's bit for bit and an
    # extra f32 reader of it (a dot with a seeded vector) matches the oracle's fixed-order sum
    # bit for bit and the float64 dot within its rounding bound
    torch = H.torch()
    wl = W.make(3, glu_op=op)
    print("GLU workload full size", op, flush=True)
    T, K = wl.T, wl.K
    gu = H.dev(wl.gu)
    y = H.sentinel_f32(T, K)
    img = H.sentinel_u8(qimg.image_bytes(T, K))
    qimg.emit_glu(op, gu[:, :K], gu[:, K:], y, img)
    outs, specs = [], []
    for r in wl.readers:
        N = r.d.shape[-2]
        out = H.sentinel_f32(T, N)
        specs.append((qimg.tile_q4_0(H.dev(r.qs), H.dev(r.d), K), N, out))
        outs.append(out)
    qimg.mmvq(specs, img, T, K)
    v = H.dev(wl.extra_v.reshape(1, K))
    fo = H.sentinel_f32(T, 1)
    qimg.f32_reader(y, v, fo)
    sync()
    y_h, img_h = H.host(y), H.host(img)
    _, img_o = check_producer(wl, y_h, img_h)   # y read after both readers ran
    check_ordinary(wl, img_o, [H.host(o) for o in outs])
    y_o = H.oracle_producer(wl)[0]
    f_o = O.moe_router(y_o, wl.extra_v.reshape(1, K), T)
    got = H.host(fo)
    assert np.array_equal(got.view(np.uint32), f_o.view(np.uint32)), "extra f32 reader differs"
    exact = y_o.astype(np.float64) @ wl.extra_v.astype(np.float64)
    J = -(-K // 256)
    n = 3 + int(np.ceil(np.log2(J))) + 7
    mag = np.abs(y_o.astype(np.float64)) @ np.abs(wl.extra_v.astype(np.float64))
    bound = n * H.U / (1 - n * H.U) * mag + 2.0 ** -50 * mag
    assert (np.abs(got[:, 0] - exact) <= bound).all()


@pytest.mark.parametrize("live", [None, 5])
def test_declined_emission_when_the_image_overlaps_the_inputs(live):
    # an image placed over the producer's own input is not emitted in the same pass: the call
    # runs the producer (y only) and then the separate quantizer, with the same bytes as an
    # emitting call; image rows past the live count keep the input bytes they overlap
    torch = H.torch()
    T, K = 8, 2592
    g = np.random.default_rng(2024)
    x = g.standard_normal((T, K)).astype(np.float32)
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    L = T if live is None else live
    lt = H.live_tensor(live) if live is not None else None
    nb = qimg.image_bytes(T, K)
    RB = qimg.row_blocks(K)
    # RMS: the image at the start of x's buffer
    buf = H.dev(x).view(torch.uint8).reshape(-1)
    before = H.host(buf).copy()
    y = H.sentinel_f32(T, K)
    qimg.emit_rmsnorm(buf.view(torch.float32).view(T, K), H.dev(gamma), W.EPS, y, buf[:nb], lt)
    sync()
    y_o = O.rmsnorm(x[:L], gamma, W.EPS)
    img_o = O.quantize(y_o, img_rows=T)
    img_h = H.host(buf)[:nb]
    assert np.array_equal(H.host(y)[:L].view(np.uint32), y_o.view(np.uint32))
    c, d = split_image(img_h, T, K)
    co, do = split_image(img_o, T, K)
    cb, db = split_image(before[:nb], T, K)
    assert np.array_equal(c[:L], co[:L]) and np.array_equal(d[:L], do[:L]), "declined RMS image differs"
    assert np.array_equal(c[L:], cb[L:]) and np.array_equal(d[L:], db[L:]), "padding image rows written"
    # GLU: the image over the packed gate|up rows
    gu = g.standard_normal((T, 2 * K)).astype(np.float32)
    gbuf = H.dev(gu)
    y2 = H.sentinel_f32(T, K)
    qimg.emit_glu("swiglu", gbuf[:, :K], gbuf[:, K:], y2, gbuf.view(torch.uint8).reshape(-1)[:nb], lt)
    sync()
    yg_o = O.glu_ex(gu[:L, :K], gu[:L, K:], "swiglu")
    assert np.array_equal(H.host(y2)[:L].view(np.uint32), yg_o.view(np.uint32))
    gi = H.host(gbuf.view(torch.uint8).reshape(-1))[:nb]
    c2, d2 = split_image(gi, T, K)
    co2, do2 = split_image(O.quantize(yg_o, img_rows=T), T, K)
    assert np.array_equal(c2[:L], co2[:L]) and np.array_equal(d2[:L], do2[:L]), "declined GLU image differs"
    # the same bytes as the emitting path on separate buffers
    y3 = H.sentinel_f32(T, K)
    img3 = H.sentinel_u8(nb)
    qimg.emit_rmsnorm(H.dev(x), H.dev(gamma), W.EPS, y3, img3, lt)
    sync()
    c3, d3 = split_image(H.host(img3), T, K)
    assert np.array_equal(c3[:L], c[:L]) and np.array_equal(d3[:L], d[:L])
    assert RB * 36 * T == nb


# the last two: more half tiles (8 weight rows) than workgroups, readers with an odd number of
# half tiles, so that workgroup runs start and end inside tiles and at reader boundaries
@pytest.mark.parametrize("K,T,Ns", [(32, 1, [5]), (2592, 13, [37, 64, 3]), (32768, 2, [9]), (2048, 8, [1, 300]),
                                    (2592, 8, [4100, 2056, 4100]), (4096, 3, [2049, 8, 2055])])
def test_ordinary_edge_shapes(K, T, Ns):
    g = np.random.default_rng(K * 7 + T)
    x = g.standard_normal((T, K)).astype(np.float32)
    wl = W.Workload(0, "edge", T, K, "rmsnorm", x=x, gamma=g.normal(1, 0.1, K).astype(np.float32),
                    readers=[W.q4_0_weights(g, (N,), K) for N in Ns])
    y, img = run_producer(wl)
    _, img_o = check_producer(wl, y, img)
    check_ordinary(wl, img_o, run_readers(wl, img), nmse=False)


def test_ordinary_live_rows_and_empty():
    wl = W.make(2, small=True)
    y, img = run_producer(wl)
    _, img_o = check_producer(wl, y, img)
    for live in (0, 3, 8):
        check_ordinary(wl, img_o, run_readers(wl, img, live=live), live=live, nmse=False)
    # zero rows is a no-op
    qimg.mmvq([(qimg.tile_q4_0(H.dev(r.qs), H.dev(r.d), wl.K), r.d.shape[0], H.sentinel_f32(1, r.d.shape[0]))
               for r in wl.readers], H.dev(img), 0, wl.K)
    qimg.emit_rmsnorm(H.dev(wl.x[:0]), H.dev(wl.gamma), W.EPS, H.sentinel_f32(0, wl.K), None)


def test_readers_deterministic():
    wl = W.make(2)
    y, img = run_producer(wl)
    a = run_readers(wl, img)
    for _ in range(2):
        b = run_readers(wl, img)
        for u, v in zip(a, b):
            assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


# ---- routed readers ------------------------------------------------------------------------------
def run_routed(wl, img_dev, ids_host, live=None, bucket=None):
    torch = H.torch()
    B = wl.T if bucket is None else bucket
    ws = torch.empty(qimg.workspace_bytes(B, wl.top_k, wl.E) // 4, dtype=torch.int32, device="cuda")
    ws.fill_(-7)
    outs, specs = [], []
    for r in wl.readers:
        N = r.d.shape[-2]
        out = H.sentinel_f32(B, wl.top_k, N)
        specs.append((r._dev_w, N, out))
        outs.append(out)
    qimg.mmvq_id(specs, wl.E, img_dev, H.dev(ids_host), H.live_tensor(live) if live is not None else None,
                 wl.K, ws)
    sync()
    return [H.host(o) for o in outs], H.host(ws)


def attach_dev_weights(wl):
    for r in wl.readers:
        if not hasattr(r, "_dev_w"):
            r._dev_w = qimg.tile_q4_0(H.dev(r.qs), H.dev(r.d), wl.K)


def check_plan(ws, ids, live, E, top_k):
    counts, offsets, members, bad = O.plan(ids, live, E)
    P = live * top_k
    assert ws[0] == 0 and ws[1] == P
    g_counts = ws[4: 4 + E]
    g_offsets = ws[4 + E: 4 + 2 * E + 1]
    g_members = ws[4 + 2 * E + 1: 4 + 2 * E + 1 + P]
    assert np.array_equal(g_counts, counts) and np.array_equal(g_offsets, offsets)
    assert np.array_equal(g_members, members)
    assert g_counts.sum() == P and (P == 0 or g_members.max() == P - 1)


def check_routed(wl, img_o, outs, live, ids=None, nmse=False):
    ids = wl.ids if ids is None else ids
    P = live * wl.top_k
    for i, (r, out) in enumerate(zip(wl.readers, outs)):
        o64 = O.mmvq_id(r.qs, r.d, wl.E, wl.K, img_o, wl.T, ids, live)   # [P][N]
        got = out.reshape(-1, out.shape[-1])
        A = H.routed_abs_sum(r.qs, r.d, wl.E, wl.K, img_o, wl.T, ids, live)
        H.check_reader(got[:P], o64, A, wl.K, "routed reader %d" % i)
        assert (got[P:].view(np.uint8) == H.SENTINEL_BYTE).all(), "padding pairs were written"
        if nmse and P:
            ref = H.unquantized_routed_ref(wl, r.qs, r.d, live, ids)
            e = H.nmse(got[:P], ref)
            assert e <= 5e-4, "routed reader %d NMSE %.3g" % (i, e)


def test_routed_config4_full():
    wl = W.make(4)
    attach_dev_weights(wl)
    y, img = run_producer(wl)
    _, img_o = check_producer(wl, y, img)
    outs, ws = run_routed(wl, H.dev(img), wl.ids)
    check_plan(ws, wl.ids, wl.T, wl.E, wl.top_k)
    check_routed(wl, img_o, outs, wl.T, nmse=True)


def test_routed_agrees_with_ordinary_reader_of_the_expert():
    # a pair's routed output is the ordinary reader of its expert on its image row (an oracle
    # identity); the two GPU paths sum in different orders, so they agree to the rounding bound
    wl = W.make(4, small=True)
    attach_dev_weights(wl)
    y, img = run_producer(wl)
    outs, _ = run_routed(wl, H.dev(img), wl.ids)
    _, img_o = H.oracle_producer(wl)
    for p in (0, 13, 63):
        t, e = p // wl.top_k, wl.ids.reshape(-1)[p]
        r = wl.readers[0]
        ow = W.Workload(0, "ord", wl.T, wl.K, "rmsnorm", readers=[W.Q4Weights(r.qs[e], r.d[e])])
        o = run_readers(ow, img)[0]
        o64 = O.mmvq(r.qs[e], r.d[e], wl.K, img_o, wl.T, wl.T)[t]
        scale = np.abs(o64).max()
        assert np.abs(o[t].astype(np.float64) - outs[0][t, p % wl.top_k]).max() <= 2e-5 * scale


def test_routed_bad_expert_ids_are_skipped_and_flagged():
    wl = W.make(4, small=True)
    attach_dev_weights(wl)
    y, img = run_producer(wl)
    ids = wl.ids.copy()
    ids[2, 3] = wl.E + 5
    ids[5, 0] = -1
    outs, ws = run_routed(wl, H.dev(img), ids)
    assert ws[0] & qimg.ERR_EXPERT_RANGE
    for out in outs:
        assert (out[2, 3].view(np.uint8) == H.SENTINEL_BYTE).all()
        assert (out[5, 0].view(np.uint8) == H.SENTINEL_BYTE).all()
    counts, offsets, members, bad = O.plan(ids, wl.T, wl.E)
    assert bad == 2 and ws[4 + 2 * wl.E] == offsets[wl.E]
    # live count above the bucket is clamped and flagged
    outs, ws = run_routed(wl, H.dev(img), wl.ids, live=wl.T + 3)
    assert ws[0] & qimg.ERR_LIVE_CLAMPED and ws[1] == wl.T * wl.top_k


@pytest.mark.parametrize("live", [128, 37])
def test_routed_crowded_experts_and_repeated_ids(live):
    # every live row routes to the same nine experts, so each of them has `live` pairs and needs
    # several column passes; one row names an expert twice (two pairs, both computed)
    print("crowded experts live", live, flush=True)
    wl = W.make(5, live=live, small=True)
    attach_dev_weights(wl)
    rng = np.random.default_rng([77, live])
    ids = np.empty_like(wl.ids)
    for t in range(wl.T):
        ids[t] = rng.permutation(wl.top_k) * 3
    ids[1, 4] = ids[1, 2]
    y, img = run_producer(wl, live=live)
    _, img_o = check_producer(wl, y, img, live=live)
    outs, ws = run_routed(wl, H.dev(img), ids, live=live)
    check_plan(ws, ids, live, wl.E, wl.top_k)
    check_routed(wl, img_o, outs, live, ids=ids)


def test_routed_single_expert_and_all_pairs_bad():
    wl = W.make(4, small=True)
    attach_dev_weights(wl)
    y, img = run_producer(wl)
    _, img_o = H.oracle_producer(wl)
    ids = np.full_like(wl.ids, wl.E - 1)  # every pair on the last expert
    outs, ws = run_routed(wl, H.dev(img), ids)
    check_plan(ws, ids, wl.T, wl.E, wl.top_k)
    check_routed(wl, img_o, outs, wl.T, ids=ids)
    bad = np.full_like(wl.ids, wl.E)  # no valid pair: nothing written, plan empty, flagged
    outs, ws = run_routed(wl, H.dev(img), bad)
    assert ws[0] == qimg.ERR_EXPERT_RANGE and ws[1] == wl.T * wl.top_k
    assert (ws[4:4 + 2 * wl.E + 1] == 0).all()
    for out in outs:
        assert (out.view(np.uint8) == H.SENTINEL_BYTE).all()


@pytest.mark.parametrize("live", [0, 1, 3])
def test_routed_register_plan_partial_bucket(live):
    # a bucket of 8 rows x top-8 (64 pairs: the launch keeps its plan in registers) with only
    # `live` rows live: padding rows' ids are never planned and their outputs stay unwritten
    wl = W.make(4, small=True)
    attach_dev_weights(wl)
    y, img = run_producer(wl, live=live)
    _, img_o = check_producer(wl, y, img, live=live)
    outs, ws = run_routed(wl, H.dev(img), wl.ids, live=live)
    check_plan(ws, wl.ids, live, wl.E, wl.top_k)
    if live:
        check_routed(wl, img_o, outs, live)
    for out in outs:
        assert (out[live:].view(np.uint8) == H.SENTINEL_BYTE).all()


@pytest.mark.parametrize("K", [128, 1024, 1536, 2560])
def test_routed_k_halves_and_one_row_runs(K):
    # K 128: units whole (one chunk); 1024, 1536, 2560: cut into two K halves (4 + 4, 6 + 6,
    # 10 + 10 chunks). Few tiles per expert and many workgroups, so a unit's halves often fall to
    # two waves (the first half's sums then go through a carry slot); every live row must still
    # equal its one-row run byte for byte
    print("routed K halves", K, flush=True)
    g = np.random.default_rng(K)
    B, E, k = 64, 12, 3
    x = g.standard_normal((B, K)).astype(np.float32)
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    ids, w = W.topk_ids(g, B, E, k)
    for live in (B, 3):
        wl = W.Workload(0, "parts", B, K, "rmsnorm", x=x, gamma=gamma,
                        readers=[W.q4_0_weights(g, (E, 40), K)], E=E, top_k=k, ids=ids, route_w=w, live=live)
        attach_dev_weights(wl)
        y, img = run_producer(wl, live=live)
        _, img_o = check_producer(wl, y, img, live=live)
        outs, ws = run_routed(wl, H.dev(img), ids, live=live)
        check_plan(ws, ids, live, E, k)
        check_routed(wl, img_o, outs, live)
        for t in sorted({0, live // 2, live - 1}):
            w1 = W.Workload(0, "one row", 1, K, "rmsnorm", x=x[t:t + 1].copy(), gamma=gamma,
                            readers=wl.readers, E=E, top_k=k, ids=ids[t:t + 1].copy())
            y1, img1 = run_producer(w1)
            o1, _ = run_routed(w1, H.dev(img1), w1.ids)
            assert np.array_equal(o1[0][0].view(np.uint32), outs[0][t].view(np.uint32)), "row %d" % t


# ---- padded bucket -------------------------------------------------------------------------------
@pytest.mark.parametrize("live", [1, 9, 113, 114, 128])
def test_padded_bucket(live):
    print("padded bucket live", live, flush=True)
    wl = W.make(5, live=live)
    attach_dev_weights(wl)
    y, img = run_producer(wl, live=live)
    _, img_o = check_producer(wl, y, img, live=live)
    img_d = H.dev(img)
    outs, ws = run_routed(wl, img_d, wl.ids, live=live)
    check_plan(ws, wl.ids, live, wl.E, wl.top_k)
    check_routed(wl, img_o, outs, live, nmse=True)
    # a different poison in the padding rows changes nothing
    x2 = wl.x.copy()
    W.poison_rows(x2, live, phase=1)
    y2, img2 = run_producer(wl, live=live, x=x2)
    assert np.array_equal(y2[:live].view(np.uint32), y[:live].view(np.uint32))
    assert np.array_equal(img2, img)
    # live rows equal one-row runs, byte for byte
    for t in sorted({0, live // 2, live - 1}):
        w1 = W.Workload(5, "one row", 1, wl.K, "rmsnorm", x=wl.x[t:t + 1].copy(), gamma=wl.gamma,
                        readers=wl.readers, E=wl.E, top_k=wl.top_k, ids=wl.ids[t:t + 1].copy())
        y1, img1 = run_producer(w1)
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32))
        o1, _ = run_routed(w1, H.dev(img1), w1.ids)
        for a, b in zip(o1, outs):
            assert np.array_equal(a[0].view(np.uint32), b[t].view(np.uint32))


def test_padded_bucket_graph_replay_at_changing_live_counts():
    torch = H.torch()
    wl = W.make(5, live=128)
    attach_dev_weights(wl)
    B, K, k = wl.T, wl.K, wl.top_k
    x_d = H.dev(wl.x)
    g_d = H.dev(wl.gamma)
    ids_d = H.dev(wl.ids)
    live_d = H.live_tensor(B)
    y_d = H.sentinel_f32(B, K)
    img_d = H.sentinel_u8(qimg.image_bytes(B, K))
    ws = torch.empty(qimg.workspace_bytes(B, k, wl.E) // 4, dtype=torch.int32, device="cuda")
    outs = [H.sentinel_f32(B, k, r.d.shape[-2]) for r in wl.readers]
    specs = [(r._dev_w, r.d.shape[-2], o) for r, o in zip(wl.readers, outs)]

    def step():
        qimg.emit_rmsnorm(x_d, g_d, W.EPS, y_d, img_d, live_d)
        qimg.mmvq_id(specs, wl.E, img_d, ids_d, live_d, K, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for phase, live in enumerate([1, 9, 113, 114, 128, 113, 9, 1]):
        x = wl.x.copy()
        W.poison_rows(x, live, phase)
        x_d.copy_(torch.from_numpy(x))
        live_d.fill_(live)
        y_d.view(torch.uint8).fill_(H.SENTINEL_BYTE)
        img_d.fill_(H.SENTINEL_BYTE)
        for o in outs:
            o.view(torch.uint8).fill_(H.SENTINEL_BYTE)
        sync()
        graph.replay()
        sync()
        w_live = W.Workload(5, "replay", B, K, "rmsnorm", x=x, gamma=wl.gamma, readers=wl.readers,
                            E=wl.E, top_k=k, ids=wl.ids, live=live)
        _, img_o = check_producer(w_live, H.host(y_d), H.host(img_d), live=live)
        check_plan(H.host(ws), wl.ids, live, wl.E, k)
        check_routed(w_live, img_o, [H.host(o) for o in outs], live)


def skewed_ids(g, pattern, B, E, k):
    """Routing ids concentrated on few experts (distinct within a row): every row on the same
    k experts, or one expert in every row's first slot with the other slots from top-k."""
    if pattern == "same_experts":
        base = (np.arange(k, dtype=np.int32) * 37 + 3) % E
        return np.stack([g.permutation(base) for _ in range(B)]).astype(np.int32)
    ids, _ = W.topk_ids(g, B, E, k)
    hot = 5
    for r in range(B):
        rest = [e for e in ids[r] if e != hot][: k - 1]
        ids[r] = [hot] + rest
    return ids.astype(np.int32)


@pytest.mark.parametrize("pattern,live", [("same_experts", 512), ("same_experts", 201),
                                          ("one_hot_expert", 512)])
def test_routed_plan_skewed(pattern, live):
    # skewed routing at the pair limit: up to 512 pairs of one expert, i.e. 64 segments of 8
    # columns whose members are exported by as many workgroups; the plan must still list each
    # expert's pairs in ascending order and every pair's outputs must match the oracle
    g = np.random.default_rng(3 + live)
    B, K, E, k = 512, 2048, 256, 8
    x = g.standard_normal((B, K)).astype(np.float32)
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    ids = skewed_ids(g, pattern, B, E, k)
    w = np.full((B, k), 1.0 / k, np.float32)
    wl = W.Workload(0, "skewed", B, K, "rmsnorm", x=x, gamma=gamma,
                    readers=[W.q4_0_weights(g, (E, 24), K)], E=E, top_k=k, ids=ids, route_w=w, live=live)
    attach_dev_weights(wl)
    y, img = run_producer(wl, live=live)
    _, img_o = check_producer(wl, y, img, live=live)
    outs, ws = run_routed(wl, H.dev(img), ids, live=live)
    check_plan(ws, ids, live, E, k)
    check_routed(wl, img_o, outs, live)


@pytest.mark.parametrize("live", [512, 455])
def test_routed_plan_at_the_pair_limit(live):
    # bucket 512 x top-8 = 4096 pairs (the largest plan one launch takes), far past the 1,024
    # pairs of a one-block plan; padding rows' stale ids are never planned
    g = np.random.default_rng(live)
    B, K, E, k = 512, 2048, 256, 8
    x = g.standard_normal((B, K)).astype(np.float32)
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    ids, w = W.topk_ids(g, B, E, k)
    wl = W.Workload(0, "pair limit", B, K, "rmsnorm", x=x, gamma=gamma,
                    readers=[W.q4_0_weights(g, (E, 24), K)], E=E, top_k=k, ids=ids, route_w=w, live=live)
    attach_dev_weights(wl)
    y, img = run_producer(wl, live=live)
    _, img_o = check_producer(wl, y, img, live=live)
    outs, ws = run_routed(wl, H.dev(img), ids, live=live)
    check_plan(ws, ids, live, E, k)
    check_routed(wl, img_o, outs, live)
