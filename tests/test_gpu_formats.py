"""GPU parity of the Q8_0 and Q4_1 ordinary readers over the shared Q8_1 image, through the C
ABI, against the CPU oracle: the image is the fused producer's (bit-exact), the tiles hold the
standard planes' blocks, and the reader outputs are within normwise 1e-5 of the float64 oracle
and the per-element rounding bound, with NMSE <= 5e-4 against the unquantized float64
activation.
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
    qimg.lib()
    yield
    torch.cuda.synchronize()


def sync():
    H.torch().cuda.synchronize()


def tile(w, K):
    m = None if w.m is None else H.dev(w.m)
    return qimg.tile_weights(H.dev(w.qs.view(np.uint8)), H.dev(w.d), K, fmt=w.fmt, w_m=m)


def abs_bound(w, img, img_rows, rows, K):
    """A[t][n] = sum_b |d_w| |d_a| qmax sum|c| (+ |m_w| |s_a| for Q4_1): the scale of the reader's
    rounding error (qmax = 127 for Q8_0, 15 for Q4_1)."""
    codes, da, sa = O.image_planes(img, img_rows, K)
    Kb = K // 32
    qmax = 127.0 if w.fmt == "q8_0" else 15.0
    ta = np.abs(H.f16(da[:rows, :Kb])) * qmax * np.abs(codes[:rows, :Kb].astype(np.float64)).sum(-1)
    A = ta @ np.abs(H.f16(w.d)).T
    if w.m is not None:
        A += np.abs(H.f16(sa[:rows, :Kb])) @ np.abs(H.f16(w.m)).T
    return A


def dequantized(w):
    if w.fmt == "q8_0":
        return w.qs.astype(np.float64) * H.f16(w.d)[..., None]
    lo = (w.qs & 15).astype(np.float64)
    hi = (w.qs >> 4).astype(np.float64)
    return np.concatenate([lo, hi], axis=-1) * H.f16(w.d)[..., None] + H.f16(w.m)[..., None]


def run(wl, fmt, live=None):
    from test_gpu_parity import run_producer, check_producer
    y, img = run_producer(wl, live=live)
    _, img_o = check_producer(wl, y, img, live=live)
    L = wl.T if live is None else live
    outs, specs = [], []
    for r in wl.readers:
        N = r.d.shape[-2]
        out = H.sentinel_f32(wl.T, N)
        specs.append((tile(r, wl.K), N, out))
        outs.append(out)
    qimg.mmvq(specs, H.dev(img), wl.T, wl.K, H.live_tensor(live) if live is not None else None, fmt=fmt)
    sync()
    return [H.host(o) for o in outs], img_o, L


@pytest.mark.parametrize("fmt", ["q8_0", "q4_1"])
def test_format_reader_full_size(fmt):
    # the K8192/T8 workload's three readers (N 8192, 1024, 1024) in the other format
    wl = W.make(2, wfmt=fmt)
    outs, img_o, L = run(wl, fmt)
    y64 = None
    for i, (r, out) in enumerate(zip(wl.readers, outs)):
        o64 = O.mmvq_fmt(fmt, r.qs, r.d, r.m, wl.K, img_o, wl.T, L)
        H.check_reader(out[:L], o64, abs_bound(r, img_o, wl.T, L, wl.K), wl.K, "%s reader %d" % (fmt, i))
        if i > 0:  # the N=1024 readers: against the unquantized float64 activation
            if y64 is None:
                x = wl.x.astype(np.float64)
                y64 = x / np.sqrt(np.mean(x * x, 1, keepdims=True) + W.EPS) * wl.gamma
            ref = y64 @ dequantized(r).reshape(r.d.shape[0], -1).T
            assert H.nmse(out[:L], ref) <= 5e-4


@pytest.mark.parametrize("fmt", ["q8_0", "q4_1"])
# the last: more half tiles (8 weight rows) than workgroups and readers with an odd number of
# them, so that workgroup runs start and end inside tiles and at reader boundaries
@pytest.mark.parametrize("K,T,live,Ns", [(2592, 13, 11, (37, 16)), (32, 2, None, (5,)), (8192, 8, 3, (64, 24)),
                                         (2592, 8, None, (4100, 2056, 1032))])
def test_format_reader_edge_shapes(fmt, K, T, live, Ns):
    g = np.random.default_rng(K + T + len(Ns))
    x = g.standard_normal((T, K)).astype(np.float32)
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    readers = [W.WEIGHT_MAKERS[fmt](g, (N,), K) for N in Ns]
    wl = W.Workload(2, "edge", T, K, "rmsnorm", x=x, gamma=gamma, readers=readers)
    outs, img_o, L = run(wl, fmt, live=live)
    for i, (r, out) in enumerate(zip(readers, outs)):
        o64 = O.mmvq_fmt(fmt, r.qs, r.d, r.m, K, img_o, T, L)
        H.check_reader(out[:L], o64, abs_bound(r, img_o, T, L, K), K, "%s reader %d" % (fmt, i))
        assert (out[L:].view(np.uint8) == H.SENTINEL_BYTE).all(), "rows past the live count written"


@pytest.mark.parametrize("fmt", ["q8_0", "q4_1"])
def test_format_tiles_hold_the_standard_blocks(fmt):
    g = np.random.default_rng(61)
    N, K = 37, 2592
    w = W.WEIGHT_MAKERS[fmt](g, (N,), K)
    t = H.host(tile(w, K))
    Kb, TL, KC = K // 32, (N + 15) // 16, (K // 32 + 3) // 4
    cb = 2048 if fmt == "q8_0" else 1024
    assert t.size == TL * KC * (cb + (128 if fmt == "q8_0" else 256))
    codes = t[: TL * KC * cb]
    scales = t[TL * KC * cb:]
    for tile_i in range(TL):
        for s in range(KC):
            c = tile_i * KC + s
            for lane in (0, 17, 35, 63):
                row, blk = tile_i * 16 + (lane & 15), 4 * s + (lane >> 4)
                ok = row < N and blk < Kb
                if fmt == "q8_0":
                    got = np.concatenate([codes[(2 * c) * 1024 + 16 * lane:][:16], codes[(2 * c + 1) * 1024 + 16 * lane:][:16]])
                    want = w.qs[row, blk].view(np.uint8) if ok else np.zeros(32, np.uint8)
                    sc = scales.view(np.uint16)[c * 64 + lane]
                    assert sc == (w.d[row, blk] if ok else 0)
                else:
                    got = codes[c * 1024 + 16 * lane:][:16]
                    want = w.qs[row, blk] if ok else np.zeros(16, np.uint8)
                    word = scales.view(np.uint32)[c * 64 + lane]
                    assert word == ((int(w.d[row, blk]) | (int(w.m[row, blk]) << 16)) if ok else 0)
                assert np.array_equal(got, want)
