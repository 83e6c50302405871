"""GPU parity of the prefill (many-row) Q4_0 reader over the shared Q8_1 image, through the C
ABI, against the CPU oracle: outputs within normwise 1e-5 of the float64 oracle and the
per-element rounding bound, NMSE <= 5e-4 against the unquantized float64 activation, rows past
the live count untouched. At the full prompt size the oracle checks a seeded sample of rows.
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


def produce(x, gamma, live=None):
    T, K = x.shape
    y = H.sentinel_f32(T, K)
    img = H.sentinel_u8(qimg.image_bytes(T, K))
    qimg.emit_rmsnorm(H.dev(x), H.dev(gamma), W.EPS, y, img, H.live_tensor(live) if live is not None else None)
    return y, img


def read(readers, img, T, K, live=None, fmt="mmq"):
    outs, specs = [], []
    for r in readers:
        N = r.d.shape[-2]
        out = H.sentinel_f32(T, N)
        specs.append((qimg.tile_q4_0(H.dev(r.qs), H.dev(r.d), K), N, out))
        outs.append(out)
    qimg.mmvq(specs, img, T, K, H.live_tensor(live) if live is not None else None, fmt=fmt)
    sync()
    return [H.host(o) for o in outs]


def check(out, r, img_o, img_rows, rows, K, what):
    o64 = O.mmvq(r.qs, r.d, K, img_o, img_rows, rows)
    A = H.reader_abs_sum(r.qs, r.d, K, img_o, img_rows, rows)
    H.check_reader(out[:rows], o64, A, K, what)


@pytest.mark.parametrize("T,live,K,Ns", [(200, 187, 2592, (37, 64, 16)), (64, None, 32, (5,)),
                                         (130, 65, 8192, (48, 16)), (96, 1, 544, (24, 40)),
                                         (128, 0, 256, (16,))])
def test_prefill_reader_ragged(T, live, K, Ns):
    g = np.random.default_rng(T + K)
    x = g.standard_normal((T, K)).astype(np.float32)
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    readers = [W.q4_0_weights(g, (N,), K) for N in Ns]
    _, img = produce(x, gamma, live)
    outs = read(readers, img, T, K, live)
    L = T if live is None else live
    img_o = O.quantize(O.rmsnorm(x[:L], gamma, W.EPS), img_rows=T) if L else None
    for i, (r, out) in enumerate(zip(readers, outs)):
        if L:
            check(out, r, img_o, T, L, K, "prefill reader %d" % i)
        assert (out[L:].view(np.uint8) == H.SENTINEL_BYTE).all(), "rows past the live count written"


def test_prefill_reader_agrees_with_the_matvec_reader():
    # the same readers and image through both kernels: each within the rounding bound of the
    # oracle, so within twice that bound of each other
    wl = W.make(2, small=True)
    _, img = produce(wl.x, wl.gamma)
    a = read(wl.readers, img, wl.T, wl.K, fmt="mmq")
    b = read(wl.readers, img, wl.T, wl.K, fmt="q4_0")
    img_o = O.quantize(O.rmsnorm(wl.x, wl.gamma, W.EPS))
    for r, oa, ob in zip(wl.readers, a, b):
        check(oa, r, img_o, wl.T, wl.T, wl.K, "prefill")
        check(ob, r, img_o, wl.T, wl.T, wl.K, "mat-vec")


def test_prefill_full_size_sampled_rows():
    # the prompt workload (3325 tokens, K 3584, q/k/v readers 3584/512/512): the image is checked
    # bit for bit on every row, the outputs on a seeded sample of rows
    wl = W.make(6)
    T, K = wl.T, wl.K
    y, img = produce(wl.x, wl.gamma)
    outs = read(wl.readers, img, T, K, fmt="q4_0")  # rows >= 64: the prefill path
    img_h = H.host(img)
    y_o = O.rmsnorm(wl.x, wl.gamma, W.EPS)
    assert np.array_equal(H.host(y).view(np.uint32), y_o.view(np.uint32))
    img_o = O.quantize(y_o)
    assert np.array_equal(img_h, img_o), "prefill image differs"
    sample = np.sort(np.random.default_rng(66).choice(T, 24, replace=False))
    img_s = O.quantize(y_o[sample])
    x64 = wl.x[sample].astype(np.float64)
    y64 = x64 / np.sqrt(np.mean(x64 * x64, 1, keepdims=True) + W.EPS) * wl.gamma
    for i, (r, out) in enumerate(zip(wl.readers, outs)):
        check(out[sample], r, img_s, len(sample), len(sample), K, "prefill reader %d" % i)
        if i > 0:
            lo = (r.qs & 15).astype(np.float64)
            hi = (r.qs >> 4).astype(np.float64)
            wd = ((np.concatenate([lo, hi], -1) - 8.0) * H.f16(r.d)[..., None]).reshape(r.d.shape[0], -1)
            assert H.nmse(out[sample], y64 @ wd.T) <= 5e-4
