"""GPU parity of the remaining producer variants, through the C ABI, against the CPU oracle:
ReGLU, GeGLU (tanh form), GeGLU-quick, SwiGLU-OAI and SwiGLU-clamp (with alpha/limit), the two
original GLU ops through the general entry, separate / packed / packed-swapped inputs with
independent row strides, and the RMS+MUL+ADD and RMS+SCALE producers. Bars: f32 output and Q8_1
image bytes bit-exact; rows past the live count untouched.
"""
import numpy as np
import pytest

import helpers as H
from oracle import oracle as O
from q8_activation_quant_amd import qimg
from q8_activation_quant_amd import workloads as W

pytestmark = pytest.mark.gpu

ALL_GLU = ["swiglu", "geglu_erf", "reglu", "geglu", "geglu_quick", "swiglu_oai", "swiglu_clamp"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = H.torch()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qimg.lib()
    yield
    torch.cuda.synchronize()


def sync():
    H.torch().cuda.synchronize()


def check(y, img, y_o, rows, K, live, what):
    img_o = O.quantize(y_o, img_rows=rows)
    assert np.array_equal(y[:live].view(np.uint32), y_o.view(np.uint32)), what + ": f32 output differs"
    assert (y[live:].view(np.uint8) == H.SENTINEL_BYTE).all(), what + ": padding rows of y written"
    RB = qimg.row_blocks(K)
    c, d = img[: rows * RB * 32].reshape(rows, -1), img[rows * RB * 32:].reshape(rows, -1)
    co, do = img_o[: rows * RB * 32].reshape(rows, -1), img_o[rows * RB * 32:].reshape(rows, -1)
    assert np.array_equal(c[:live], co[:live]) and np.array_equal(d[:live], do[:live]), what + ": image differs"
    assert (c[live:] == H.SENTINEL_BYTE).all() and (d[live:] == H.SENTINEL_BYTE).all(), what + ": padding image rows"


def run_glu(op, gate_dev, up_dev, rows, K, live=None, alpha=O.OAI_ALPHA, limit=O.OAI_LIMIT):
    y = H.sentinel_f32(rows, K)
    img = H.sentinel_u8(qimg.image_bytes(rows, K))
    qimg.emit_glu_ex(op, gate_dev, up_dev, y, img, H.live_tensor(live) if live is not None else None,
                     alpha=alpha, limit=limit)
    sync()
    return H.host(y), H.host(img)


@pytest.mark.parametrize("op", ALL_GLU)
def test_glu_variant_full_size_packed(op):
    # the GLU workload's shape: packed gate|up [8, 2 x 14336], gate half first
    wl = W.make(3)
    K = wl.K
    gu = H.dev(wl.gu)
    y, img = run_glu(op, gu[:, :K], gu[:, K:], wl.T, K)
    check(y, img, O.glu_ex(wl.gu[:, :K], wl.gu[:, K:], op), wl.T, K, wl.T, op)


@pytest.mark.parametrize("op", ALL_GLU)
def test_glu_variant_swapped_and_strided(op):
    # packed-swapped rows (up half first) and separate buffers with their own row strides, a
    # ragged K (81 blocks: a partial slice and padding blocks) and a live count
    g = np.random.default_rng(31)
    T, K, live = 13, 2592, 11
    ug = (g.standard_normal((T, 2 * K)) * 4).astype(np.float32)
    ugd = H.dev(ug)
    y, img = run_glu(op, ugd[:, K:], ugd[:, :K], T, K, live=live)
    check(y, img, O.glu_ex(ug[:, K:], ug[:, :K], op, rows=live), T, K, live, op + " swapped")
    gate = np.zeros((T, K + 64), np.float32)
    up = np.zeros((T, K + 128), np.float32)
    gate[:, :K] = (g.standard_normal((T, K)) * 6).astype(np.float32)
    up[:, :K] = (g.standard_normal((T, K)) * 6).astype(np.float32)
    gd, udv = H.dev(gate), H.dev(up)
    y, img = run_glu(op, gd[:, :K], udv[:, :K], T, K)
    check(y, img, O.glu_ex(gate[:, :K], up[:, :K], op), T, K, T, op + " strided")


@pytest.mark.parametrize("op,alpha,limit", [("swiglu_oai", 1.0, 3.5), ("swiglu_oai", 2.5, 0.0),
                                            ("swiglu_clamp", 1.702, 1.25)])
def test_glu_clamped_parameters(op, alpha, limit):
    g = np.random.default_rng(32)
    T, K = 4, 4096
    gu = (g.standard_normal((T, 2 * K)) * 5).astype(np.float32)
    gd = H.dev(gu)
    y, img = run_glu(op, gd[:, :K], gd[:, K:], T, K, alpha=alpha, limit=limit)
    check(y, img, O.glu_ex(gu[:, :K], gu[:, K:], op, alpha=alpha, limit=limit), T, K, T, op)


@pytest.mark.parametrize("K,beta,scale", [(8192, True, 1.0), (8192, False, 0.5), (2560, True, 3.0),
                                          (2592, True, 0.7)])
def test_rmsnorm_add_and_scale(K, beta, scale):
    g = np.random.default_rng(K + int(10 * scale))
    T, live = 8, 6
    x = g.standard_normal((T, K)).astype(np.float32)
    x[0, g.choice(K, K // 100, replace=False)] *= 20
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    b = g.normal(0.0, 0.5, K).astype(np.float32) if beta else None
    y = H.sentinel_f32(T, K)
    img = H.sentinel_u8(qimg.image_bytes(T, K))
    qimg.emit_rmsnorm_ex(H.dev(x), H.dev(gamma), None if b is None else H.dev(b), scale, W.EPS, y, img,
                         H.live_tensor(live))
    sync()
    y_o = O.rmsnorm_ex(x, gamma, b, scale, W.EPS, rows=live)
    check(H.host(y), H.host(img), y_o, T, K, live, "rms add/scale")
