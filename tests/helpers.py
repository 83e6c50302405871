"""Shared helpers of the GPU parity tests: device copies, the oracle side of a workload, and
the tolerance checks (bit-exact bytes; float outputs within the stated bounds)."""
from __future__ import annotations

import math

import numpy as np

from oracle import oracle as O
from q8_activation_quant_amd import workloads as W

U = 2.0 ** -24
SENTINEL_BYTE = 0xA5
SENTINEL_F32 = np.frombuffer(bytes([SENTINEL_BYTE] * 4), np.float32)[0]


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return t.from_numpy(a).to("cuda")


def host(x) -> np.ndarray:
    return x.detach().cpu().numpy()


def sentinel_u8(nbytes):
    return torch().full((nbytes,), SENTINEL_BYTE, dtype=torch().uint8, device="cuda")


def sentinel_f32(*shape):
    t = torch().empty(*shape, dtype=torch().float32, device="cuda")
    t.view(torch().uint8).fill_(SENTINEL_BYTE)
    return t


def live_tensor(n):
    return torch().tensor([n], dtype=torch().int32, device="cuda")


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# ---- oracle side ------------------------------------------------------------------------------
def oracle_producer(wl: W.Workload, live=None):
    live = wl.T if live is None else live
    if wl.producer == "rmsnorm":
        y = O.rmsnorm(wl.x[:live], wl.gamma, W.EPS)
    else:
        y = O.glu_ex(wl.gu[:live, :wl.K], wl.gu[:live, wl.K:], wl.producer)
    img = O.quantize(y, img_rows=wl.T)
    return y, img


def reader_abs_sum(qs, d16, K, img, img_rows, rows):
    """A[t][n] = sum_b |d_w| (|d16 sumi| + 8 |s16|): the scale of the reader's rounding error."""
    sumi = O.blockdots(qs, K, img, img_rows, rows).astype(np.float64)  # [rows][N][Kb]
    codes, da, sa = O.image_planes(img, img_rows, K)
    Kb = K // 32
    dw = np.abs(f16(d16.reshape(-1, Kb)))                                # [N][Kb]
    term = np.abs(f16(da[:rows, :Kb]))[:, None, :] * np.abs(sumi) + 8 * np.abs(f16(sa[:rows, :Kb]))[:, None, :]
    return np.einsum("nb,tnb->tn", dw, term)


def _sub_image(img, img_rows, K, rows):
    """The image rows `rows` (in that order) as an image of their own."""
    RB = O.row_blocks(K)
    img = np.asarray(img, dtype=np.uint8)
    codes = img[: img_rows * RB * 32].reshape(img_rows, RB * 32)[rows]
    ds = img[img_rows * RB * 32: img_rows * RB * 36].reshape(img_rows, RB * 4)[rows]
    return np.concatenate([codes.reshape(-1), ds.reshape(-1)])


def routed_abs_sum(qs, d16, E, K, img, img_rows, ids, live, per_slot=False):
    """A[p][n] = sum_b |d_w| (|d16 sumi| + 8 |s16|) of every live pair p with an in-range
    expert (the pair's expert weights and image row: its token's row, or row p per slot);
    0 for the other pairs."""
    top_k = ids.shape[1]
    P = live * top_k
    flat = np.asarray(ids).reshape(-1)[:P]
    Kb = K // 32
    N = qs.shape[-3]
    A = np.zeros((P, N), np.float64)
    _, da, sa = O.image_planes(img, img_rows, K)
    for e in np.unique(flat):
        if e < 0 or e >= E:
            continue
        pairs = np.flatnonzero(flat == e)
        rows = pairs if per_slot else pairs // top_k
        sub = _sub_image(img, img_rows, K, rows)
        sumi = O.blockdots(qs[e], K, sub, len(rows), len(rows)).astype(np.float64)  # [c][N][Kb]
        dw = np.abs(f16(d16[e].reshape(-1, Kb)))
        term = np.abs(f16(da[rows, :Kb]))[:, None, :] * np.abs(sumi) + 8 * np.abs(f16(sa[rows, :Kb]))[:, None, :]
        A[pairs] = np.einsum("nb,pnb->pn", dw, term)
    return A


def check_reader(out, o64, A, K, what=""):
    """Normwise relative error <= 1e-5 and the per-element bound gamma_{Kb+3} A + 2^-50 A."""
    out = out.astype(np.float64)
    if out.size == 0:
        return 0.0
    assert np.isfinite(out).all(), what + ": non-finite output"
    err = np.abs(out - o64)
    n = K // 32 + 3
    gam = n * U / (1 - n * U)
    bad = err > gam * A + 2.0 ** -50 * A
    assert not bad.any(), "%s: %d elements beyond the rounding bound (max err %.3g)" % (what, bad.sum(), err.max())
    nw = err.max() / max(np.abs(o64).max(), 1e-300)
    assert nw <= 1e-5, "%s: normwise relative error %.3g" % (what, nw)
    return nw


def nmse(out, ref):
    return float(np.sum((out.astype(np.float64) - ref) ** 2) / np.sum(ref ** 2))


def producer_f64(wl: W.Workload, rows):
    """The producer output in float64 (textbook formulas, libm f64 exp/erf)."""
    import scipy.special
    K = wl.K
    if wl.producer == "rmsnorm":
        x = wl.x[:rows].astype(np.float64)
        y64 = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + W.EPS) * wl.gamma.astype(np.float64)
    else:
        g = wl.gu[:rows, :K].astype(np.float64)
        u = wl.gu[:rows, K:].astype(np.float64)
        if wl.producer == "swiglu":
            y64 = g / (1 + np.exp(-g)) * u
        else:
            y64 = 0.5 * g * scipy.special.erfc(-g / math.sqrt(2)) * u
    return y64


def dequant_q4_0(qs, d16, K):
    """float64 weights [N][K] of standard Q4_0 planes of one reader or expert."""
    Kb = K // 32
    lo = (qs & 15).astype(np.float64)
    hi = (qs >> 4).astype(np.float64)
    wq = (np.concatenate([lo, hi], axis=-1) - 8.0) * f16(d16)[..., None]
    return wq.reshape(wq.shape[0], Kb * 32)


def unquantized_ref(wl: W.Workload, qs, d16, rows):
    """float64 producer output (libm f64 exp/erf) dotted with the dequantized Q4_0 weights."""
    return producer_f64(wl, rows) @ dequant_q4_0(qs, d16, wl.K).T


def unquantized_routed_ref(wl: W.Workload, qs, d16, live, ids=None):
    """Routed: pair p's output from its token's float64 producer row and its expert's
    dequantized weights; NaN for pairs with an out-of-range expert. [live*top_k][N]."""
    ids = wl.ids if ids is None else ids
    k = ids.shape[1]
    flat = np.asarray(ids).reshape(-1)[: live * k]
    y64 = producer_f64(wl, live)
    out = np.full((live * k, qs.shape[-3]), np.nan)
    for e in np.unique(flat):
        if 0 <= e < wl.E:
            pairs = np.flatnonzero(flat == e)
            out[pairs] = y64[pairs // k] @ dequant_q4_0(qs[e], d16[e], wl.K).T
    return out
