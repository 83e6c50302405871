"""Python view of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the benchmark's
CPU-baseline leg, never by the product package. It shares no code with the HIP library.

Each wrapper names the C function it calls; the definitions and the passages of the pages
they follow are at those functions in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c99"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (plain gcc; no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        sig = {
            "orc_f32_to_f16": (ctypes.c_uint16, [f32]),
            "orc_f32_to_f16_array": (None, [P, P, i64]),
            "orc_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_exp_q": (f32, [f32]),
            "orc_exp_q_array": (None, [P, P, i64]),
            "orc_erfc_q": (f32, [f32]),
            "orc_erfc_q_array": (None, [P, P, i64]),
            "orc_glu_act": (f32, [i32, f32]),
            "orc_glu_act_array": (None, [i32, P, P, i64]),
            "orc_glu_ex": (None, [i32, f32, f32, P, i64, P, i64, i32, i32, P, i64]),
            "orc_glu_pair_array": (None, [i32, f32, f32, P, f32, P, i64]),
            "orc_rmsnorm_ex": (None, [P, i64, P, P, f32, f32, i32, i32, P, i64]),
            "orc_rms_scale_array": (None, [P, P, i64]),
            "orc_mmvq_id_per_slot": (None, [P, P, i32, i32, i32, P, i32, P, i32, i32, P]),
            "orc_moe_combine": (None, [P, i64, P, P, i32, i32, i32, i32, P, i64]),
            "orc_moe_router": (None, [P, i64, P, i32, i32, i32, P, i64]),
            "orc_mmvq_fmt": (None, [i32, P, P, P, i32, i32, P, i32, i32, P]),
            "orc_moe_topk": (None, [P, i64, i32, i32, i32, P, P]),
            "orc_quant_recip_array": (None, [P, P, i64]),
            "orc_quant_scale_array": (None, [P, P, i64]),
            "orc_f32_to_f16_word_array": (None, [P, P, i64]),
            "orc_glu": (None, [i32, P, i64, P, i64, i32, i32, P, i64]),
            "orc_rms_sumsq": (f32, [P, i32]),
            "orc_rmsnorm": (None, [P, i64, P, f32, i32, i32, P, i64]),
            "orc_row_blocks": (i32, [i32]),
            "orc_quantize": (i32, [P, i64, i32, i32, P]),
            "orc_blockdots": (None, [P, i32, i32, P, i32, i32, P]),
            "orc_mmvq": (None, [P, P, i32, i32, P, i32, i32, P]),
            "orc_plan": (i32, [P, i32, i32, i32, P, P, P]),
            "orc_mmvq_id": (None, [P, P, i32, i32, i32, P, i32, P, i32, i32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def row_blocks(K: int) -> int:
    return int(lib().orc_row_blocks(K))


def image_bytes(rows: int, K: int) -> int:
    return rows * row_blocks(K) * 36


# ---- scalar / elementwise --------------------------------------------------------------------
def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def f16_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(int(h)))


def _out_like(x: np.ndarray, out: np.ndarray | None) -> np.ndarray:
    """A result array shaped like x: a new one, or the caller's (f32, C-contiguous, same size)."""
    if out is None:
        return np.empty_like(x)
    assert out.dtype == np.float32 and out.flags["C_CONTIGUOUS"] and out.size == x.size
    return out


def exp_q(x, out: np.ndarray | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = _out_like(x, out)
    lib().orc_exp_q_array(_p(x), _p(out), x.size)
    return out


def erfc_q(z, out: np.ndarray | None = None) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32)
    out = _out_like(z, out)
    lib().orc_erfc_q_array(_p(z), _p(out), z.size)
    return out


def glu_act(g, op: str, out: np.ndarray | None = None) -> np.ndarray:
    """orc_glu_act element-wise: the GLU activation alone (no up factor)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = _out_like(g, out)
    lib().orc_glu_act_array(GLU_OPS[op], _p(g), _p(out), g.size)
    return out


def rms_scale(v, out: np.ndarray | None = None) -> np.ndarray:
    """orc_rms_scale element-wise: 1 / sqrt(v)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = _out_like(v, out)
    lib().orc_rms_scale_array(_p(v), _p(out), v.size)
    return out


def quant_recip(amax, out: np.ndarray | None = None) -> np.ndarray:
    """1 / (amax / 127) element-wise: the quantizer's code multiplier."""
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = _out_like(amax, out)
    lib().orc_quant_recip_array(_p(amax), _p(out), amax.size)
    return out


def quant_scale(amax, out: np.ndarray | None = None) -> np.ndarray:
    """amax / 127 element-wise: the quantizer's block scale d."""
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = _out_like(amax, out)
    lib().orc_quant_scale_array(_p(amax), _p(out), amax.size)
    return out


def f32_to_f16_words(x, out: np.ndarray | None = None) -> np.ndarray:
    """f32 -> binary16 bits in the low half of a 32-bit word, returned as float32 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = _out_like(x, out)
    lib().orc_f32_to_f16_word_array(_p(x), _p(out), x.size)
    return out


# ---- producers -------------------------------------------------------------------------------
def rms_sumsq(x_row: np.ndarray) -> np.float32:
    x_row = np.ascontiguousarray(x_row, dtype=np.float32)
    return np.float32(lib().orc_rms_sumsq(_p(x_row), x_row.shape[0]))


def rmsnorm(x: np.ndarray, gamma: np.ndarray | None, eps: float, rows: int | None = None) -> np.ndarray:
    """orc_rmsnorm over the first `rows` rows of x [R][K]; returns y [rows][K] f32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    rows = R if rows is None else rows
    y = np.zeros((rows, K), dtype=np.float32)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    lib().orc_rmsnorm(_p(x), K, None if g is None else _p(g), ctypes.c_float(eps), rows, K, _p(y), K)
    return y


GLU_OPS = {"swiglu": 0, "geglu_erf": 1, "reglu": 2, "geglu": 3, "geglu_quick": 4, "swiglu_oai": 5,
           "swiglu_clamp": 6}
OAI_ALPHA, OAI_LIMIT = 1.702, 7.0  # the OpenAI-style SwiGLU defaults


def glu(gu: np.ndarray, op: str, rows: int | None = None) -> np.ndarray:
    """orc_glu over packed gate|up rows gu [R][2K] (gate half first); returns y [rows][K].
    Ops without parameters only (the clamped SwiGLU forms go through glu_ex)."""
    assert GLU_OPS[op] < 5, "use glu_ex for the ops with alpha/limit"
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    R, K2 = gu.shape
    K = K2 // 2
    rows = R if rows is None else rows
    y = np.zeros((rows, K), dtype=np.float32)
    base = gu.ctypes.data
    lib().orc_glu(GLU_OPS[op], ctypes.c_void_p(base), K2, ctypes.c_void_p(base + 4 * K), K2,
                  rows, K, _p(y), K)
    return y


def glu_pair(g, op: str, u: float, alpha: float = OAI_ALPHA, limit: float = OAI_LIMIT,
             out: np.ndarray | None = None) -> np.ndarray:
    """orc_glu_pair element-wise over gates g with one up value u."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = _out_like(g, out)
    lib().orc_glu_pair_array(GLU_OPS[op], ctypes.c_float(alpha), ctypes.c_float(limit), _p(g),
                             ctypes.c_float(u), _p(out), g.size)
    return out


def glu_ex(gate: np.ndarray, up: np.ndarray, op: str, alpha: float = OAI_ALPHA, limit: float = OAI_LIMIT,
           rows: int | None = None) -> np.ndarray:
    """orc_glu_ex over separate gate [R][K] and up [R][K] views (any row strides); y [rows][K]."""
    gate = np.asarray(gate, dtype=np.float32)
    up = np.asarray(up, dtype=np.float32)
    assert gate.strides[1] == 4 and up.strides[1] == 4 and gate.shape == up.shape
    R, K = gate.shape
    rows = R if rows is None else rows
    y = np.zeros((rows, K), dtype=np.float32)
    lib().orc_glu_ex(GLU_OPS[op], ctypes.c_float(alpha), ctypes.c_float(limit),
                     ctypes.c_void_p(gate.ctypes.data), gate.strides[0] // 4,
                     ctypes.c_void_p(up.ctypes.data), up.strides[0] // 4, rows, K, _p(y), K)
    return y


def rmsnorm_ex(x: np.ndarray, gamma, beta, scale: float, eps: float, rows: int | None = None) -> np.ndarray:
    """orc_rmsnorm_ex: RMS (x gamma) (+ beta) (x scale) over the first rows of x [R][K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    rows = R if rows is None else rows
    y = np.zeros((rows, K), dtype=np.float32)
    gm = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    bt = None if beta is None else np.ascontiguousarray(beta, dtype=np.float32)
    lib().orc_rmsnorm_ex(_p(x), K, None if gm is None else _p(gm), None if bt is None else _p(bt),
                         ctypes.c_float(scale), ctypes.c_float(eps), rows, K, _p(y), K)
    return y


# ---- quantizer -------------------------------------------------------------------------------
def quantize(y: np.ndarray, img_rows: int | None = None) -> np.ndarray:
    """orc_quantize: Q8_1 image bytes (uint8) of y [rows][K] laid out for img_rows rows.

    Rows of the image beyond y's rows are left zero here (the GPU leaves them unwritten)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    rows, K = y.shape
    img_rows = rows if img_rows is None else img_rows
    RB = row_blocks(K)
    full = np.zeros(img_rows * RB * 36, dtype=np.uint8)
    part = np.zeros(rows * RB * 36, dtype=np.uint8)
    bad = lib().orc_quantize(_p(y), K, rows, K, _p(part))
    if bad:
        raise ValueError("oracle quantizer met %d non-finite or out-of-range values" % bad)
    # place the `rows`-row planes into the img_rows-row layout
    full[: rows * RB * 32] = part[: rows * RB * 32]
    full[img_rows * RB * 32: img_rows * RB * 32 + rows * RB * 4] = part[rows * RB * 32:]
    return full


def image_planes(img: np.ndarray, img_rows: int, K: int):
    """Views (codes int8 [rows][RB][32], d16 uint16 [rows][RB], s16 uint16 [rows][RB])."""
    RB = row_blocks(K)
    img = np.asarray(img, dtype=np.uint8)
    codes = img[: img_rows * RB * 32].view(np.int8).reshape(img_rows, RB, 32)
    ds = img[img_rows * RB * 32: img_rows * RB * 36].view(np.uint32).reshape(img_rows, RB)
    return codes, (ds & 0xFFFF).astype(np.uint16), (ds >> 16).astype(np.uint16)


# ---- readers ---------------------------------------------------------------------------------
def blockdots(qs: np.ndarray, K: int, img: np.ndarray, img_rows: int, rows: int) -> np.ndarray:
    """orc_blockdots: sumi [rows][N][Kb] int32."""
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    Kb = K // 32
    N = qs.size // (Kb * 16)
    out = np.empty((rows, N, Kb), dtype=np.int32)
    img = np.ascontiguousarray(img, dtype=np.uint8)
    lib().orc_blockdots(_p(qs), N, K, _p(img), img_rows, rows, _p(out))
    return out


def mmvq(qs: np.ndarray, d16: np.ndarray, K: int, img: np.ndarray, img_rows: int, rows: int) -> np.ndarray:
    """orc_mmvq: float64 out [rows][N] of one ordinary Q4_0 reader."""
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    d16 = np.ascontiguousarray(d16, dtype=np.uint16)
    Kb = K // 32
    N = qs.size // (Kb * 16)
    out = np.empty((rows, N), dtype=np.float64)
    img = np.ascontiguousarray(img, dtype=np.uint8)
    lib().orc_mmvq(_p(qs), _p(d16), N, K, _p(img), img_rows, rows, _p(out))
    return out


WEIGHT_FMTS = {"q8_0": 1, "q4_1": 2}


def mmvq_fmt(fmt: str, qs: np.ndarray, d16: np.ndarray, m16, K: int, img: np.ndarray, img_rows: int,
             rows: int) -> np.ndarray:
    """orc_mmvq_fmt: float64 out [rows][N] of one ordinary Q8_0 or Q4_1 reader."""
    qs = np.ascontiguousarray(qs).view(np.uint8)
    d16 = np.ascontiguousarray(d16, dtype=np.uint16)
    m = None if m16 is None else np.ascontiguousarray(m16, dtype=np.uint16)
    Kb = K // 32
    N = d16.size // Kb
    out = np.empty((rows, N), dtype=np.float64)
    img = np.ascontiguousarray(img, dtype=np.uint8)
    lib().orc_mmvq_fmt(WEIGHT_FMTS[fmt], _p(qs), _p(d16), None if m is None else _p(m), N, K, _p(img),
                       img_rows, rows, _p(out))
    return out


def plan(ids: np.ndarray, live: int, E: int):
    """orc_plan: (counts[E], offsets[E+1], members[valid pairs], n_bad)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    top_k = ids.shape[1]
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    members = np.full(max(live * top_k, 1), -1, dtype=np.int32)
    bad = lib().orc_plan(_p(ids), live, top_k, E, _p(counts), _p(offsets), _p(members))
    return counts, offsets, members[: offsets[E]].copy(), int(bad)


def mmvq_id(qs: np.ndarray, d16: np.ndarray, E: int, K: int, img: np.ndarray, img_rows: int,
            ids: np.ndarray, live: int, per_slot: bool = False) -> np.ndarray:
    """orc_mmvq_id (image row = token) or orc_mmvq_id_per_slot (image row = pair):
    float64 out [live*top_k][N]; pairs with a bad expert stay NaN."""
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    d16 = np.ascontiguousarray(d16, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    top_k = ids.shape[1]
    Kb = K // 32
    N = qs.size // (E * Kb * 16)
    out = np.full((live * top_k, N), np.nan, dtype=np.float64)
    img = np.ascontiguousarray(img, dtype=np.uint8)
    fn = lib().orc_mmvq_id_per_slot if per_slot else lib().orc_mmvq_id
    fn(_p(qs), _p(d16), E, N, K, _p(img), img_rows, _p(ids), live, top_k, _p(out))
    return out


def moe_combine(x: np.ndarray, w: np.ndarray, ids: np.ndarray, E: int, live: int) -> np.ndarray:
    """orc_moe_combine over x [rows][top_k][N] f32: out [live][N] f32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rows, top_k, N = x.shape
    out = np.zeros((live, N), dtype=np.float32)
    lib().orc_moe_combine(_p(x), N, _p(w), _p(ids), E, live, top_k, N, _p(out), N)
    return out


def moe_router(x: np.ndarray, w: np.ndarray, live: int) -> np.ndarray:
    """orc_moe_router: logits [live][E] of x [R][K] against router weights w [E][K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    E, K = w.shape
    out = np.zeros((live, E), dtype=np.float32)
    lib().orc_moe_router(_p(x), x.shape[1], _p(w), E, live, K, _p(out), E)
    return out


def moe_topk(logits: np.ndarray, k: int, live: int | None = None):
    """orc_moe_topk: (ids [live][k] int32, weights [live][k] f32)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    R, E = logits.shape
    live = R if live is None else live
    ids = np.zeros((live, k), dtype=np.int32)
    w = np.zeros((live, k), dtype=np.float32)
    lib().orc_moe_topk(_p(logits), E, E, live, k, _p(ids), _p(w))
    return ids, w
