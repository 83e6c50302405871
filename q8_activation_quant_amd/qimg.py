"""Python binding of libqimg.so (the C ABI declared in include/qimg.h).

Argument marshalling only: tensors are passed as device pointers with their strides, and the
stream is torch's current HIP stream. Every step of the path runs in the library's kernels.
The library must be built (``python -m q8_activation_quant_amd.build`` or
``__graft_entry__.build()``); there is no fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqimg.so")

OK, EINVAL, EALIGN, EALIAS, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6
GLU_SWIGLU, GLU_GEGLU_ERF, GLU_REGLU, GLU_GEGLU, GLU_GEGLU_QUICK, GLU_SWIGLU_OAI, GLU_SWIGLU_CLAMP = range(7)
GLU_OPS = {"swiglu": GLU_SWIGLU, "geglu_erf": GLU_GEGLU_ERF, "reglu": GLU_REGLU, "geglu": GLU_GEGLU,
           "geglu_quick": GLU_GEGLU_QUICK, "swiglu_oai": GLU_SWIGLU_OAI, "swiglu_clamp": GLU_SWIGLU_CLAMP}
ERR_EXPERT_RANGE, ERR_LIVE_CLAMPED = 1, 2
MAX_READERS = 8
ABI_VERSION = 12

EXPORTS = (
    "qimg_strerror", "qimg_abi_version", "qimg_row_blocks", "qimg_image_bytes",
    "qimg_emit_rmsnorm", "qimg_emit_glu", "qimg_quantize_q8_1", "mmvq_q4_0_q8_1",
    "mmvq_id_workspace_bytes", "mmvq_id_q4_0_q8_1", "mmvq_q4_0_q8_1_blockdots",
    "qimg_q4_0_tiled_bytes", "qimg_q4_0_tile", "qimg_eval_math",
    "qimg_emit_glu_per_slot", "mmvq_id_q4_0_q8_1_per_slot", "qimg_moe_combine",
    "qimg_emit_rmsnorm_ex", "qimg_emit_glu_ex", "qimg_moe_router", "qimg_moe_topk",
    "qimg_q8_0_tiled_bytes", "qimg_q4_1_tiled_bytes", "qimg_q8_0_tile", "qimg_q4_1_tile",
    "mmvq_q8_0_q8_1", "mmvq_q4_1_q8_1", "mmq_q4_0_q8_1", "qimg_f32_reader", "mmvq_id_q4_0_q8_1_noalloc",
    "qimg_read_ceiling",
)
CEILING_SINK_WORDS = 2048
MATH_FNS = {"exp": 0, "erfc": 1, "swiglu": 2, "geglu_erf": 3, "rsqrt": 4, "qscale": 5, "qdiv": 6, "f2h": 7, "reglu": 8,
            "geglu": 9, "geglu_quick": 10, "swiglu_oai_gate": 11}


class QimgError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, strerror(status), status))


class Reader(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("N", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64)]


class ExpertReader(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("N", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("ld_pair", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqimg.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqimg.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "qimg_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "qimg_abi_version": (ctypes.c_int, []),
            "qimg_row_blocks": (i32, [i32]),
            "qimg_image_bytes": (i64, [i32, i32]),
            "qimg_emit_rmsnorm": (ctypes.c_int, [P, i64, P, f32, i32, P, i32, P, i64, P, P]),
            "qimg_emit_glu": (ctypes.c_int, [i32, P, i64, P, i64, i32, P, i32, P, i64, P, P]),
            "qimg_quantize_q8_1": (ctypes.c_int, [P, i64, i32, P, i32, P, P]),
            "mmvq_q4_0_q8_1": (ctypes.c_int, [ctypes.POINTER(Reader), i32, P, i32, P, i32, P]),
            "mmvq_id_workspace_bytes": (ctypes.c_size_t, [i32, i32, i32]),
            "mmvq_id_q4_0_q8_1": (ctypes.c_int, [ctypes.POINTER(ExpertReader), i32, i32, P, P, i32,
                                                 i32, P, i32, P, ctypes.c_size_t, P]),
            "mmvq_q4_0_q8_1_blockdots": (ctypes.c_int, [ctypes.POINTER(Reader), P, i32, i32, P, P]),
            "qimg_q4_0_tiled_bytes": (i64, [i32, i32, i32]),
            "qimg_q4_0_tile": (ctypes.c_int, [P, P, i32, i32, i32, P, P]),
            "qimg_eval_math": (ctypes.c_int, [i32, ctypes.c_uint32, i64, P, P]),
            "qimg_emit_glu_per_slot": (ctypes.c_int, [i32, P, i64, P, i64, i32, i32, P, i32, P, i64, P, P]),
            "mmvq_id_q4_0_q8_1_per_slot": (ctypes.c_int, [ctypes.POINTER(ExpertReader), i32, i32, P, P,
                                                          i32, i32, P, i32, P, ctypes.c_size_t, P]),
            "qimg_moe_combine": (ctypes.c_int, [P, i64, P, P, i32, i32, i32, P, i32, P, i64, P]),
            "qimg_emit_rmsnorm_ex": (ctypes.c_int, [P, i64, P, P, f32, f32, i32, P, i32, P, i64, P, P]),
            "qimg_emit_glu_ex": (ctypes.c_int, [i32, f32, f32, P, i64, P, i64, i32, P, i32, P, i64, P, P]),
            "qimg_moe_router": (ctypes.c_int, [P, i64, P, i32, i32, P, i32, P, i64, P]),
            "qimg_q8_0_tiled_bytes": (i64, [i32, i32, i32]),
            "qimg_q4_1_tiled_bytes": (i64, [i32, i32, i32]),
            "qimg_q8_0_tile": (ctypes.c_int, [P, P, i32, i32, i32, P, P]),
            "qimg_q4_1_tile": (ctypes.c_int, [P, P, P, i32, i32, i32, P, P]),
            "mmvq_q8_0_q8_1": (ctypes.c_int, [ctypes.POINTER(Reader), i32, P, i32, P, i32, P]),
            "mmvq_q4_1_q8_1": (ctypes.c_int, [ctypes.POINTER(Reader), i32, P, i32, P, i32, P]),
            "mmq_q4_0_q8_1": (ctypes.c_int, [ctypes.POINTER(Reader), i32, P, i32, P, i32, P]),
            "qimg_f32_reader": (ctypes.c_int, [P, i64, P, i32, i32, P, i32, P, i64, P]),
            "qimg_read_ceiling": (ctypes.c_int, [P, i64, P, P]),
            "mmvq_id_q4_0_q8_1_noalloc": (ctypes.c_int, [ctypes.POINTER(ExpertReader), i32, i32, P, P, i32, i32,
                                                         P, i32, P]),
            "qimg_moe_topk": (ctypes.c_int, [P, i64, i32, i32, P, i32, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.qimg_abi_version() != ABI_VERSION:
            raise RuntimeError("libqimg.so ABI %d, binding expects %d" % (L.qimg_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().qimg_strerror(status).decode()


def _check(status: int, fn: str) -> None:
    if status != OK:
        raise QimgError(status, fn)


def row_blocks(K: int) -> int:
    return int(lib().qimg_row_blocks(K))


def image_bytes(rows: int, K: int) -> int:
    return int(lib().qimg_image_bytes(rows, K))


def workspace_bytes(bucket: int, top_k: int, E: int) -> int:
    return int(lib().mmvq_id_workspace_bytes(bucket, top_k, E))


# ---- torch marshalling --------------------------------------------------------------------
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ld(t):
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


def emit_rmsnorm(x, gamma, eps, y, img=None, live_rows=None, stream=None):
    """y = rmsnorm(x) * gamma (gamma may be None); img (uint8) receives the Q8_1 image."""
    rows, K = x.shape
    _check(lib().qimg_emit_rmsnorm(_ptr(x), _ld(x), _ptr(gamma), ctypes.c_float(eps), rows,
                                   _ptr(live_rows), K, _ptr(y), _ld(y), _ptr(img), _stream(stream)),
           "qimg_emit_rmsnorm")


def emit_glu(op, gate, up, y, img=None, live_rows=None, stream=None):
    """y = act(gate) * up; gate/up may be the halves of one packed [rows, 2K] tensor."""
    op = GLU_OPS[op] if isinstance(op, str) else op
    rows, K = gate.shape
    _check(lib().qimg_emit_glu(op, _ptr(gate), _ld(gate), _ptr(up), _ld(up), rows, _ptr(live_rows),
                               K, _ptr(y), _ld(y), _ptr(img), _stream(stream)), "qimg_emit_glu")


def emit_rmsnorm_ex(x, gamma, beta, scale, eps, y, img=None, live_rows=None, stream=None):
    """y = ((rmsnorm(x) * gamma) + beta) * scale (gamma, beta may be None)."""
    rows, K = x.shape
    _check(lib().qimg_emit_rmsnorm_ex(_ptr(x), _ld(x), _ptr(gamma), _ptr(beta), ctypes.c_float(scale),
                                      ctypes.c_float(eps), rows, _ptr(live_rows), K, _ptr(y), _ld(y),
                                      _ptr(img), _stream(stream)), "qimg_emit_rmsnorm_ex")


def emit_glu_ex(op, gate, up, y, img=None, live_rows=None, alpha=1.702, limit=7.0, stream=None):
    """Any GLU variant; gate and up are [rows, K] views with their own row strides."""
    op = GLU_OPS[op] if isinstance(op, str) else op
    rows, K = gate.shape
    _check(lib().qimg_emit_glu_ex(op, ctypes.c_float(alpha), ctypes.c_float(limit), _ptr(gate), _ld(gate),
                                  _ptr(up), _ld(up), rows, _ptr(live_rows), K, _ptr(y), _ld(y), _ptr(img),
                                  _stream(stream)), "qimg_emit_glu_ex")


def quantize_q8_1(y, img, live_rows=None, stream=None):
    rows, K = y.shape
    _check(lib().qimg_quantize_q8_1(_ptr(y), _ld(y), rows, _ptr(live_rows), K, _ptr(img),
                                    _stream(stream)), "qimg_quantize_q8_1")


def tiled_bytes(N, K, E=1):
    return int(lib().qimg_q4_0_tiled_bytes(N, K, E))


def tile_q4_0(qs, d, K, stream=None):
    """Reorder standard Q4_0 planes (qs [.., N, K/32, 16] u8, d [.., N, K/32] fp16 bits) into
    the readers' tiled order; returns a new uint8 device tensor."""
    import torch
    N = qs.shape[-3]
    E = 1 if qs.dim() == 3 else qs.shape[0]
    out = torch.empty(tiled_bytes(N, K, E), dtype=torch.uint8, device=qs.device)
    _check(lib().qimg_q4_0_tile(_ptr(qs), _ptr(d), N, K, E, _ptr(out), _stream(stream)), "qimg_q4_0_tile")
    return out


def _readers(specs, cls):
    """specs: [(tiled weights tensor, N, out tensor)]."""
    arr = (cls * len(specs))()
    for i, (w, N, out) in enumerate(specs):
        arr[i] = cls(ctypes.c_void_p(w.data_ptr()), N, 0, ctypes.c_void_p(out.data_ptr()), out.stride(-2))
    return arr


def mmvq(readers, img, rows, K, live_rows=None, stream=None, fmt="q4_0"):
    """Ordinary readers: readers = [(tiled weights of format fmt, N, out [rows, N] f32)];
    fmt "mmq" forces the many-row (prefill) Q4_0 reader."""
    arr = _readers(readers, Reader)
    name = {"q4_0": "mmvq_q4_0_q8_1", "q8_0": "mmvq_q8_0_q8_1", "q4_1": "mmvq_q4_1_q8_1",
            "mmq": "mmq_q4_0_q8_1"}[fmt]
    _check(getattr(lib(), name)(arr, len(readers), _ptr(img), rows, _ptr(live_rows), K, _stream(stream)), name)


def tile_weights(w_qs, w_d, K, fmt="q4_0", w_m=None, stream=None):
    """Reorder standard planes of any reader format into its tiles (new uint8 device tensor)."""
    import torch
    if fmt == "q4_0":
        return tile_q4_0(w_qs, w_d, K, stream)
    N = w_d.shape[-2]
    E = 1 if w_d.dim() == 2 else w_d.shape[0]
    nbytes = int(getattr(lib(), "qimg_%s_tiled_bytes" % fmt)(N, K, E))
    out = torch.empty(nbytes, dtype=torch.uint8, device=w_qs.device)
    if fmt == "q8_0":
        _check(lib().qimg_q8_0_tile(_ptr(w_qs), _ptr(w_d), N, K, E, _ptr(out), _stream(stream)), "qimg_q8_0_tile")
    else:
        _check(lib().qimg_q4_1_tile(_ptr(w_qs), _ptr(w_d), _ptr(w_m), N, K, E, _ptr(out), _stream(stream)),
               "qimg_q4_1_tile")
    return out


def mmvq_id(readers, E, img, ids, live_rows, K, workspace, stream=None):
    """Routed readers: readers = [(tiled weights of E experts, N, out [bucket, top_k, N])];
    ids [bucket, top_k] int32; live_rows: int32 device tensor of one element, or None."""
    bucket, top_k = ids.shape
    arr = _readers(readers, ExpertReader)
    _check(lib().mmvq_id_q4_0_q8_1(arr, len(readers), E, _ptr(img), _ptr(ids), bucket, top_k,
                                   _ptr(live_rows), K, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "mmvq_id_q4_0_q8_1")


def _pair_ld(t):
    """Row stride of the (token, slot) pair rows of a [bucket, top_k, width] tensor."""
    assert t.dim() == 3 and t.stride(2) == 1 and t.stride(0) == t.shape[1] * t.stride(1), \
        "pair tensors are [bucket, top_k, width] with evenly spaced pair rows"
    return t.stride(1)


def mmvq_id_noalloc(readers, E, img, ids, live_rows, K, stream=None):
    """Routed readers without a workspace (the library's per-GPU plan array; nothing is
    allocated): as mmvq_id."""
    bucket, top_k = ids.shape
    arr = _readers(readers, ExpertReader)
    _check(lib().mmvq_id_q4_0_q8_1_noalloc(arr, len(readers), E, _ptr(img), _ptr(ids), bucket, top_k,
                                           _ptr(live_rows), K, _stream(stream)), "mmvq_id_q4_0_q8_1_noalloc")


def read_ceiling(buf, sink, stream=None):
    """Measurement aid: stream buf (a contiguous device tensor, bytes % 1024 == 0) once with the
    plain read kernel; sink: int32 device tensor of CEILING_SINK_WORDS words."""
    _check(lib().qimg_read_ceiling(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "qimg_read_ceiling")


def mmvq_id_per_slot(readers, E, img, ids, live_rows, K, workspace, stream=None):
    """Routed readers over a per-slot image (image row = pair): as mmvq_id, img has
    bucket*top_k rows."""
    bucket, top_k = ids.shape
    arr = _readers(readers, ExpertReader)
    _check(lib().mmvq_id_q4_0_q8_1_per_slot(arr, len(readers), E, _ptr(img), _ptr(ids), bucket, top_k,
                                            _ptr(live_rows), K, _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream)),
           "mmvq_id_q4_0_q8_1_per_slot")


def emit_glu_per_slot(op, gate, up, y, img=None, live_rows=None, stream=None):
    """y [bucket, top_k, K] = act(gate) * up over the pair rows of live tokens; gate and up are
    [bucket, top_k, K] views (e.g. the routed gate and up readers' outputs)."""
    op = GLU_OPS[op] if isinstance(op, str) else op
    bucket, top_k, K = gate.shape
    _check(lib().qimg_emit_glu_per_slot(op, _ptr(gate), _pair_ld(gate), _ptr(up), _pair_ld(up), bucket,
                                        top_k, _ptr(live_rows), K, _ptr(y), _pair_ld(y), _ptr(img),
                                        _stream(stream)), "qimg_emit_glu_per_slot")


def moe_combine(x, weights, ids, E, out, live_rows=None, stream=None):
    """out [bucket, N] = routing-weighted sum over the slots of x [bucket, top_k, N] (live rows)."""
    bucket, top_k, N = x.shape
    _check(lib().qimg_moe_combine(_ptr(x), _pair_ld(x), _ptr(weights), _ptr(ids), E, bucket, top_k,
                                  _ptr(live_rows), N, _ptr(out), _ld(out), _stream(stream)),
           "qimg_moe_combine")


def blockdots(w, N, img, rows, K, sumi, stream=None):
    """sumi [rows, N, K/32] int32: the block dots of one reader's tiled weights (debug export)."""
    r = Reader(ctypes.c_void_p(w.data_ptr()), N, 0, ctypes.c_void_p(sumi.data_ptr()), N)
    _check(lib().mmvq_q4_0_q8_1_blockdots(ctypes.byref(r), _ptr(img), rows, K, _ptr(sumi),
                                          _stream(stream)), "mmvq_q4_0_q8_1_blockdots")


def eval_math(fn, first_bits, out, stream=None):
    """out[i] = fn(x_i) with x_i the f32 of bit pattern first_bits + i (out: float32 device)."""
    fn = MATH_FNS[fn] if isinstance(fn, str) else fn
    _check(lib().qimg_eval_math(fn, ctypes.c_uint32(first_bits & 0xFFFFFFFF), out.numel(), _ptr(out),
                                _stream(stream)), "qimg_eval_math")


def moe_router(x, w, logits, live_rows=None, stream=None):
    """logits [bucket, E] = x [bucket, K] . w [E, K]^T for live rows (fixed summation order)."""
    bucket, K = x.shape
    E = w.shape[0]
    _check(lib().qimg_moe_router(_ptr(x), _ld(x), _ptr(w), E, bucket, _ptr(live_rows), K, _ptr(logits),
                                 _ld(logits), _stream(stream)), "qimg_moe_router")


def f32_reader(y, v, out, live_rows=None, stream=None):
    """out [rows, N] = y [rows, K] . v [N, K]^T for live rows: an extra f32 reader of a
    producer's kept output (the router's fixed summation order)."""
    rows, K = y.shape
    N = v.shape[0]
    _check(lib().qimg_f32_reader(_ptr(y), _ld(y), _ptr(v), N, rows, _ptr(live_rows), K, _ptr(out), _ld(out),
                                 _stream(stream)), "qimg_f32_reader")


def moe_topk(logits, ids, weights=None, live_rows=None, stream=None):
    """ids [bucket, k] (and softmax weights [bucket, k]) of the k largest logits per live row."""
    bucket, E = logits.shape
    k = ids.shape[1]
    _check(lib().qimg_moe_topk(_ptr(logits), _ld(logits), E, bucket, _ptr(live_rows), k, _ptr(ids),
                               _ptr(weights), _stream(stream)), "qimg_moe_topk")
