"""Host-side checks of the C ABI (no GPU needed).

The library is loaded with ctypes; every function that include/qimg.h declares must be exported,
the size helpers must follow the documented layouts, and every argument error must be reported
by the host validation before anything is enqueued. Only invalid calls are made here (and
calls with nothing to do), so no kernel is ever launched: the pointers below are plain integers
that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from q8_activation_quant_amd import qimg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qimg.h")

A = 1 << 20  # 16-byte aligned stand-in addresses, far apart
B = 1 << 28
C = 1 << 32
D = 1 << 36
S = None  # default stream handle


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return", "sizeof")))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qimg.LIB_PATH):
        pytest.skip("libqimg.so not built")
    return qimg.lib()


def test_header_declares_the_documented_entry_points():
    names = header_functions()
    for must in ("qimg_emit_rmsnorm", "qimg_emit_glu", "mmvq_q4_0_q8_1", "mmvq_id_q4_0_q8_1"):
        assert must in names
    assert set(names) == set(qimg.EXPORTS), "binding and header disagree"


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name
    assert L.qimg_abi_version() == qimg.ABI_VERSION


def test_strerror_names_every_status(L):
    seen = set()
    for st in (qimg.OK, qimg.EINVAL, qimg.EALIGN, qimg.EALIAS, qimg.EUNSUPPORTED,
               qimg.EWORKSPACE, qimg.EHIP):
        s = qimg.strerror(st)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert qimg.strerror(12345) == "unknown status"


@pytest.mark.parametrize("K,rb", [(32, 16), (512, 16), (544, 32), (2560, 80), (8192, 256),
                                  (14336, 448), (32768, 1024)])
def test_row_blocks_and_image_bytes(L, K, rb):
    assert qimg.row_blocks(K) == rb
    assert qimg.image_bytes(8, K) == 8 * rb * 36
    assert qimg.image_bytes(0, K) == 0


@pytest.mark.parametrize("K", [0, -32, 31, 48, 32768 + 32])
def test_bad_k_sizes(L, K):
    assert qimg.row_blocks(K) == 0
    assert qimg.image_bytes(4, K) == 0
    assert L.qimg_q4_0_tiled_bytes(16, K, 1) == 0


def test_tiled_bytes():
    # 16-row tiles x 4-block chunks; 1 KB codes + 128 B scales per chunk
    assert qimg.lib().qimg_q4_0_tiled_bytes(8192, 8192, 1) == 512 * 64 * 1152
    assert qimg.lib().qimg_q4_0_tiled_bytes(17, 160, 3) == 3 * 2 * 2 * 1152
    assert qimg.lib().qimg_q4_0_tiled_bytes(0, 256, 1) == 0
    assert qimg.lib().qimg_q4_0_tiled_bytes(16, 256, 0) == 0


def test_workspace_bytes(L):
    w = qimg.workspace_bytes(128, 9, 256)
    assert w % 256 == 0 and w >= 4 * (4 + 256 + 257 + 128 * 9)
    assert qimg.workspace_bytes(0, 9, 256) >= 4 * (4 + 256 + 257)
    assert qimg.workspace_bytes(-1, 9, 256) == 0
    assert qimg.workspace_bytes(8, 0, 256) == 0
    assert qimg.workspace_bytes(8, 8, 0) == 0


# ---- producers ----------------------------------------------------------------------------
def emit_rms(L, x=A, ldx=256, gamma=B, rows=4, live=None, K=256, y=C, ldy=256, img=D):
    return L.qimg_emit_rmsnorm(x, ldx, gamma, ctypes.c_float(1e-6), rows, live, K, y, ldy, img, S)


def test_emit_rmsnorm_validation(L):
    assert emit_rms(L, K=48) == qimg.EINVAL
    assert emit_rms(L, K=32768 + 512) == qimg.EUNSUPPORTED
    assert emit_rms(L, rows=-1) == qimg.EINVAL
    assert emit_rms(L, rows=0) == qimg.OK  # nothing to do, nothing launched
    assert emit_rms(L, x=None) == qimg.EINVAL
    assert emit_rms(L, y=None) == qimg.EINVAL
    assert emit_rms(L, ldx=128) == qimg.EINVAL
    assert emit_rms(L, ldy=255) == qimg.EINVAL
    assert emit_rms(L, x=A + 4) == qimg.EALIGN
    assert emit_rms(L, ldx=257) == qimg.EALIGN
    assert emit_rms(L, y=C + 8) == qimg.EALIGN
    assert emit_rms(L, img=D + 4) == qimg.EALIGN
    assert emit_rms(L, gamma=B + 4) == qimg.EALIGN
    assert emit_rms(L, live=B + 2) == qimg.EALIGN
    # outputs overlapping inputs or each other
    assert emit_rms(L, y=A) == qimg.EALIAS
    # an image over x or gamma is declined to the two-step path (it launches: GPU tests); an
    # image over y or over the live count stays an error
    assert emit_rms(L, img=C + 16) == qimg.EALIAS
    assert emit_rms(L, img=C - 64) == qimg.EALIAS
    assert emit_rms(L, img=A + 1024, y=A + 2048) == qimg.EALIAS
    assert emit_rms(L, gamma=C + 512) == qimg.EALIAS
    assert emit_rms(L, live=D + 64) == qimg.EALIAS


def test_emit_glu_validation(L):
    def glu(op=0, g=A, ldg=512, u=A + 1024, ldu=512, rows=4, K=256, y=C, ldy=256, img=D):
        return L.qimg_emit_glu(op, g, ldg, u, ldu, rows, None, K, y, ldy, img, S)

    assert glu(op=7) == qimg.EINVAL
    assert glu(op=-1) == qimg.EINVAL
    # the clamped forms need alpha and limit: only through qimg_emit_glu_ex
    assert glu(op=qimg.GLU_SWIGLU_OAI) == qimg.EINVAL
    assert glu(op=qimg.GLU_SWIGLU_CLAMP) == qimg.EINVAL
    assert glu(u=None) == qimg.EINVAL
    assert glu(ldu=128) == qimg.EINVAL
    assert glu(u=A + 1028) == qimg.EALIGN
    assert glu(y=A + 2048) == qimg.EALIAS
    assert glu(rows=0) == qimg.OK


def test_quantize_validation(L):
    assert L.qimg_quantize_q8_1(A, 256, 4, None, 256, None, S) == qimg.EINVAL
    assert L.qimg_quantize_q8_1(A, 256, 4, None, 200, D, S) == qimg.EINVAL
    assert L.qimg_quantize_q8_1(A, 256, 4, None, 256, A + 512, S) == qimg.EALIAS
    assert L.qimg_quantize_q8_1(A, 256, 4, None, 256, D + 8, S) == qimg.EALIGN


def test_tile_validation(L):
    qs_bytes = 2 * 16 * 8 * 16  # E=2, N=16, K=256
    assert L.qimg_q4_0_tile(None, B, 16, 256, 2, C, S) == qimg.EINVAL
    assert L.qimg_q4_0_tile(A, B, 0, 256, 2, C, S) == qimg.EINVAL
    assert L.qimg_q4_0_tile(A, B, 16, 256, 0, C, S) == qimg.EINVAL
    assert L.qimg_q4_0_tile(A, B, 16, 100, 2, C, S) == qimg.EINVAL
    assert L.qimg_q4_0_tile(A + 4, B, 16, 256, 2, C, S) == qimg.EALIGN
    assert L.qimg_q4_0_tile(A, B + 1, 16, 256, 2, C, S) == qimg.EALIGN
    assert L.qimg_q4_0_tile(A, B, 16, 256, 2, C + 8, S) == qimg.EALIGN
    assert L.qimg_q4_0_tile(A, B, 16, 256, 2, A + qs_bytes - 16, S) == qimg.EALIAS
    assert L.qimg_q4_0_tile(A, B, 16, 256, 2, B - 1024, S) == qimg.EALIAS


# ---- readers ------------------------------------------------------------------------------
def readers(*specs):
    arr = (qimg.Reader * len(specs))()
    for i, (w, N, out, ldo) in enumerate(specs):
        arr[i].w, arr[i].N, arr[i].out, arr[i].ldo = w, N, out, ldo
    return arr


def test_mmvq_validation(L):
    r = readers((A, 64, C, 64))
    assert L.mmvq_q4_0_q8_1(r, 0, D, 4, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(r, 9, D, 4, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(r, 1, D, 4, None, 250, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(r, 1, D, -1, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(r, 1, D, 0, None, 256, S) == qimg.OK
    assert L.mmvq_q4_0_q8_1(r, 1, None, 4, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(r, 1, D + 4, 4, None, 256, S) == qimg.EALIGN
    assert L.mmvq_q4_0_q8_1(r, 1, D, 4, B + 2, 256, S) == qimg.EALIGN
    assert L.mmvq_q4_0_q8_1(readers((A, 64, C, 63)), 1, D, 4, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(readers((A, 0, C, 64)), 1, D, 4, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(readers((None, 64, C, 64)), 1, D, 4, None, 256, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1(readers((A + 8, 64, C, 64)), 1, D, 4, None, 256, S) == qimg.EALIGN
    # a code plane of 4 GiB or more (32-bit buffer offsets)
    big = 262144  # rows: 16384 tiles x 256 chunks x 1 KB = 4 GiB at K = 32768
    assert L.mmvq_q4_0_q8_1(readers((A, big, C, big)), 1, D, 4, None, 32768, S) == qimg.EUNSUPPORTED
    assert L.mmvq_q8_0_q8_1(readers((A, big // 2, C, big)), 1, D, 4, None, 32768, S) == qimg.EUNSUPPORTED
    assert L.mmvq_q4_1_q8_1(readers((A, big, C, big)), 1, D, 4, None, 32768, S) == qimg.EUNSUPPORTED
    assert L.mmvq_q4_0_q8_1(readers((A, 64, C + 2, 64)), 1, D, 4, None, 256, S) == qimg.EALIGN
    # output over the weights, the image, the live count or another output
    assert L.mmvq_q4_0_q8_1(readers((A, 64, A + 64, 64)), 1, D, 4, None, 256, S) == qimg.EALIAS
    assert L.mmvq_q4_0_q8_1(readers((A, 64, D + 64, 64)), 1, D, 4, None, 256, S) == qimg.EALIAS
    assert L.mmvq_q4_0_q8_1(readers((A, 64, C, 64)), 1, D, 4, C + 16, 256, S) == qimg.EALIAS
    assert L.mmvq_q4_0_q8_1(readers((A, 64, C, 64), (B, 64, C + 512, 64)), 2, D, 4, None, 256,
                            S) == qimg.EALIAS
    assert L.mmvq_q4_0_q8_1(readers((A, 64, C, 64), (B, 64, A + 1024, 64)), 2, D, 4, None, 256,
                            S) == qimg.EALIAS


def expert_readers(*specs):
    arr = (qimg.ExpertReader * len(specs))()
    for i, (w, N, out, ld) in enumerate(specs):
        arr[i].w, arr[i].N, arr[i].out, arr[i].ld_pair = w, N, out, ld
    return arr


def test_mmvq_id_validation(L):
    E, bucket, k, K = 8, 16, 2, 256
    ws_bytes = qimg.workspace_bytes(bucket, k, E)
    r = expert_readers((A, 64, C, 64))
    WS, IDS = B, B + (1 << 20)

    def call(r=r, n=1, E=E, img=D, ids=IDS, bucket=bucket, k=k, live=None, K=K, ws=WS,
             wsb=ws_bytes):
        return L.mmvq_id_q4_0_q8_1(r, n, E, img, ids, bucket, k, live, K, ws, wsb, S)

    assert call(K=100) == qimg.EINVAL
    assert call(n=0) == qimg.EINVAL
    assert call(E=0) == qimg.EINVAL
    assert call(k=0) == qimg.EINVAL
    assert call(ids=None) == qimg.EINVAL
    assert call(bucket=-1) == qimg.EINVAL
    assert call(bucket=0) == qimg.OK
    assert call(ws=None) == qimg.EWORKSPACE
    assert call(wsb=ws_bytes - 256) == qimg.EWORKSPACE
    assert call(ws=WS + 4) == qimg.EALIGN
    assert call(ids=IDS + 2) == qimg.EALIGN
    assert call(live=IDS + 4096 + 1) == qimg.EALIGN
    assert call(img=D + 4) == qimg.EALIGN
    assert call(ws=D) == qimg.EALIAS
    assert call(ws=IDS - 64) == qimg.EALIAS
    assert call(r=expert_readers((A, 64, WS, 64))) == qimg.EALIAS
    assert call(r=expert_readers((A, 64, IDS, 64))) == qimg.EALIAS
    assert call(r=expert_readers((A, 64, A + 4096, 64))) == qimg.EALIAS
    assert call(r=expert_readers((A, 64, C, 64), (A + (1 << 19), 64, C + 4096, 64)), n=2) == qimg.EALIAS
    assert call(r=expert_readers((A, 64, C, 60))) == qimg.EINVAL


def test_blockdots_validation(L):
    r = readers((A, 64, None, 0))
    assert L.mmvq_q4_0_q8_1_blockdots(r, D, 4, 256, None, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1_blockdots(r, D, 4, 250, C, S) == qimg.EINVAL
    assert L.mmvq_q4_0_q8_1_blockdots(r, D, 0, 256, C, S) == qimg.OK
    assert L.mmvq_q4_0_q8_1_blockdots(r, D, 4, 256, C + 2, S) == qimg.EALIGN
    assert L.mmvq_q4_0_q8_1_blockdots(r, D, 4, 256, D + 64, S) == qimg.EALIAS
    assert L.mmvq_q4_0_q8_1_blockdots(r, D, 4, 256, A, S) == qimg.EALIAS


def test_mmvq_id_limits(L):
    r = expert_readers((A, 64, C, 64))
    WS, IDS = B, B + (1 << 24)
    big = qimg.workspace_bytes(4097, 1, 8)
    assert L.mmvq_id_q4_0_q8_1(r, 1, 8, D, IDS, 4097, 1, None, 256, WS, big, S) == qimg.EUNSUPPORTED
    assert L.mmvq_id_q4_0_q8_1(r, 1, 8, D, IDS, 1024, 5, None, 256, WS,
                               qimg.workspace_bytes(1024, 5, 8), S) == qimg.EUNSUPPORTED
    assert L.mmvq_id_q4_0_q8_1(r, 1, 1025, D, IDS, 8, 2, None, 256, WS,
                               qimg.workspace_bytes(8, 2, 1025), S) == qimg.EUNSUPPORTED


def test_per_slot_routed_validation(L):
    """The per-slot image has bucket*top_k rows: an image that overlaps an output within that
    extent (but past a token-row image) is an alias only for the per-slot reader."""
    E, bucket, k, K = 8, 16, 4, 256
    ws_bytes = qimg.workspace_bytes(bucket, k, E)
    WS, IDS = B, B + (1 << 20)
    out = D + qimg.image_bytes(bucket, K) + 256  # just past a token-row image
    r = expert_readers((A, 64, out, 64))
    per = L.mmvq_id_q4_0_q8_1_per_slot
    args = lambda f, **kw: f(kw.get("r", r), 1, E, D, IDS, kw.get("bucket", bucket), k, None, K, WS,
                             ws_bytes, S)
    assert args(per) == qimg.EALIAS
    assert args(per, bucket=0) == qimg.OK
    assert per(r, 1, E, D, IDS, bucket, k, None, 100, WS, ws_bytes, S) == qimg.EINVAL
    assert per(r, 1, E, D, IDS, 1024, 5, None, K, WS, qimg.workspace_bytes(1024, 5, E), S) == qimg.EUNSUPPORTED


def test_emit_glu_per_slot_validation(L):
    def glu(op=0, g=A, ldg=512, u=A + 1024, ldu=512, bucket=4, k=2, K=256, y=C, ldy=256, img=D):
        return L.qimg_emit_glu_per_slot(op, g, ldg, u, ldu, bucket, k, None, K, y, ldy, img, S)

    assert glu(op=7) == qimg.EINVAL
    assert glu(op=qimg.GLU_SWIGLU_OAI) == qimg.EINVAL
    assert glu(k=0) == qimg.EINVAL
    assert glu(bucket=-1) == qimg.EINVAL
    assert glu(bucket=0) == qimg.OK
    assert glu(bucket=1025, k=4) == qimg.EUNSUPPORTED
    assert glu(K=48) == qimg.EINVAL
    assert glu(u=A + 1028) == qimg.EALIGN
    # the image spans bucket*top_k rows: 8 rows here
    assert glu(img=C - qimg.image_bytes(8, 256) + 16) == qimg.EALIAS


def test_moe_combine_validation(L):
    def comb(x=A, ldp=256, w=B, ids=B + 4096, E=8, bucket=4, k=2, live=None, N=256, out=C, ldo=256):
        return L.qimg_moe_combine(x, ldp, w, ids, E, bucket, k, live, N, out, ldo, S)

    assert comb(x=None) == qimg.EINVAL
    assert comb(w=None) == qimg.EINVAL
    assert comb(ids=None) == qimg.EINVAL
    assert comb(out=None) == qimg.EINVAL
    assert comb(E=0) == qimg.EINVAL
    assert comb(k=0) == qimg.EINVAL
    assert comb(N=0) == qimg.EINVAL
    assert comb(ldp=128) == qimg.EINVAL
    assert comb(ldo=128) == qimg.EINVAL
    assert comb(bucket=-1) == qimg.EINVAL
    assert comb(bucket=0) == qimg.OK
    assert comb(N=250, ldp=256, ldo=256) == qimg.EUNSUPPORTED
    assert comb(x=A + 4) == qimg.EALIGN
    assert comb(out=C + 8) == qimg.EALIGN
    assert comb(ldo=258) == qimg.EALIGN
    assert comb(ldp=258) == qimg.EALIGN
    assert comb(w=B + 2) == qimg.EALIGN
    assert comb(live=B + 8192 + 2) == qimg.EALIGN
    assert comb(out=A + 1024) == qimg.EALIAS
    assert comb(out=B) == qimg.EALIAS
    assert comb(out=B + 4096) == qimg.EALIAS
    assert comb(live=C + 64) == qimg.EALIAS


def test_emit_glu_ex_validation(L):
    inf, nan = float("inf"), float("nan")

    def glu(op=5, alpha=1.702, limit=7.0, g=A, ldg=512, u=A + 1024, ldu=512, rows=4, K=256, y=C,
            ldy=256, img=D):
        return L.qimg_emit_glu_ex(op, ctypes.c_float(alpha), ctypes.c_float(limit), g, ldg, u, ldu, rows,
                                  None, K, y, ldy, img, S)

    assert glu(op=7) == qimg.EINVAL
    assert glu(alpha=nan) == qimg.EINVAL
    assert glu(alpha=inf) == qimg.EINVAL
    assert glu(limit=-1.0) == qimg.EINVAL
    assert glu(limit=nan) == qimg.EINVAL
    assert glu(op=6, limit=-0.5) == qimg.EINVAL
    assert glu(rows=0) == qimg.OK
    assert glu(u=None) == qimg.EINVAL
    assert glu(g=A + 4) == qimg.EALIGN
    assert glu(y=A + 1024) == qimg.EALIAS


def test_emit_rmsnorm_ex_validation(L):
    def rms(beta=B + 4096, scale=1.0, x=A, gamma=B, y=C, img=D):
        return L.qimg_emit_rmsnorm_ex(x, 256, gamma, beta, ctypes.c_float(scale), ctypes.c_float(1e-6), 4,
                                      None, 256, y, 256, img, S)

    assert rms(scale=float("nan")) == qimg.EINVAL
    assert rms(scale=float("inf")) == qimg.EINVAL
    assert rms(beta=B + 4100) == qimg.EALIGN
    assert rms(y=B + 4096) == qimg.EALIAS
    assert rms(img=C + 64) == qimg.EALIAS
    assert rms(x=None) == qimg.EINVAL


def test_moe_router_validation(L):
    def router(x=A, ldx=256, w=B, E=8, bucket=4, live=None, K=256, lg=C, ldl=8):
        return L.qimg_moe_router(x, ldx, w, E, bucket, live, K, lg, ldl, S)

    assert router(K=100) == qimg.EINVAL
    assert router(E=0) == qimg.EINVAL
    assert router(x=None) == qimg.EINVAL
    assert router(ldx=128) == qimg.EINVAL
    assert router(ldl=4) == qimg.EINVAL
    assert router(bucket=0) == qimg.OK
    assert router(x=A + 4) == qimg.EALIGN
    assert router(ldx=258) == qimg.EALIGN
    assert router(lg=C + 2) == qimg.EALIGN
    assert router(lg=A + 64) == qimg.EALIAS
    assert router(lg=B + 1024) == qimg.EALIAS


def test_moe_topk_validation(L):
    def topk(lg=A, ldl=256, E=256, bucket=4, live=None, k=8, ids=B, w=C):
        return L.qimg_moe_topk(lg, ldl, E, bucket, live, k, ids, w, S)

    assert topk(k=0) == qimg.EINVAL
    assert topk(k=257) == qimg.EINVAL
    assert topk(ldl=100) == qimg.EINVAL
    assert topk(ids=None) == qimg.EINVAL
    assert topk(E=2048, ldl=2048) == qimg.EUNSUPPORTED
    assert topk(k=65, E=256) == qimg.EUNSUPPORTED
    assert topk(bucket=0) == qimg.OK
    assert topk(ids=B + 2) == qimg.EALIGN
    assert topk(ids=A + 64) == qimg.EALIAS
    assert topk(w=B + 16) == qimg.EALIAS
    assert topk(live=B + 32) == qimg.EALIAS


def test_f32_reader_validation(L):
    def rd(y=A, ldy=256, v=B, N=1, rows=8, live=None, K=256, out=C, ldo=1):
        return L.qimg_f32_reader(y, ldy, v, N, rows, live, K, out, ldo, S)

    assert rd(K=100) == qimg.EINVAL
    assert rd(N=0) == qimg.EINVAL
    assert rd(v=None) == qimg.EINVAL
    assert rd(ldy=128) == qimg.EINVAL
    assert rd(rows=0) == qimg.OK
    assert rd(y=A + 4) == qimg.EALIGN
    assert rd(out=A + 64) == qimg.EALIAS
    assert rd(out=B) == qimg.EALIAS


def test_noalloc_routed_validation(L):
    r = expert_readers((A, 64, C, 64))
    na = lambda bucket=16, k=2, E=8, ids=B, rd=r, n=1: L.mmvq_id_q4_0_q8_1_noalloc(
        rd, n, E, D, ids, bucket, k, None, 256, S)
    assert na(ids=None) == qimg.EINVAL
    assert na(E=0) == qimg.EINVAL
    assert na(n=0) == qimg.EINVAL
    assert na(bucket=0) == qimg.OK
    # beyond the per-GPU plan array (and the routed pair limit): rejected before anything else
    assert na(bucket=4097, k=1) == qimg.EUNSUPPORTED
    assert na(E=2048) == qimg.EUNSUPPORTED


def test_read_ceiling_validation(L):
    rc = lambda buf=A, n=1 << 20, sink=D: L.qimg_read_ceiling(buf, n, sink, S)
    assert rc(buf=None) == qimg.EINVAL
    assert rc(sink=None) == qimg.EINVAL
    assert rc(n=0) == qimg.EINVAL
    assert rc(n=1000) == qimg.EINVAL
    assert rc(n=1 << 31) == qimg.EINVAL
    assert rc(buf=A + 4) == qimg.EALIGN
    assert rc(sink=D + 2) == qimg.EALIGN
    assert rc(sink=A + 1024) == qimg.EALIAS
