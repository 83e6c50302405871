"""The allocation-free routed reader (mmvq_id_q4_0_q8_1_noalloc) against the workspace one.

Both run the same kernels; the first keeps the routing plan in the library's per-GPU static
array instead of a caller workspace. Two calls in a row, the second with a smaller bucket, must
each give the bytes of mmvq_id_q4_0_q8_1 on the same inputs (the array keeps the previous
call's plan, which the kernel rewrites entirely).
"""
import numpy as np
import pytest

import helpers as H
from q8_activation_quant_amd import qimg
from q8_activation_quant_amd import workloads as W

pytestmark = pytest.mark.gpu


def _case(cfg, live, small):
    torch = H.torch()
    wl = W.make(cfg, live=live, small=small)
    B, k, K = wl.T, wl.top_k, wl.K
    L = wl.T if live is None else live
    x = H.dev(wl.x)
    y = H.sentinel_f32(B, K)
    img = H.sentinel_u8(qimg.image_bytes(B, K))
    lt = H.live_tensor(L)
    qimg.emit_rmsnorm(x, H.dev(wl.gamma), W.EPS, y, img, lt)
    ids = H.dev(wl.ids)
    tiles = [qimg.tile_q4_0(H.dev(r.qs), H.dev(r.d), K) for r in wl.readers]
    res = []
    for noalloc in (True, False):
        outs = [H.sentinel_f32(B, k, r.d.shape[-2]) for r in wl.readers]
        specs = [(t, r.d.shape[-2], o) for t, r, o in zip(tiles, wl.readers, outs)]
        if noalloc:
            qimg.mmvq_id_noalloc(specs, wl.E, img, ids, lt, K)
        else:
            ws = torch.empty(qimg.workspace_bytes(B, k, wl.E) // 4, dtype=torch.int32, device="cuda")
            qimg.mmvq_id(specs, wl.E, img, ids, lt, K, ws)
        torch.cuda.synchronize()
        res.append([H.host(o) for o in outs])
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "cfg %d live %s differs" % (cfg, live)
        assert (a.reshape(B * k, -1)[L * k:].view(np.uint8) == H.SENTINEL_BYTE).all()


def test_noalloc_routed_equals_workspace_routed_twice():
    print("noalloc: padded bucket live 113, then routed T8", flush=True)
    _case(5, 113, False)   # 1,017 live pairs of a 128 x 9 bucket
    _case(4, None, True)   # then 64 pairs: a smaller plan over the same array
