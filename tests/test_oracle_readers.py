"""Pins of the oracle's readers and routed plan (CPU only).

block dot    -> brute force over an explicitly unpacked weight vector; closed-form nibbles
reader (f64) -> brute-force float64 dequantize-and-dot, which differs from the Q8_1 form by
                a known closed form (the image stores s in fp16)
accuracy     -> NMSE against the unquantized float64 activation <= 5e-4, the CPU bound of
                "Share temporary Q8_1 activation images", GLU producer evidence
plan         -> brute-force sort of the live pairs; the receipt counts of the padded-bucket page
routed       -> reduces to the ordinary reader with the pair's expert and image row
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from q8_activation_quant_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unpack_weights(qs):
    """Element j of a block: low nibble of byte j (j < 16), high nibble of byte j-16."""
    lo = (qs & 15).astype(np.int64)
    hi = (qs >> 4).astype(np.int64)
    return np.concatenate([lo, hi], axis=-1)  # [..., 32]


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _random_image(g, rows, K):
    y = g.standard_normal((rows, K)).astype(np.float32)
    return y, O.quantize(y)


def test_blockdots_brute_force():
    g = np.random.default_rng(0)
    K, N, T = 96, 5, 3
    w = W.q4_0_weights(g, (N,), K)
    y, img = _random_image(g, T, K)
    sumi = O.blockdots(w.qs, K, img, T, T)
    codes, _, _ = O.image_planes(img, T, K)
    wq = _unpack_weights(w.qs)  # [N][Kb][32]
    ref = np.einsum("nbj,tbj->tnb", wq, codes[:, : K // 32].astype(np.int64))
    assert np.array_equal(sumi, ref)
    assert np.abs(sumi).max() <= 15 * 127 * 32


@pytest.mark.parametrize("byte,expect", [(0x00, "zero"), (0xFF, "all15"), (0x0F, "lo15"), (0xF0, "hi15")])
def test_blockdots_closed_form_nibbles(byte, expect):
    g = np.random.default_rng(1)
    K = 32
    y, img = _random_image(g, 1, K)
    codes, _, _ = O.image_planes(img, 1, K)
    c = codes[0, 0].astype(np.int64)
    qs = np.full((1, 1, 16), byte, np.uint8)
    s = int(O.blockdots(qs, K, img, 1, 1)[0, 0, 0])
    want = {"zero": 0, "all15": 15 * c.sum(), "lo15": 15 * c[:16].sum(), "hi15": 15 * c[16:].sum()}[expect]
    assert s == want


def test_reader_matches_bruteforce_dequantize_and_dot():
    g = np.random.default_rng(2)
    for K, N, T in [(32, 3, 1), (64, 4, 2), (2592, 3, 2)]:
        w = W.q4_0_weights(g, (N,), K)
        y, img = _random_image(g, T, K)
        out = O.mmvq(w.qs, w.d, K, img, T, T)
        Kb = K // 32
        codes, d16, s16 = O.image_planes(img, T, K)
        wq = _unpack_weights(w.qs).astype(np.float64) - 8.0      # [N][Kb][32]
        wd = wq * _f16(w.d)[..., None]                            # dequantized weights
        ad = codes[:, :Kb].astype(np.float64) * _f16(d16[:, :Kb])[..., None]  # dequantized act
        bf = np.einsum("nbj,tbj->tn", wd, ad)
        # the Q8_1 form subtracts 8*d_w*s16 where the dequantized form subtracts
        # 8*d_w*d16*sum(c): o - bf = sum_b 8 d_w (d16 sum(c) - s16)
        diff = np.einsum("nb,tb->tn", _f16(w.d),
                         8.0 * (_f16(d16[:, :Kb]) * codes[:, :Kb].astype(np.float64).sum(-1) - _f16(s16[:, :Kb])))
        scale = np.einsum("nbj,tbj->tn", np.abs(wd), np.abs(ad)) + np.abs(diff) + 1e-300
        assert (np.abs(out - bf - diff) <= 1e-12 * scale).all()


def test_all_eight_weight_block_shows_the_stored_sum():
    # every nibble 8 -> dequantized weight 0, so the dequantized dot is 0 and the Q8_1 form
    # returns exactly sum_b d_w * 8 * (d16*sum(c) - s16)
    g = np.random.default_rng(3)
    K = 256
    y, img = _random_image(g, 1, K)
    qs = np.full((1, K // 32, 16), 0x88, np.uint8)
    d = np.full((1, K // 32), np.float16(0.5).view(np.uint16), np.uint16)
    out = O.mmvq(qs, d, K, img, 1, 1)[0, 0]
    codes, d16, s16 = O.image_planes(img, 1, K)
    Kb = K // 32
    expect = np.sum(0.5 * 8.0 * (_f16(d16[0, :Kb]) * codes[0, :Kb].sum(-1) - _f16(s16[0, :Kb])))
    assert abs(out - expect) <= 1e-15 * (np.abs(_f16(s16)).sum() * 4 + 1e-300)


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_nmse_against_unquantized_float64(config):
    wl = W.make(config, small=True)
    K = wl.K
    if wl.producer == "rmsnorm":
        y = O.rmsnorm(wl.x, wl.gamma, W.EPS)
        x64 = wl.x.astype(np.float64)
        y64 = x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + W.EPS) * wl.gamma.astype(np.float64)
    else:
        import scipy.special
        y = O.glu(wl.gu, wl.producer)
        g64, u64 = wl.gu[:, :K].astype(np.float64), wl.gu[:, K:].astype(np.float64)
        y64 = g64 / (1 + np.exp(-g64)) * u64
    img = O.quantize(y)
    T = y.shape[0]
    for r in wl.readers:
        qs = r.qs.reshape(-1, K // 32, 16)[:64]
        d = r.d.reshape(-1, K // 32)[:64]
        out = O.mmvq(qs, d, K, img, T, T)
        wd = (_unpack_weights(qs).astype(np.float64) - 8.0) * _f16(d)[..., None]
        ref = y64 @ wd.reshape(wd.shape[0], -1).T  # unquantized activation, same weights
        nmse = np.sum((out - ref) ** 2) / np.sum(ref ** 2)
        assert nmse <= 5e-4, nmse


def _read_receipt():
    rows = []
    for line in open(os.path.join(GOLDEN, "routed_plan_receipt.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([int(v) for v in line.split()])
    return rows


@pytest.mark.parametrize("bucket,live,top_k,pairs,largest", _read_receipt())
def test_plan_receipt_counts(bucket, live, top_k, pairs, largest):
    E = 256
    g = np.random.default_rng(bucket * 1000 + live)
    ids, _ = W.topk_ids(g, bucket, E, top_k)
    counts, offsets, members, bad = O.plan(ids, live, E)
    assert bad == 0 and counts.sum() == pairs and offsets[E] == pairs
    assert members.max() == largest and len(members) == pairs


def test_plan_against_brute_force_sort():
    g = np.random.default_rng(4)
    for bucket, k, E in [(128, 9, 256), (8, 8, 128), (5, 3, 4), (1, 1, 1)]:
        ids, _ = W.topk_ids(g, bucket, E, k) if k <= E else (None, None)
        for live in sorted({0, 1, bucket // 2, bucket}):
            counts, offsets, members, bad = O.plan(ids, live, E)
            P = live * k
            flat = ids.reshape(-1)[:P]
            ref = [p for _, p in sorted((int(flat[p]), p) for p in range(P))]
            assert members.tolist() == ref
            assert np.array_equal(counts, np.bincount(flat, minlength=E))
            assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
            assert sorted(members.tolist()) == list(range(P))


def test_plan_skips_out_of_range_experts():
    ids = np.array([[0, 5], [9, 1], [-1, 2]], np.int32)
    counts, offsets, members, bad = O.plan(ids, 3, 6)
    assert bad == 2
    assert members.tolist() == [0, 3, 5, 1]  # experts 0, 1, 2, 5
    assert offsets[6] == 4


def test_routed_reduces_to_ordinary_reader():
    g = np.random.default_rng(5)
    E, N, K, B, k, live = 6, 3, 64, 4, 2, 3
    w = W.q4_0_weights(g, (E, N), K)
    ids, _ = W.topk_ids(g, B, E, k)
    y, img = _random_image(g, B, K)
    out = O.mmvq_id(w.qs, w.d, E, K, img, B, ids, live)
    codes, d16, s16 = O.image_planes(img, B, K)
    Kb = K // 32
    for p in range(live * k):
        t, e = p // k, ids.reshape(-1)[p]
        wd = (_unpack_weights(w.qs[e]).astype(np.float64) - 8.0) * _f16(w.d[e])[..., None]
        ad = codes[t, :Kb].astype(np.float64) * _f16(d16[t, :Kb])[..., None]
        diff = 8.0 * (_f16(d16[t, :Kb]) * codes[t, :Kb].sum(-1) - _f16(s16[t, :Kb]))
        ref = np.einsum("nbj,bj->n", wd, ad) + _f16(w.d[e]) @ diff
        assert np.allclose(out[p], ref, rtol=1e-12, atol=1e-14)


def test_per_slot_routed_reader_uses_the_pair_image_row():
    """Per-slot image (one row per (token, slot) pair): the routed reader of pair p equals the
    brute-force float64 dequantize-and-dot of expert ids[p] with image row p; bad ids stay NaN."""
    g = np.random.default_rng(6)
    E, N, K, B, k, live = 5, 3, 96, 4, 3, 3
    w = W.q4_0_weights(g, (E, N), K)
    ids, _ = W.topk_ids(g, B, E, k)
    ids[1, 2] = E  # out of range: skipped
    y, img = _random_image(g, B * k, K)
    out = O.mmvq_id(w.qs, w.d, E, K, img, B * k, ids, live, per_slot=True)
    tok = O.mmvq_id(w.qs, w.d, E, K, img, B * k, ids, live)  # token rows: a different answer
    codes, d16, s16 = O.image_planes(img, B * k, K)
    Kb = K // 32
    for p in range(live * k):
        e = ids.reshape(-1)[p]
        if e >= E:
            assert np.isnan(out[p]).all()
            continue
        wd = (_unpack_weights(w.qs[e]).astype(np.float64) - 8.0) * _f16(w.d[e])[..., None]
        ad = codes[p, :Kb].astype(np.float64) * _f16(d16[p, :Kb])[..., None]
        diff = 8.0 * (_f16(d16[p, :Kb]) * codes[p, :Kb].sum(-1) - _f16(s16[p, :Kb]))
        ref = np.einsum("nbj,bj->n", wd, ad) + _f16(w.d[e]) @ diff
        assert np.allclose(out[p], ref, rtol=1e-12, atol=1e-14)
    assert not np.allclose(out[k:2 * k], tok[k:2 * k], equal_nan=True)


def test_moe_combine_against_float64():
    """fma chain over the slots: within top_k roundings of the exact float64 weighted sum."""
    wl = W.make(4, moe=True)
    x, w, ids = wl.pair_x, wl.route_w, wl.ids
    out = O.moe_combine(x, w, ids, wl.E, wl.T)
    prod = w.astype(np.float64)[:, :, None] * x.astype(np.float64)
    exact = prod.sum(axis=1)
    bound = wl.top_k * 2.0 ** -24 * np.abs(prod).sum(axis=1)
    assert (np.abs(out - exact) <= bound).all()
    assert np.abs(out - exact).max() > 0  # f32 rounding is visible: not a float64 sum


def test_moe_combine_closed_forms():
    g = np.random.default_rng(7)
    rows, k, N, E = 3, 4, 64, 6
    x = g.standard_normal((rows, k, N)).astype(np.float32)
    ids = np.array([[0, 1, 2, 3], [4, 5, 0, 1], [2, 3, 4, 5]], np.int32)
    # one-hot weights give that slot's row exactly
    for s in range(k):
        w = np.zeros((rows, k), np.float32)
        w[:, s] = 1.0
        assert np.array_equal(O.moe_combine(x, w, ids, E, rows), x[:, s])
    # small integers: every product and partial sum is exact
    xi = g.integers(-50, 50, size=(rows, k, N)).astype(np.float32)
    wi = g.integers(-8, 8, size=(rows, k)).astype(np.float32)
    want = (wi[:, :, None].astype(np.int64) * xi.astype(np.int64)).sum(axis=1)
    assert np.array_equal(O.moe_combine(xi, wi, ids, E, rows), want.astype(np.float32))
    # a pair whose expert is out of range contributes nothing, as a zero weight would
    bad = ids.copy()
    bad[1, 2] = E
    bad[2, 0] = -1
    wz = wi.copy()
    wz[1, 2] = 0.0
    wz[2, 0] = 0.0
    assert np.array_equal(O.moe_combine(xi, wi, bad, E, rows), O.moe_combine(xi, wz, ids, E, rows))
    # live rows only
    assert O.moe_combine(x, wi, ids, E, 2).shape == (2, N)


# ---- device router and top-k ------------------------------------------------------------------
@pytest.mark.parametrize("K", [256, 2560, 2592])
def test_router_against_float64(K):
    g = np.random.default_rng(K)
    x = g.standard_normal((5, K)).astype(np.float32)
    w = (g.standard_normal((40, K)) * 0.05).astype(np.float32)
    got = O.moe_router(x, w, 5).astype(np.float64)
    prod = np.abs(x.astype(np.float64))[:, None, :] * np.abs(w.astype(np.float64))[None, :, :]
    J = -(-K // 256)
    levels = max(0, math.ceil(math.log2(J)))
    bound = (3 + levels + 6 + 1) * 2.0 ** -24 * prod.sum(-1)  # leaf fma chain, then two pairwise trees
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert (np.abs(got - exact) <= bound).all()


def test_router_closed_forms():
    g = np.random.default_rng(41)
    K, E = 1024, 24
    w = g.standard_normal((E, K)).astype(np.float32)
    # a one-hot activation picks one weight column exactly
    x = np.zeros((3, K), np.float32)
    x[0, 5], x[1, 700], x[2, 1023] = 1.0, 1.0, -1.0
    assert np.array_equal(O.moe_router(x, w, 3), np.stack([w[:, 5], w[:, 700], -w[:, 1023]]))
    # small integers: every partial sum is exact in any order
    xi = g.integers(-8, 8, size=(2, K)).astype(np.float32)
    wi = g.integers(-8, 8, size=(E, K)).astype(np.float32)
    assert np.array_equal(O.moe_router(xi, wi, 2), (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float32))
    # live rows only
    assert O.moe_router(xi, wi, 1).shape == (1, E)


def test_topk_against_stable_sort_and_softmax():
    g = np.random.default_rng(42)
    R, E, k = 64, 256, 9
    logits = g.standard_normal((R, E)).astype(np.float32)
    logits[3, 10] = logits[3, 200] = logits[3].max() + 1  # a tie at the top: lower id first
    logits[7, :] = 0.5                                    # all equal: ids 0..k-1
    ids, w = O.moe_topk(logits, k)
    want = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, want)
    assert ids[3, 0] == 10 and ids[3, 1] == 200
    assert np.array_equal(ids[7], np.arange(k)) and (w[7] == np.float32(1.0) / np.float32(k)).all()
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    sm = np.exp(sel - sel[:, :1])
    sm /= sm.sum(axis=1, keepdims=True)
    assert np.abs(w - sm).max() <= 8 * 2.0 ** -24
    assert (np.diff(w, axis=1) <= 0).all()  # descending logits give non-increasing weights
    # k = E: a full stable sort
    ids_all, _ = O.moe_topk(logits[:2], E)
    assert np.array_equal(ids_all, np.argsort(-logits[:2], axis=1, kind="stable"))
    # live rows only
    assert O.moe_topk(logits, k, live=5)[0].shape == (5, k)


# ---- other weight formats (Q8_0, Q4_1) --------------------------------------------------------
def test_q8_0_reader_is_the_dequantized_dot():
    g = np.random.default_rng(51)
    N, K, T = 5, 160, 3
    w = W.q8_0_weights(g, (N,), K)
    y, img = _random_image(g, T, K)
    out = O.mmvq_fmt("q8_0", w.qs, w.d, None, K, img, T, T)
    codes, d16, s16 = O.image_planes(img, T, K)
    Kb = K // 32
    wd = w.qs.astype(np.float64) * _f16(w.d)[..., None]                       # [N][Kb][32]
    ad = codes[:, :Kb].astype(np.float64) * _f16(d16[:, :Kb])[..., None]    # [T][Kb][32]
    ref = np.einsum("nbj,tbj->tn", wd, ad)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-15)


def test_q4_1_reader_is_the_dequantized_dot_up_to_the_stored_sum():
    g = np.random.default_rng(52)
    N, K, T = 6, 96, 4
    w = W.q4_1_weights(g, (N,), K)
    y, img = _random_image(g, T, K)
    out = O.mmvq_fmt("q4_1", w.qs, w.d, w.m, K, img, T, T)
    codes, d16, s16 = O.image_planes(img, T, K)
    Kb = K // 32
    wd = _unpack_weights(w.qs).astype(np.float64) * _f16(w.d)[..., None] + _f16(w.m)[..., None]
    ad = codes[:, :Kb].astype(np.float64) * _f16(d16[:, :Kb])[..., None]
    bf = np.einsum("nbj,tbj->tn", wd, ad)
    # the stored half sum replaces d_a * sum(c): out - bf = sum_b m_w (s16 - d16 sum c)
    diff = _f16(s16[:, :Kb]) - _f16(d16[:, :Kb]) * codes[:, :Kb].astype(np.float64).sum(-1)
    assert np.allclose(out - bf, diff @ _f16(w.m).T, rtol=1e-9, atol=1e-14)


def test_q4_1_with_minimum_minus_8d_is_q4_0():
    # m = -8 d (exact in fp16) turns Q4_1's d q + m into Q4_0's d (q - 8)
    g = np.random.default_rng(53)
    N, K, T = 7, 256, 3
    w = W.q4_0_weights(g, (N,), K)
    m = (-8.0 * w.d.view(np.float16).astype(np.float32)).astype(np.float16).view(np.uint16)
    y, img = _random_image(g, T, K)
    q41 = O.mmvq_fmt("q4_1", w.qs, w.d, m, K, img, T, T)
    q40 = O.mmvq(w.qs, w.d, K, img, T, T)
    assert np.allclose(q41, q40, rtol=1e-13, atol=1e-16)
