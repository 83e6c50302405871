"""Pins of the oracle's scalar numerics against libraries and closed forms (CPU only).

binary16 conversion  -> numpy's IEEE float16 conversion (a library routine)
exp_q / erfc_q       -> float64 libm / scipy within the published error of the method
RMS / GLU producers  -> float64 textbook formulas within a rounding-count bound, plus
                        closed-form rows whose f32 result is known exactly
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import oracle as O

U = 2.0 ** -24  # unit roundoff of binary32


# ---- binary16 --------------------------------------------------------------------------------
def test_f32_to_f16_matches_numpy_on_dense_bit_sweep():
    g = np.random.default_rng(7)
    # random bit patterns over the whole f32 range plus a dense sweep of the f16-relevant range
    pats = [g.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)]
    lo, hi = np.float32(2.0 ** -26).view(np.uint32), np.float32(70000.0).view(np.uint32)
    pats.append(np.arange(lo, hi, 61, dtype=np.uint32))
    bits = np.concatenate(pats)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ours = O.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_to_f16_ties_go_to_even():
    # midpoints between consecutive f16 values (normal and subnormal) are exact in f32
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).view(np.float16).astype(np.float64)
    mid = ((a + b) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (a + b) / 2)  # midpoints representable
    ours = O.f32_to_f16_bits(mid)
    expect = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(ours, expect)
    assert O.f32_to_f16_bits(np.float32(65520.0))[()] == 0x7C00  # rounds up to +inf
    assert O.f32_to_f16_bits(np.float32(65519.996))[()] == 0x7BFF


def test_f16_to_f64_exact_for_all_patterns():
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    ours = np.array([O.f16_to_f64(int(v)) for v in h[::7]])
    r = ref[::7]
    ok = np.isnan(r) & np.isnan(ours) | (ours == r)
    assert ok.all()


# ---- exp_q -----------------------------------------------------------------------------------
def _ulp_err(ours, ref):
    ours = ours.astype(np.float64)
    return np.abs(ours - ref) / np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)


def test_exp_q_accuracy_against_libm():
    x = np.concatenate([np.linspace(-86.0, 88.7, 2_000_001, dtype=np.float32),
                        np.random.default_rng(1).uniform(-5, 5, 500_000).astype(np.float32)])
    ref = np.exp(x.astype(np.float64))
    err = _ulp_err(O.exp_q(x), ref)
    assert err.max() <= 2.0, err.max()


def test_exp_q_special_values_and_monotone():
    e = O.exp_q(np.array([0.0, -0.0, np.inf, -np.inf, 89.0, 88.8, -86.01, -1e30, 1e30], np.float32))
    assert e[0] == 1.0 and e[1] == 1.0
    assert e[2] == np.inf and e[3] == 0.0 and e[4] == np.inf
    assert np.isfinite(e[5]) or e[5] == np.inf  # boundary: either side of overflow is allowed
    assert e[6] == 0.0 and e[7] == 0.0 and e[8] == np.inf
    assert np.isnan(O.exp_q(np.array([np.nan], np.float32))[0])
    x = np.sort(np.random.default_rng(2).uniform(-20, 20, 200_000).astype(np.float32))
    y = O.exp_q(x)
    assert (np.diff(y) >= 0).all()
    # exact powers: e^(k ln2) for integer k lands within 1 ulp of 2^k
    k = np.arange(-100, 101)
    xk = (k * math.log(2.0)).astype(np.float32)
    assert (_ulp_err(O.exp_q(xk), np.exp(xk.astype(np.float64))) <= 1.5).all()


# ---- erfc_q ----------------------------------------------------------------------------------
def test_erfc_q_accuracy_against_scipy():
    z = np.concatenate([np.linspace(0, 9.0, 1_000_001, dtype=np.float32),
                        np.abs(np.random.default_rng(3).standard_normal(200_000)).astype(np.float32)])
    ref = scipy.special.erfc(z.astype(np.float64))
    ours = O.erfc_q(z).astype(np.float64)
    # Numerical Recipes' erfcc: fractional error < 1.2e-7; f32 evaluation adds the rounding of
    # the exponent argument (about z^2 ulps of 2^-24) and a few roundings of the rest.
    bound = ref * (1.2e-7 + (z.astype(np.float64) ** 2 + 8.0) * U)
    assert (np.abs(ours - ref) <= bound).all()


def test_erfc_q_special_values():
    v = O.erfc_q(np.array([0.0, np.inf, 20.0], np.float32))
    assert abs(v[0] - 1.0) <= 2e-7
    assert v[1] == 0.0 and v[2] == 0.0


# ---- GLU producers ---------------------------------------------------------------------------
def _glu_f64(g, u, op):
    g = g.astype(np.float64)
    u = u.astype(np.float64)
    if op == "swiglu":
        act = g / (1.0 + np.exp(-g))
    else:  # 1 + erf(z) == erfc(-z), which keeps relative accuracy for negative z
        act = 0.5 * g * scipy.special.erfc(-g / math.sqrt(2.0))
    return act * u


@pytest.mark.parametrize("op", ["swiglu", "geglu_erf"])
def test_glu_against_float64_textbook(op):
    g = np.random.default_rng(4)
    K = 4096
    gu = (g.standard_normal((3, 2 * K)) * np.array([1.0, 3.0, 8.0])[:, None]).astype(np.float32)
    y = O.glu(gu, op).astype(np.float64)
    ref = _glu_f64(gu[:, :K], gu[:, K:], op)
    if op == "swiglu":
        # exp_q within 2 ulp, then 1+e, g/den and *u: a few more roundings
        rel = 10 * U
    else:
        # erfcc's published 1.2e-7, plus the rounding of z = g/sqrt2 amplified by the slope
        # of log erfc (about 2z per unit of z), plus the exponent-argument rounding (z^2 ulps)
        z2 = (gu[:, :K].astype(np.float64) ** 2) / 2.0
        rel = 1.2e-7 + (4.0 * z2 + 16.0) * U
    # exp_q flushes results below e^-86 to zero: for gates below about -13 the f32 act may be
    # zero where the true one is below 1e-37 * |g|
    absf = 1e-36 * np.abs(gu[:, :K].astype(np.float64) * gu[:, K:].astype(np.float64))
    assert (np.abs(y - ref) <= rel * np.abs(ref) + absf).all()


def test_glu_closed_forms():
    z = np.zeros((1, 8), np.float32)
    for op in ("swiglu", "geglu_erf"):
        assert (O.glu(z, op) == 0).all()
    # gate >= 18: e^-g < 2^-25, so 1 + e^-g and Phi(g) round to 1 and act(g) == g exactly
    gu = np.array([[18.0, 20.0, 30.0, 40.0, 1.5, -2.0, 0.25, 3.0]], np.float32)
    for op in ("swiglu", "geglu_erf"):
        y = O.glu(gu, op)
        assert np.array_equal(y[0], gu[0, :4] * gu[0, 4:])
    # large negative gate: SwiGLU act tends to -0 / tiny negative, GeGLU act to -0
    gu = np.array([[-100.0, -200.0, 1.0, 1.0]], np.float32)
    assert (np.abs(O.glu(gu, "swiglu")) < 1e-30).all()
    assert (np.abs(O.glu(gu, "geglu_erf")) < 1e-30).all()


# ---- RMS producer ----------------------------------------------------------------------------
def _rms_f64(x, gamma, eps):
    x = x.astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    y = x * r
    return y if gamma is None else y * gamma.astype(np.float64)


@pytest.mark.parametrize("K", [32, 256, 2048, 2560, 2592, 8192, 14336])
def test_rmsnorm_against_float64_textbook(K):
    g = np.random.default_rng(K)
    x = g.standard_normal((3, K)).astype(np.float32)
    x[1] *= 1e-3
    x[2, g.choice(K, K // 100 + 1, replace=False)] *= 20  # outliers
    gamma = g.normal(1.0, 0.1, K).astype(np.float32)
    for gm in (gamma, None):
        y = O.rmsnorm(x, gm, 1e-6)
        ref = _rms_f64(x, gm, 1e-6)
        Jp = 1 << max(0, math.ceil(math.log2(max(1, math.ceil(K / 256)))))
        bound = (math.log2(Jp) + 20) * U  # roundings in the sum of squares tree and after it
        assert (np.abs(y - ref) <= bound * np.abs(ref) + 1e-38).all()


def test_rmsnorm_closed_forms():
    K = 2560
    sgn = np.where(np.random.default_rng(5).random(K) < 0.5, -1.0, 1.0).astype(np.float32)
    gamma = np.random.default_rng(6).normal(1.0, 0.1, K).astype(np.float32)
    # |x| == 1: every partial sum of squares is a small integer, so S == K exactly in any order,
    # mean == 1 and r == 1/sqrt(1 + eps) with correctly rounded sqrt and division.
    y = O.rmsnorm(sgn[None, :], gamma, 1e-6)[0]
    r = np.float32(1.0) / np.sqrt(np.float32(1.0) + np.float32(1e-6))
    assert np.array_equal(y, (sgn * r) * gamma)
    assert O.rms_sumsq(sgn) == np.float32(K)
    # zero row: r = 1/sqrt(eps), y = 0
    assert (O.rmsnorm(np.zeros((1, K), np.float32), gamma, 1e-6) == 0).all()
    # a single nonzero element a: S == a*a rounded once, y_k = (a * r) * gamma_k
    x = np.zeros(K, np.float32)
    x[1234] = np.float32(3.0)
    S = O.rms_sumsq(x)
    assert S == np.float32(9.0)
    r = np.float32(1.0) / np.sqrt(np.float32(9.0) / np.float32(K) + np.float32(1e-6))
    y = O.rmsnorm(x[None, :], gamma, 1e-6)[0]
    assert y[1234] == (np.float32(3.0) * r) * gamma[1234] and np.count_nonzero(y) == 1


def test_rms_sumsq_is_exact_for_integer_rows():
    # integers with exact squares summing below 2^24: every order gives the exact sum
    x = np.random.default_rng(8).integers(-60, 61, 8192).astype(np.float32)
    assert O.rms_sumsq(x) == np.float32(np.sum(x.astype(np.int64) ** 2))


# ---- remaining GLU variants and RMS+ADD / RMS+SCALE ------------------------------------------
def _glu_variant_f64(g, u, op, alpha=O.OAI_ALPHA, limit=O.OAI_LIMIT):
    g = g.astype(np.float64)
    u = u.astype(np.float64)
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    if op == "reglu":
        return np.maximum(g, 0.0) * u
    if op == "geglu":
        # 0.5 (1 + tanh z) = expit(2 z): scipy's logistic keeps the far negative tail, where
        # 1 + tanh(z) cancels to zero in float64 (the tanh form itself is checked for |g| < 3)
        z = math.sqrt(2.0 / math.pi) * (g + 0.044715 * g ** 3)
        tanh_form = 0.5 * g * (1.0 + np.tanh(z)) * u
        logistic = g * scipy.special.expit(2.0 * z) * u
        near = np.abs(g) < 3
        assert np.allclose(tanh_form[near], logistic[near], rtol=1e-10, atol=0)
        return logistic
    if op == "geglu_quick":
        return g * sig(float(np.float32(1.702)) * g) * u
    gg = np.minimum(g, limit)
    uu = np.clip(u, -limit, limit)
    if op == "swiglu_oai":
        return gg * sig(float(np.float32(alpha)) * gg) * (uu + 1.0)
    return gg * sig(gg) * uu


@pytest.mark.parametrize("op", ["reglu", "geglu", "geglu_quick", "swiglu_oai", "swiglu_clamp"])
def test_glu_variants_against_float64_textbook(op):
    rng = np.random.default_rng(21)
    K = 4096
    gu = (rng.standard_normal((3, 2 * K)) * np.array([1.0, 3.0, 8.0])[:, None]).astype(np.float32)
    g, u = gu[:, :K], gu[:, K:]
    y = O.glu_ex(g, u, op).astype(np.float64)
    ref = _glu_variant_f64(g, u, op)
    gd = g.astype(np.float64)
    if op == "reglu":
        rel = U  # one rounding: the product
    elif op == "geglu":
        # g^3 and the inner sum (4 roundings), the f32 constant, exp_q (2 ulp) of an argument
        # known to a few ulps of its size, then 1+e, g/den and *u
        arg = np.abs(1.5957691216057308 * (gd + 0.044715 * gd ** 3))
        rel = (12.0 + 6.0 * arg) * U
    else:
        gg = np.minimum(gd, O.OAI_LIMIT) if op.startswith("swiglu") else gd
        c = 1.702 if op in ("geglu_quick", "swiglu_oai") else 1.0
        rel = (12.0 + 3.0 * c * np.abs(gg)) * U
    absf = 1e-36 * np.abs(gd * u.astype(np.float64)) + 1e-36
    assert (np.abs(y - ref) <= rel * np.abs(ref) + absf).all()


def test_glu_variant_closed_forms():
    rng = np.random.default_rng(22)
    K = 512
    g = (rng.standard_normal((2, K)) * 5).astype(np.float32)
    u = (rng.standard_normal((2, K)) * 5).astype(np.float32)
    # ReGLU: gate <= 0 gives a zero, gate > 0 the rounded product
    y = O.glu_ex(g, u, "reglu")
    assert (y[g <= 0] == 0).all() and np.array_equal(y[g > 0], (g * u)[g > 0])
    # the gate clamp: any gate at or above the limit acts as the limit itself
    big = np.full_like(g, 100.0)
    lim = np.full_like(g, np.float32(O.OAI_LIMIT))
    for op in ("swiglu_oai", "swiglu_clamp"):
        assert np.array_equal(O.glu_ex(big, u, op), O.glu_ex(lim, u, op))
        # the up clamp: |u| beyond the limit acts as +-limit
        assert np.array_equal(O.glu_ex(g, u * 1e6, op), O.glu_ex(g, np.sign(u) * lim, op))
    # SwiGLU-OAI at u = -1 multiplies by (u + 1) = 0
    assert (O.glu_ex(g, -np.ones_like(u), "swiglu_oai") == 0).all()
    # limits that never bind reduce the clamped forms to plain SwiGLU (a different code path:
    # the packed-row GLU with the up values as given, or shifted by the exact + 1)
    gu = np.concatenate([g, u], axis=1)
    assert np.array_equal(O.glu_ex(g, u, "swiglu_clamp", limit=3e38), O.glu(gu, "swiglu"))
    gu1 = np.concatenate([g, (u + np.float32(1.0)).astype(np.float32)], axis=1)
    assert np.array_equal(O.glu_ex(g, u, "swiglu_oai", alpha=1.0, limit=3e38), O.glu(gu1, "swiglu"))
    # the two original ops through the general entry
    for op in ("swiglu", "geglu_erf"):
        assert np.array_equal(O.glu_ex(g, u, op), O.glu(gu, op))
    # packed-swapped input (up half first) with independent strides
    ug = np.concatenate([u, g], axis=1)
    assert np.array_equal(O.glu_ex(ug[:, K:], ug[:, :K], "geglu"), O.glu_ex(g, u, "geglu"))


def test_rmsnorm_add_and_scale():
    rng = np.random.default_rng(23)
    K = 2048
    x = rng.standard_normal((3, K)).astype(np.float32)
    gamma = rng.normal(1.0, 0.1, K).astype(np.float32)
    beta = rng.normal(0.0, 0.5, K).astype(np.float32)
    base = O.rmsnorm(x, gamma, 1e-6)
    # beta = -0 and scale = 1 leave every value (signed zeros included) unchanged
    assert np.array_equal(O.rmsnorm_ex(x, gamma, np.full(K, -0.0, np.float32), 1.0, 1e-6).view(np.uint32),
                          base.view(np.uint32))
    assert np.array_equal(O.rmsnorm_ex(x, None, None, 1.0, 1e-6), O.rmsnorm(x, None, 1e-6))
    # a power-of-two scale is exact
    assert np.array_equal(O.rmsnorm_ex(x, None, None, 0.25, 1e-6), O.rmsnorm(x, None, 1e-6) * np.float32(0.25))
    # against float64: (x r gamma + beta) * c
    c = 0.7
    y = O.rmsnorm_ex(x, gamma, beta, c, 1e-6).astype(np.float64)
    t = _rms_f64(x, gamma, 1e-6)
    ref = (t + beta.astype(np.float64)) * float(np.float32(c))
    bound = 26 * U * (np.abs(t) + np.abs(beta)) * abs(c)
    assert (np.abs(y - ref) <= bound + 1e-38).all()
