"""Pins of the oracle's Q8_1 quantizer (CPU only): closed-form blocks, the golden tie block,
library conversions and invariants that any correct reading of the block rule must satisfy."""
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _quant_block(vals):
    """Quantize one 32-value row; return (codes int8[32], d16, s16, raw image bytes)."""
    y = np.zeros((1, 32), np.float32)
    y[0, : len(vals)] = vals
    img = O.quantize(y)
    codes, d16, s16 = O.image_planes(img, 1, 32)
    return codes[0, 0], int(d16[0, 0]), int(s16[0, 0]), img


def _read_golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = v.split()
    return out


def test_golden_tie_block():
    g = _read_golden("q8_1_tie_block.txt")
    vals = np.array([float(v) for v in g["input"]], np.float32)
    codes, d16, s16, _ = _quant_block(vals)
    assert codes.tolist() == [int(v) for v in g["codes"]]
    assert d16 == int(g["d16"][0], 16)
    assert s16 == int(g["s16"][0], 16)


def test_zero_block_and_padding_are_zero_bytes():
    _, _, _, img = _quant_block([])
    assert not img.any()
    # K = 2592: 81 blocks, RB = 96; blocks 81..95 are padding and must be zero
    K = 2592
    y = np.random.default_rng(0).standard_normal((2, K)).astype(np.float32)
    img = O.quantize(y)
    codes, d16, s16 = O.image_planes(img, 2, K)
    assert O.row_blocks(K) == 96
    assert not codes[:, 81:].any() and not d16[:, 81:].any() and not s16[:, 81:].any()
    assert (np.abs(codes[:, :81]).max(axis=2) == 127).all()


def test_single_value_blocks():
    codes, d16, s16, _ = _quant_block([127.0])
    assert codes[0] == 127 and not codes[1:].any()
    assert d16 == 0x3C00 and s16 == 0x57F0  # d = 1.0, s = 127.0
    codes, d16, s16, _ = _quant_block([-3.5])
    # d = 3.5/127, 1/d, -3.5 * (1/d) rounds to -127
    assert codes[0] == -127 and d16 == O.f32_to_f16_bits(np.float32(3.5) / np.float32(127))[()]
    assert s16 == O.f32_to_f16_bits(np.float32(-127.0) * (np.float32(3.5) / np.float32(127)))[()]


def test_scaled_integer_blocks_give_their_integers():
    # y = m * 2^-3 with max |m| = 127: d = 2^-3 exactly, 1/d = 8, codes = m exactly
    g = np.random.default_rng(1)
    for _ in range(50):
        m = g.integers(-127, 128, 32)
        m[g.integers(32)] = 127 if g.random() < 0.5 else -127
        codes, d16, s16, _ = _quant_block(m.astype(np.float32) / 8)
        assert np.array_equal(codes.astype(int), m)
        assert d16 == 0x3000  # 0.125
        assert s16 == np.float16(np.float32(m.sum()) * np.float32(0.125)).view(np.uint16)


def test_block_invariants_on_random_rows():
    g = np.random.default_rng(2)
    K = 2560
    y = (g.standard_normal((6, K)) * np.array([1, 1e-3, 1e3, 20, 1e-30, 5])[:, None]).astype(np.float32)
    y[3, g.choice(K, 30, replace=False)] *= 20
    img = O.quantize(y)
    codes, d16, s16 = O.image_planes(img, 6, K)
    Kb = K // 32
    yb = y.reshape(6, Kb, 32).astype(np.float64)
    c = codes[:, :Kb].astype(np.int64)
    amax = np.abs(yb).max(axis=2)
    assert (np.abs(c) <= 127).all()
    assert (np.abs(c).max(axis=2) == 127).all()  # every nonzero block reaches 127
    assert ((c == 0) | (np.sign(c) == np.sign(yb))).all()
    d64 = amax / 127.0
    assert (np.abs(yb / d64[..., None] - c) <= 0.5 + 1e-5).all()
    # scale and sum against numpy's IEEE binary16 conversion of the f32 values
    d32 = (amax.astype(np.float32) / np.float32(127))
    assert np.array_equal(d16[:, :Kb], d32.astype(np.float16).view(np.uint16))
    s32 = c.sum(axis=2).astype(np.float32) * d32
    assert np.array_equal(s16[:, :Kb], s32.astype(np.float16).view(np.uint16))
    # purity: quantizing the same input again gives identical bytes
    assert np.array_equal(img, O.quantize(y.copy()))


def test_subnormal_scale_block_is_zero_block():
    # amax so small that 1/d overflows: the block is written as zeros
    codes, d16, s16, img = _quant_block([1e-38, -2e-39])
    assert not img.any()


def test_quantizer_rejects_nonfinite_live_values():
    y = np.zeros((1, 32), np.float32)
    y[0, 3] = np.nan
    with pytest.raises(ValueError):
        O.quantize(y)
