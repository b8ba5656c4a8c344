"""Oracle pins: the 2-bit and 8-bit codecs against closed forms and special cases."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codec

F32 = np.float32


def _bf16_rows(rng, shape, scale=1.0):
    x = (rng.normal(0, scale, shape)).astype(F32)
    return (x.view(np.uint32) & 0xFFFF0000).view(F32)  # on the bf16 grid


def check_q2_invariants(quantize, dequantize, x):
    """Properties any correct uniform 4-level min/scale quantizer has; returns a list of failures."""
    c, s, m = quantize(x)
    xh = dequantize(c, s, m)
    bad = []
    if c.min() < 0 or c.max() > 3:
        bad.append("code range")
    if not np.array_equal(m, x.min(axis=-1)):
        bad.append("min")
    slack = 4 * np.spacing(np.abs(x).max(axis=-1, keepdims=True).astype(F32))
    err = np.abs(x.astype(np.float64) - xh)
    if np.any(err > s[..., None] * 0.5 * (1 + 1e-6) + slack):
        bad.append("error above scale/2")
    # nearest level: no other level of the row's grid is strictly closer (beyond rounding)
    levels = m[..., None, None].astype(np.float64) + np.arange(4) * s[..., None, None].astype(np.float64)
    best = np.abs(x[..., None].astype(np.float64) - levels).min(axis=-1)
    if np.any(err > best + slack):
        bad.append("not the nearest level")
    # the span is split into exactly three steps
    span = (x.max(axis=-1) - x.min(axis=-1)).astype(np.float64)
    nz = span > 0
    if np.any(np.abs(s[nz] * 3 - span[nz]) > 4 * np.spacing(span[nz].astype(F32))):
        bad.append("scale is not span/3")
    return bad


def test_q2_invariants_random_rows():
    rng = np.random.default_rng(11)
    x = _bf16_rows(rng, (4096, 256))
    x[:, ::16] *= 4
    assert check_q2_invariants(codec.q2_quantize, codec.q2_dequantize, x) == []


def test_q2_invariants_catch_planted_mistakes():
    rng = np.random.default_rng(12)
    x = _bf16_rows(rng, (512, 256))

    def floor_codes(x):
        c, s, m = codec.q2_quantize(x)
        t = np.divide(np.subtract(x, m[..., None], dtype=F32), s[..., None], dtype=F32)
        return np.clip(np.floor(t), 0, 3).astype(np.uint8), s, m

    def quarter_scale(x):
        mn = x.min(-1)
        s = ((x.max(-1) - mn) / F32(4)).astype(F32)
        t = ((x - mn[..., None]) / s[..., None]).astype(F32)
        return np.clip(np.rint(t), 0, 3).astype(np.uint8), s, mn

    def swapped_meta(x):
        c, s, m = codec.q2_quantize(x)
        return c, m, s

    for broken in (floor_codes, quarter_scale, swapped_meta):
        assert check_q2_invariants(broken, codec.q2_dequantize, x), broken.__name__


def test_q2_grid_rows_roundtrip_exactly():
    rng = np.random.default_rng(13)
    k = rng.integers(0, 4, (200, 256))
    k[:, 0], k[:, 1] = 0, 3
    mn = F32(-1.25)
    step = F32(0.5)
    x = (mn + k * step).astype(F32)
    c, s, m = codec.q2_quantize(x)
    assert np.all(s == step) and np.all(m == mn)
    assert np.array_equal(c, k)
    assert np.array_equal(codec.q2_dequantize(c, s, m), x)


def test_q2_half_steps_round_to_even():
    row = np.array([0, 0.5, 1.5, 2.5, 3] + [0] * 251, F32)
    c, s, m = codec.q2_quantize(row[None])
    assert s[0] == 1.0 and m[0] == 0.0
    assert list(c[0, :5]) == [0, 0, 2, 2, 3]


def test_q2_constant_row():
    x = np.full((3, 256), 0.375, F32)
    c, s, m = codec.q2_quantize(x)
    assert np.all(s == 1.0) and np.all(c == 0) and np.all(m == F32(0.375))
    assert np.all(codec.q2_dequantize(c, s, m) == F32(0.375))


def test_q2_rejects_non_finite():
    x = np.zeros((1, 256), F32)
    x[0, 5] = np.inf
    with pytest.raises(ValueError):
        codec.q2_quantize(x)


def test_q2_dequantize_is_one_rounding():
    rng = np.random.default_rng(14)
    c = rng.integers(0, 4, (64, 256)).astype(np.uint8)
    s = rng.uniform(0.01, 5, 64).astype(F32)
    m = rng.uniform(-10, 0, 64).astype(F32)
    got = codec.q2_dequantize(c, s, m)
    for i in range(0, 64, 7):
        for j in range(0, 256, 13):
            exact = Fraction(int(c[i, j])) * Fraction(float(s[i])) + Fraction(float(m[i]))
            assert got[i, j] == codec._fraction_to_f32(exact)


def test_q8_invariants():
    rng = np.random.default_rng(15)
    v = _bf16_rows(rng, (512, 128))
    v[::64] *= 6
    c, s = codec.q8_quantize_v(v)
    vh = codec.q8_dequantize(c, s[:, None])
    assert c.dtype == np.int8 and c.min() >= -127
    assert np.all(np.abs(v - vh) <= s[:, None] * 0.5 * (1 + 1e-6) + np.spacing(np.abs(v)))
    # the largest-magnitude element of each row gets code +-127
    idx = np.abs(v).argmax(axis=1)
    assert np.all(np.abs(c[np.arange(512), idx]) == 127)


def test_q8_page_per_channel_single_token_and_zero_channel():
    rng = np.random.default_rng(16)
    k = _bf16_rows(rng, (1, 2, 128))
    k[0, 0, 7] = 0
    c, s = codec.q8_quantize_k_page(k)
    assert s.shape == (2, 128)
    nz = k[0] != 0
    assert np.all(np.abs(c[0][nz]) == 127)
    assert c[0, 0, 7] == 0 and s[0, 7] == 1.0


def test_q8_page_scale_is_channel_absmax_over_present_tokens():
    rng = np.random.default_rng(17)
    k = _bf16_rows(rng, (40, 3, 128))
    c, s = codec.q8_quantize_k_page(k)
    amax = np.abs(k).max(axis=0)
    assert np.array_equal(s, np.divide(amax, F32(127), dtype=F32))
    assert np.all(np.abs(codec.q8_dequantize(c, s[None]) - k) <= s[None] * 0.5 * (1 + 1e-6) + np.spacing(np.abs(k)))
