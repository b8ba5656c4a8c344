"""The 8-bit decode's radix-128 digit scheme, emulated on the CPU.

The int8 matrix-core form of the 8-bit decode feeds the scaled query rows and
the softmax weights to v_mfma_i32_16x16x64_i8 as three balanced radix-128
digits each.  For a row whose largest magnitude lies in [2^k, 2^(k+1)) it
takes e = k - 5 and forms x 2^(14 - e) + (2^23 + 3,153,984) in one fused
multiply-add rounded to nearest even; the low 23 mantissa bits then hold
n + 3,153,984 with n = rint(x 2^(14 - e)), and

    n = 16384 d0 + 128 d1 + d2,  d0 = bits[14..22] - 192,
                                  d1 = bits[7..13] - 64,  d2 = bits[0..6] - 64.

This file checks that scheme with numpy's fp32 arithmetic (the fused
multiply-add as an exact fp64 sum rounded once to fp32): every n is recovered
exactly, the digits fit int8 (|d0| <= 127, d1 and d2 in -64..63), the value
is kept to 2^-20 of its row's largest magnitude, and the byte packing of four
digits into a word (two v_perm_b32 selections) puts digit i in byte i."""

import numpy as np

BIAS = np.float32(11542592.0)  # 2^23 + 64 (1 + 128 + 128^2) + 128^3


def digit_exp(amax: float) -> int:
    if amax <= 0:
        return 0
    k = int((np.float32(amax).view(np.uint32) >> 23) & 0xFF) - 127
    return max(k - 5, -112)


def digits(x: np.ndarray):
    x = np.asarray(x, np.float32)
    e = digit_exp(float(np.abs(x).max()))
    mul = np.float32(2.0 ** (14 - e))
    y = (x.astype(np.float64) * float(mul) + float(BIAS)).astype(np.float32)  # fma, one rounding
    u = y.view(np.uint32).astype(np.int64)
    d0 = ((u >> 14) & 511) - 192
    d1 = ((u >> 7) & 127) - 64
    d2 = (u & 127) - 64
    return e, mul, y, d0, d1, d2


def test_digits_recover_the_rounded_integer_and_fit_int8():
    rng = np.random.default_rng(20261203)
    for trial in range(600):
        scale = 10.0 ** rng.uniform(-30, 30)
        x = (rng.standard_normal(128) * scale).astype(np.float32)
        if trial % 5 == 0:
            x[rng.integers(128)] *= 50  # an outlier sets the row's exponent
        if trial % 7 == 0:
            x[: rng.integers(1, 64)] = 0.0
        e, mul, y, d0, d1, d2 = digits(x)
        assert np.all(y >= 2.0 ** 23) and np.all(y < 2.0 ** 24)
        n = 16384 * d0 + 128 * d1 + d2
        assert np.array_equal(n, np.rint(x.astype(np.float64) * float(mul)).astype(np.int64))
        assert d0.min() >= -127 and d0.max() <= 127
        assert d1.min() >= -64 and d1.max() <= 63 and d2.min() >= -64 and d2.max() <= 63
        amax = float(np.abs(x).max())
        err = np.abs(n * 2.0 ** (e - 14) - x.astype(np.float64)).max()
        assert err <= 2.0 ** -20 * amax


def test_zero_row_and_weights_of_zero():
    e, _, _, d0, d1, d2 = digits(np.zeros(64, np.float32))
    assert e == 0 and not d0.any() and not d1.any() and not d2.any()
    # a weight of zero (masked token) next to live weights gives three zero digits
    w = np.array([0.0, 1.0, 0.25, 3e-5], np.float32)
    _, _, _, d0, d1, d2 = digits(w)
    assert d0[0] == 0 and d1[0] == 0 and d2[0] == 0


def test_three_digits_are_exact_for_small_integers():
    # integers of a row whose largest element is 100: x 2^(14 - e) is exact
    x = np.array([100, -100, 37, -1, 0, 64, -64], np.float32)
    e, mul, _, d0, d1, d2 = digits(x)
    assert e == 1 and float(mul) == 2.0 ** 13
    assert np.array_equal((16384 * d0 + 128 * d1 + d2) * 2.0 ** (e - 14), x.astype(np.float64))


def _perm(s0: int, s1: int, sel: int) -> int:
    """v_perm_b32: byte i of the result is byte sel_i of {s0, s1} (s1 = bytes 0-3), 0x0c selects 0."""
    v = ((s0 & 0xFFFFFFFF) << 32) | (s1 & 0xFFFFFFFF)
    r = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        r |= (0 if b == 0x0C else (v >> (8 * b)) & 0xFF) << (8 * i)
    return r


def test_four_digits_pack_into_bytes_in_order():
    for a, b, c, d in [(1, -1, 127, -127), (-64, 63, 0, 5), (0, 0, 0, -1)]:
        lo = _perm(b & 0xFFFFFFFF, a & 0xFFFFFFFF, 0x0C0C0400)
        hi = _perm(d & 0xFFFFFFFF, c & 0xFFFFFFFF, 0x04000C0C)
        word = lo | hi
        got = [int(np.uint8((word >> (8 * i)) & 0xFF).astype(np.int8)) for i in range(4)]
        assert got == [a, b, c, d]
