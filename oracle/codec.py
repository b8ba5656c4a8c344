"""Quantize / dequantize, written from the definitions.

2-bit format (the hq-e8-2b byte budget of "KV at 9 KB a token", section "How
it works": 64 B of 2-bit code plus an 8-byte metadata row per head per token).
The pages size the row but do not give its codebook; this library uses
uniform asymmetric codes per (token, head) row, in emulated fp32:
    mn = min x, mx = max x                         (exact; a zero is taken as +0)
    scale = fl32(fl32(mx - mn) / 3);  scale == 0 -> 1.0
    c_i = clamp(rint(fl32(fl32(x_i - mn) / scale)), 0, 3)   (rint = nearest even)
    dequantized x_i = fl32(c_i * scale + mn)       (one rounding, as fmaf)
Per-token scaling of K as well as V follows the page "Half the Cache, Twice the
Context" (section "What the cache loses when you round it", reading 1): at 2
bits per-token scaling beats per-channel for K too.
Pins: closed-form invariants (0 <= c <= 3, |x - x^| <= scale/2 up to rounding,
rows on the grid round-trip exactly, round-half-even ties, a constant row gives
scale 1.0 and codes 0) in tests/test_oracle_codec.py.

Symmetric absmax quantizer (the page "Half the Cache, Twice the Context",
section "What the cache loses when you round it", Block 2): qmax = 2^(b-1)-1,
scale = max|x| / qmax along an axis, a zero scale becomes 1.0, codes =
clip(round(x / scale), -qmax, qmax).  Run in fp64 it must reproduce that
section's printed reconstruction and needle tables exactly
(tests/golden/block2_*.txt); run in fp32 with b = 8 it is the 8-bit variant's
codec: K scaled per channel over the tokens of a 64-token page, V per token.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

F32 = np.float32


def _check_finite(x):
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input to the quantizer (undefined for these formats)")


# ---------------------------------------------------------------- 2-bit ----

def q2_quantize(x):
    """Rows x[..., D] (fp32 values) -> (codes uint8[..., D], scale f32[...], mn f32[...])."""
    x = np.asarray(x, dtype=F32)
    _check_finite(x)
    mn = np.add(x.min(axis=-1), F32(0), dtype=F32)   # a zero min or max is taken as +0
    mx = np.add(x.max(axis=-1), F32(0), dtype=F32)
    span = np.subtract(mx, mn, dtype=F32)
    scale = np.divide(span, F32(3), dtype=F32)
    scale = np.where(scale == F32(0), F32(1), scale).astype(F32)
    y = np.subtract(x, mn[..., None], dtype=F32)
    t = np.divide(y, scale[..., None], dtype=F32)
    c = np.clip(np.rint(t), 0, 3).astype(np.uint8)
    return c, scale, mn


def hadamard_rows(x):
    """Unnormalised Walsh-Hadamard transform of rows x[..., D] (D a power of
    two) in emulated fp32: stages h = 1, 2, 4, .., D/2, each replacing the pair
    (x_i, x_{i+h}) (i with bit h clear) by (x_i + x_{i+h}, x_i - x_{i+h}), one
    rounding per operation.  The result is H x with H the Sylvester-ordered
    Hadamard matrix (entries +-1, H H = D I), up to the fp32 roundings of the
    butterflies, which every implementation that takes the same stages in the
    same order reproduces bit for bit.  The rotated 2-bit variant quantizes
    H k instead of k ("Half the Cache, Twice the Context", closing notes: the
    axis and rotation choices matter at 2 bits)."""
    y = np.array(x, dtype=F32, copy=True)
    D = y.shape[-1]
    assert D & (D - 1) == 0
    lead = y.shape[:-1]
    h = 1
    while h < D:
        v = y.reshape(*lead, D // (2 * h), 2, h)
        a, b = v[..., 0, :], v[..., 1, :]
        y = np.stack([np.add(a, b, dtype=F32), np.subtract(a, b, dtype=F32)], axis=-2).reshape(*lead, D)
        h *= 2
    return y


def unrotate_rows(xr):
    """Back to the original basis, in fp64: x = H x_r / D (H symmetric, H H = D I)."""
    xr = np.asarray(xr, dtype=np.float64)
    D = xr.shape[-1]
    y = xr.copy()
    lead = y.shape[:-1]
    h = 1
    while h < D:
        v = y.reshape(*lead, D // (2 * h), 2, h)
        a, b = v[..., 0, :], v[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(*lead, D)
        h *= 2
    return y / D


def _fma_f32(a64, b64, c64):
    """fl32(a*b + c) with a single rounding, for a*b exact in fp64.

    The fp64 sum is checked to be exact with TwoSum; any element whose sum is
    not exact in fp64 is recomputed in rational arithmetic.
    """
    p = a64 * b64
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    out = s.astype(F32)
    bad = np.nonzero(err != 0)
    if bad[0].size:
        flat_idx = list(zip(*bad))
        for idx in flat_idx:
            exact = Fraction(float(a64[idx])) * Fraction(float(b64[idx])) + Fraction(float(c64[idx]))
            out[idx] = _fraction_to_f32(exact)
    return out


def _fraction_to_f32(q: Fraction) -> F32:
    # nearest-even rounding of an exact rational to fp32 via two candidates
    f = F32(float(q))  # float(q) rounds correctly to fp64; refine at fp32 level
    lo, hi = np.nextafter(f, F32(-np.inf)), np.nextafter(f, F32(np.inf))
    best = min((lo, f, hi), key=lambda v: (abs(Fraction(float(v)) - q), int(np.asarray(v).view(np.uint32)) & 1))
    return F32(best)


def q2_dequantize(codes, scale, mn):
    """x^ = fl32(c * scale + mn), one rounding (what fmaf computes)."""
    c64 = np.asarray(codes, dtype=np.float64)
    s64 = np.asarray(scale, dtype=F32).astype(np.float64)[..., None]
    m64 = np.asarray(mn, dtype=F32).astype(np.float64)[..., None]
    s64, m64 = np.broadcast_to(s64, c64.shape), np.broadcast_to(m64, c64.shape)
    return _fma_f32(c64, s64, m64)


# ------------------------------------------------------------ symmetric ----

def sym_quantize(x, bits: int, axis, dtype=np.float64):
    """Symmetric absmax quantizer -> (integer codes as dtype, scale as dtype, keepdims)."""
    x = np.asarray(x, dtype=dtype)
    _check_finite(x)
    qmax = dtype(2 ** (bits - 1) - 1)
    amax = np.abs(x).max(axis=axis, keepdims=True)
    scale = np.divide(amax, qmax, dtype=dtype)
    scale = np.where(scale == 0, dtype(1), scale).astype(dtype)
    t = np.divide(x, scale, dtype=dtype)
    c = np.clip(np.rint(t), -qmax, qmax).astype(dtype)
    return c, scale


def sym_dequantize(codes, scale, dtype=np.float64):
    return np.multiply(np.asarray(codes, dtype=dtype), np.asarray(scale, dtype=dtype), dtype=dtype)


def sym_roundtrip(x, bits: int, axis, dtype=np.float64):
    c, s = sym_quantize(x, bits, axis, dtype)
    return sym_dequantize(c, s, dtype)


# ---------------------------------------------------------------- 8-bit ----

def q8_quantize_v(v):
    """V rows [..., D] fp32 -> (int8 codes [..., D], fp32 scale [...]) per token."""
    c, s = sym_quantize(v, 8, axis=-1, dtype=F32)
    return c.astype(np.int8), s[..., 0]


def q8_quantize_k_page(k):
    """K rows [n, ..., D] of one page (n <= 64 exact rows present) -> per-channel codes/scales.

    Returns (int8 codes [n, ..., D], fp32 scales [..., D]); the scale of
    channel d is max over the page's present tokens of |k[:, ..., d]| / 127.
    """
    c, s = sym_quantize(k, 8, axis=0, dtype=F32)
    return c.astype(np.int8), s[0]


def q8_dequantize(codes, scale):
    """fl32(c * s): a single fp32 product."""
    return np.multiply(np.asarray(codes, dtype=F32), np.asarray(scale, dtype=F32), dtype=F32)
