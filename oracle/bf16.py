"""bf16 helpers for the oracle.

Rounding fp32 to bf16 to nearest even is done on the bit pattern: add 0x7FFF
plus the lowest bit that survives, then drop the low 16 bits.  This is the
rounding the page "Half the Cache, Twice the Context" uses in its accumulator
model (section "The cliff is in the accumulator, not the storage", Block 3);
its printed bf16 column pins this helper (tests/golden/block3_flat_sum.txt).
Inputs are assumed finite (the oracle never rounds a NaN).
"""

import numpy as np


def round_f32_to_bf16(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even); returns fp32 values on the bf16 grid."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def bits_to_f32(u16) -> np.ndarray:
    """bf16 bit patterns (uint16) to the fp32 values they denote (exact)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bits(x) -> np.ndarray:
    """bf16 bit patterns of fp32 values that already lie on the bf16 grid."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not a bf16 number"
    return (u >> 16).astype(np.uint16)
