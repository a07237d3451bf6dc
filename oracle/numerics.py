"""Rounding helpers of the oracle (numpy only)."""

import numpy as np


def f32(x):
    """Round to IEEE binary32, nearest-even (numpy's float64->float32 cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x) -> np.ndarray:
    """Round fp32 values to bfloat16, nearest-even, returned as float32.

    bfloat16 keeps the top 16 bits of the binary32 pattern.  Rounding to
    nearest-even adds 0x7FFF plus the lowest kept bit before truncating, which
    rounds up exactly when the dropped half-word exceeds 0x8000, or equals it
    with the kept LSB odd.  NaN is passed through unchanged.
    """
    a = np.asarray(x, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + keep_lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(np.float32)
    return np.where(np.isnan(a), a, out).astype(np.float32)
