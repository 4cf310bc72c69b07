"""bf16 codec for the oracle (test infrastructure only).

bf16 is IEEE-754 binary32 truncated to its top 16 bits: 1 sign bit, 8 exponent
bits (bias 127), 7 stored mantissa bits.  Rounding from a wider value is
round-to-nearest, ties-to-even, on the 8-bit significand; below 2^-126 the
spacing stays 2^-133 (gradual underflow).
"""
from __future__ import annotations

import numpy as np


def decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_rne(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as
    fp64.  Finite inputs below bf16's overflow threshold only."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # bf16 normals start at 2^-126
    step = np.ldexp(1.0, e - 8)             # 8 significant bits
    r = np.rint(x / step) * step            # np.rint: half to even
    return np.where(x == 0, x, r)


def encode(x: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16) under round_rne."""
    r = round_rne(x).astype(np.float32)     # exact: r is a bf16 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)
