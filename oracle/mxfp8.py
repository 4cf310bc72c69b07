"""MXFP8 quantiser (oracle; test infrastructure only).

The pages name the format and the op only: MoK has an MXFP8 precision mode
([MTP] paragraph after the design decisions) and weights are pre-quantised
with ``ops.mxfp8_quantize`` ([CARD] "Core concepts", "Limitations").  The
recipe below is the OCP Microscaling (MX) v1.0 definition with E4M3 elements,
as this code reads it:

* a block is 32 consecutive values along the contraction (K) axis;
* the shared scale is an E8M0 code s (value 2^(s-127));
  shared_exp = floor(log2(amax)) - 8, where 8 is E4M3's largest normal
  exponent, clamped to [-127, 127]; s = shared_exp + 127.  A block whose amax
  is 0 gets s = 0;
* each element v becomes the E4M3 (the "FN" variant: bias 7, no infinities,
  0x7F/0xFF are NaN, largest finite 448, subnormal step 2^-9) code nearest to
  v / 2^shared_exp, ties to the even code, saturating at +-448.  The sign is
  kept, so a negative value that rounds to zero is 0x80.

Every step here is exact: bf16 inputs divided by a power of two are exact in
fp64, and the rounding is done on exact fp64 values.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0, exactly (from the binary exponent); 0 for a == 0."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))   # a = m * 2^e, 0.5 <= m < 1
    return np.where(np.asarray(a) > 0, e - 1, 0).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3-FN codes (uint8) -> fp64 values (NaN codes -> nan)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(ex == 0, man * 2.0 ** -9,
                   (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7.0))
    mag = np.where((ex == 0xF) & (man == 0x7), np.nan, mag)
    return s * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp64 values -> E4M3-FN codes: nearest, ties to even, saturating at 448.
    The sign bit of the input is kept."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    ex = np.clip(_floor_log2(a), -6, 8)                  # binade, subnormals share -6
    step = np.exp2(ex - 3)                               # 3 mantissa bits
    q = np.rint(a / step) * step                         # exact value after RNE
    q = np.where(a > 0, q, 0.0)
    # encode q exactly
    qe = np.clip(_floor_log2(q), -6, 8)
    normal = q >= 2.0 ** -6
    man_n = np.rint(q / np.exp2(qe - 3)) - 8             # 0..7
    code_n = ((qe + 7).astype(np.int64) << 3) | man_n.astype(np.int64)
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)     # 0..7
    code = np.where(normal, code_n, code_s)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def block_scale_codes(v: np.ndarray) -> np.ndarray:
    """Shared E8M0 scale code of each 32-block along the last axis."""
    v = np.asarray(v, dtype=np.float64)
    *lead, K = v.shape
    assert K % BLOCK == 0
    amax = np.abs(v.reshape(*lead, K // BLOCK, BLOCK)).max(axis=-1)
    se = _floor_log2(amax) - E4M3_EMAX
    se = np.clip(se, -127, 127)
    return np.where(amax > 0, se + 127, 0).astype(np.uint8)


def quantize_with_scales(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Element codes of v [..., K] at the given block scale codes s [..., K/32]."""
    v = np.asarray(v, dtype=np.float64)
    *lead, K = v.shape
    se = np.asarray(s).astype(np.float64) - 127.0
    scaled = v.reshape(*lead, K // BLOCK, BLOCK) / np.exp2(se)[..., None]
    return e4m3_encode(scaled).reshape(*lead, K)


def quantize(v: np.ndarray):
    """v [..., K] (bf16 values as fp64/fp32) -> (codes [..., K] uint8,
    scales [..., K/32] uint8), blocks of 32 along the last axis."""
    s = block_scale_codes(v)
    return quantize_with_scales(v, s), s


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse map: value = e4m3(code) * 2^(s - 127), per 32-block."""
    c = np.asarray(codes)
    *lead, K = c.shape
    val = e4m3_decode(c).reshape(*lead, K // BLOCK, BLOCK)
    return (val * np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)[..., None]).reshape(*lead, K)
