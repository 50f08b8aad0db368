"""Number formats the method stores data in, written from their definitions.

* E4M3 (FN variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
  subnormals m/8 * 2^-6; exponent field 15 with mantissa 7 is NaN; there are no infinities, so the
  largest finite magnitude is 1.75 * 2^8 = 448. [TR] §3.6 fixes a single E4M3 format (4-bit exponent,
  3-bit mantissa) for every FP8 GEMM operand; the FN encoding is the one gfx950 computes in natively.
* Rounding is to nearest, ties to even, with saturation to +-448 (the pages say nothing about rounding
  or overflow; this is the plainest reading, recorded with the other readings).
* fl32: rounding of a float64 value to IEEE binary32 (numpy's cast rounds to nearest even).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9


def fl32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def e4m3_decode(codes) -> np.ndarray:
    """Value (float64) of each E4M3FN byte; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    v = np.where(e == 0, sub, nrm) * sign
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_round(x) -> np.ndarray:
    """Round each value (exact in float64) to the nearest E4M3FN value, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum of the binade of a: 2^(floor(log2 a) - 3) for normals, 2^-9 below the smallest normal
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex with f in [0.5, 1)
    q = np.where(a < E4M3_MIN_NORMAL, E4M3_SUBNORMAL_QUANTUM, np.ldexp(1.0, ex - 1 - 3))
    r = np.rint(a / q) * q                              # a / q is exact; rint is ties-to-even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN byte of each value after ``e4m3_round``."""
    v = e4m3_round(x)
    a = np.abs(v)
    s = np.signbit(v).astype(np.int64) << 7
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    unb = ex - 1                                        # a = 1.m * 2^unb for normals
    is_sub = a < E4M3_MIN_NORMAL
    m_sub = np.rint(a / E4M3_SUBNORMAL_QUANTUM).astype(np.int64)
    m_nrm = np.rint((a / np.ldexp(1.0, unb) - 1.0) * 8.0).astype(np.int64)
    e_nrm = unb + 7
    code = np.where(is_sub, m_sub, (e_nrm << 3) | m_nrm)
    return (code | s).astype(np.uint8)
