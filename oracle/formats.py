"""Element and scale formats of NVFP4, written from their definitions.

Test infrastructure only (see the package docstring).

* E2M1 (the NVFP4 element): sign bit, 2 exponent bits, 1 mantissa bit
  (neurohive.io LongLive-2.0 summary, NVFP4 paragraph).  Exponent bias 1, no
  infinities or NaNs; exponent field 0 is subnormal (0.5 * m).
* E4M3FN (the FP8 block scale; the pages say only "FP8",
  tailorednewshub.com "Entrenamiento NVFP4" — E4M3 is the reading): sign bit,
  4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
  (m * 2^-9); no infinities; 0x7F / 0xFF are NaN, so the largest finite value
  is 0x7E = 448.

Conversions round to nearest, ties to the even code, and saturate to the
largest finite magnitude (reading: the pages do not state the rounding).
They are implemented as "nearest point of the finite set" searches in exact
float64 arithmetic, which is the plainest definition of RNE-satfinite.
"""

from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0
# Largest magnitude a quantized element can carry relative to its tensor scale:
# E2M1 max times E4M3 max.
GLOBAL_MAX = E2M1_MAX * E4M3_MAX  # 2688.0


def e2m1_value(code) -> np.ndarray:
    """Value of 4-bit E2M1 codes (float64), from the 2+1-bit closed form."""
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


E2M1_MAGNITUDES = e2m1_value(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6


def e4m3_value(byte) -> np.ndarray:
    """Value of E4M3FN bytes (float64); NaN for 0x7F and 0xFF."""
    byte = np.asarray(byte, dtype=np.int64)
    s = (byte >> 7) & 1
    e = (byte >> 3) & 15
    m = byte & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((byte & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


_E4M3_POS = e4m3_value(np.arange(0x7F))  # codes 0x00..0x7E, increasing


def _nearest_even(mags: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point to each |value|, ties to the even index,
    saturating at the last grid point.  ``grid`` is increasing and its index
    parity equals the mantissa parity of the code (true for E2M1 and E4M3)."""
    v = np.asarray(mags, dtype=np.float64)
    n = grid.size
    hi = np.clip(np.searchsorted(grid, v, side="left"), 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    d_lo = v - grid[lo]          # exact: float32 input vs short dyadic grid
    d_hi = grid[hi] - v
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(take_hi, hi, lo)
    idx = np.where(v >= grid[-1], n - 1, idx)
    return idx.astype(np.uint8)


def f32_to_e4m3(u) -> np.ndarray:
    """E4M3FN byte of non-negative float32 values, RNE, saturating at 448.

    Used only for block scales, which are non-negative by construction."""
    u = np.asarray(u, dtype=np.float32)
    if np.any(u < 0) or np.any(np.isnan(u)):
        raise ValueError("block scale input must be non-negative and finite")
    return _nearest_even(u, _E4M3_POS)


def f32_to_e2m1(y) -> np.ndarray:
    """4-bit E2M1 code of float32 values: sign bit taken from the input's sign
    bit (so values rounding to zero keep their sign: -0.1 -> 0x8), magnitude by
    RNE onto {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6."""
    y = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y).astype(np.uint8) << 3
    return sign | _nearest_even(np.abs(y), E2M1_MAGNITUDES)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of finite float32 values, round to nearest even.

    bf16 keeps the top 16 bits of the float32 pattern; the discarded low half
    is compared with the halfway point 0x8000, ties going to an even result."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    low = b & 0xFFFF
    keep = b >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.uint32)).astype(np.uint16)
