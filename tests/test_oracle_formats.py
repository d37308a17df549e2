"""Pins for the oracle's element/scale formats (CPU only).

The oracle is checked against things other than itself: the E2M1 grid the
format definition fixes, torch's own float8_e4m3fn and bfloat16 casts
(library routines), and exact rational nearest-even rounding written
independently with ``fractions.Fraction``.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_grid_from_closed_form():
    # The E2M1 magnitudes the NVFP4 element can take: 2 exponent bits, 1 mantissa bit.
    assert list(F.e2m1_value(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.e2m1_value(np.arange(8, 16))) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert np.signbit(F.e2m1_value(8))


def test_e4m3_table_matches_torch():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = F.e4m3_value(np.arange(256))
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(lib[~nan], ours[~nan])
    assert F.e4m3_value(0x7E) == 448.0 and F.e4m3_value(0x01) == 2.0 ** -9
    assert F.e4m3_value(0x38) == 1.0 and F.e4m3_value(0x48) == 4.0


def _frac_nearest_even(v: Fraction, grid):
    """Independent RNE onto a finite grid: exact rational distances, ties to
    the even index, saturate above the top."""
    if v >= grid[-1]:
        return len(grid) - 1
    best = None
    for i, g in enumerate(grid):
        d = abs(v - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def _sample_patterns(lo: float, hi: float, points, rng, n_random=20000, spread=64):
    """float32 values in [lo, hi]: every grid point and midpoint +-spread ulps,
    plus random patterns."""
    vals = []
    for p in points:
        b = np.float32(p).view(np.uint32).astype(np.int64)
        vals.append((b + np.arange(-spread, spread + 1)).clip(0, None).astype(np.uint32).view(np.float32))
    lo_b = np.float32(lo).view(np.uint32)
    hi_b = np.float32(hi).view(np.uint32)
    vals.append(rng.integers(lo_b, hi_b, n_random, dtype=np.uint32).view(np.float32))
    v = np.concatenate(vals)
    return v[(v >= lo) & (v <= hi)]


def test_e2m1_ties_by_hand():
    # Halfway points between grid neighbours go to the even mantissa.
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 1e30], np.float32)
    assert list(F.f32_to_e2m1(y)) == [0, 2, 2, 4, 4, 6, 6, 7, 7]
    assert list(F.f32_to_e2m1(-y)) == [8, 10, 10, 12, 12, 14, 14, 15, 15]
    assert list(F.f32_to_e2m1(np.array([-0.0, 0.0, -0.1], np.float32))) == [8, 0, 8]


def test_e2m1_against_fraction_rne():
    grid = [Fraction(x).limit_denominator() for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    v = _sample_patterns(0.0, 16.0, list(F.E2M1_MAGNITUDES) + mids, np.random.default_rng(7), 5000, 40)
    got = F.f32_to_e2m1(v)
    want = np.array([_frac_nearest_even(Fraction(float(x)), grid) for x in v], np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_against_torch_cast():
    # torch's float -> float8_e4m3fn cast is RNE; it agrees with satfinite up to 448.
    tab = F.e4m3_value(np.arange(0x7F))
    mids = list((tab[1:] + tab[:-1]) / 2)
    v = _sample_patterns(0.0, 448.0, list(tab) + mids, np.random.default_rng(11), 200000, 300)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.f32_to_e4m3(v), lib)


def test_e4m3_against_fraction_and_saturation():
    tab = [Fraction(float(t)) for t in F.e4m3_value(np.arange(0x7F))]
    v = _sample_patterns(0.0, 1000.0, [2.0 ** -10, 2.0 ** -9, 1.5 * 2.0 ** -9, 4.25, 448.0, 464.0], np.random.default_rng(3), 3000, 8)
    want = np.array([_frac_nearest_even(Fraction(float(x)), tab) for x in v], np.uint8)
    assert np.array_equal(F.f32_to_e4m3(v), want)
    assert F.f32_to_e4m3(np.float32(1e30)) == 0x7E
    assert F.f32_to_e4m3(np.float32(2.0 ** -10)) == 0x00   # tie with 0 -> even
    assert F.f32_to_e4m3(np.float32(3 * 2.0 ** -10)) == 0x02  # tie 1/2 subnormal -> even
    with pytest.raises(ValueError):
        F.f32_to_e4m3(np.float32(-1.0))


def test_bf16_against_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]  # finite only
    # force exact ties and near-ties
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    bits[1000:2000] = (bits[1000:2000] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(x), lib)
    # widening is exact
    assert np.array_equal(F.bf16_bits_to_f32(lib), torch.from_numpy(lib.view(np.int16)).view(torch.bfloat16).float().numpy())


def _sweep(lo_bits: int, hi_bits: int, check, chunk: int = 1 << 24):
    """Run check(float32 values) over every bit pattern in [lo_bits, hi_bits),
    in chunks spread over a thread pool (NumPy releases the GIL in the
    element-wise work).  Returns the number of patterns checked."""
    starts = range(lo_bits, hi_bits, chunk)

    def one(start):
        b = np.arange(start, min(start + chunk, hi_bits), dtype=np.uint32)
        check(b.view(np.float32))
        return b.size

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        return sum(ex.map(one, starts))


def test_e2m1_exhaustive_nonnegative():
    """Every non-negative float32 up to 8 (beyond the saturation point 5) and
    every one of their negatives: the converter against the threshold rule
    written from the grid (midpoints between neighbours, ties to the even
    code), and sign symmetry (-y gives the code of y with bit 3 set).
    Everything above 8 saturates like 8 does (sampled)."""
    thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])

    def check(y):
        got = F.f32_to_e2m1(y)
        yy = y.astype(np.float64)
        # ties (y == threshold) go up only where the upper neighbour is even
        want = sum(((yy >= t) if i % 2 == 1 else (yy > t)).astype(np.uint8) for i, t in enumerate(thr))
        assert np.array_equal(got, want)
        assert np.array_equal(F.f32_to_e2m1(-y), want | 8)

    n = _sweep(0, 0x41000001, check)
    assert n == 0x41000001
    big = np.random.default_rng(8).integers(0x41000000, 0x7F800000, 1 << 20, dtype=np.uint32).view(np.float32)
    assert np.all(F.f32_to_e2m1(big) == 7) and np.all(F.f32_to_e2m1(-big) == 15)


def test_e4m3_exhaustive_nonnegative():
    """Every non-negative float32 below 464 (the midpoint between 448 and the
    first unrepresentable 480, where saturation takes over): the converter
    against torch's float8_e4m3fn cast (RNE; a library routine), and 448
    (0x7E) from 464 up to the largest finite float32 (sampled, plus the
    boundary patterns)."""
    def check(y):
        lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(F.f32_to_e4m3(y), lib)

    n = _sweep(0, 0x43E80000, check)
    assert n == 0x43E80000
    hi = np.concatenate([np.arange(0x43E80000, 0x43E80000 + 4096, dtype=np.uint32),
                         np.random.default_rng(9).integers(0x43E80000, 0x7F800000, 1 << 20, dtype=np.uint32),
                         np.array([0x7F7FFFFF], np.uint32)]).view(np.float32)
    assert np.all(F.f32_to_e4m3(hi) == 0x7E)
