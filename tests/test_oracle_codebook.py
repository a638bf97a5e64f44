"""Pins for the oracle's NF4 codebook: structure, and an independent
high-precision evaluation of the normal quantiles (mpmath, 200 bits)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_sixteen_levels_sorted_in_unit_interval():
    lv = oracle.nf4_levels()
    assert lv.dtype == np.float32 and lv.shape == (16,)            # 4 bits -> 16 codes
    assert np.all(np.diff(lv.astype(np.float64)) > 0)             # strictly increasing
    assert lv[0] == -1.0 and lv[15] == 1.0                          # normalised to [-1, 1]
    assert lv[7] == 0.0 and not np.signbit(lv[7])                   # an exact (+) zero
    assert (lv < 0).sum() == 7 and (lv > 0).sum() == 8              # asymmetric 7 / 8 split


def test_levels_are_normal_quantiles_scipy():
    """Every level times the outer quantile is a standard-normal quantile at the
    evenly spaced probabilities of the construction (checked with scipy's CDF)."""
    from scipy.stats import norm
    lv = oracle.nf4_levels_f64()
    delta = float(oracle.NF4_DELTA)
    top = norm.ppf(delta)
    pos = [v for v in lv if v > 0]
    neg = sorted([-v for v in lv if v < 0])
    for k, v in enumerate(pos, start=1):
        assert abs(norm.cdf(v * top) - (0.5 + (delta - 0.5) * k / 8)) < 1e-12
    for k, v in enumerate(neg, start=1):
        assert abs(norm.cdf(v * top) - (0.5 + (delta - 0.5) * k / 7)) < 1e-12


def test_levels_match_200_bit_evaluation():
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    with mpmath.workprec(200):
        d = mpmath.mpf(31) / 32 / 2 + mpmath.mpf(29) / 30 / 2

        def ppf(p):
            return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)
        top = ppf(d)
        vals = [ppf(mpmath.mpf(1) / 2 + (d - mpmath.mpf(1) / 2) * k / 8) / top for k in range(1, 9)]
        vals += [-ppf(mpmath.mpf(1) / 2 + (d - mpmath.mpf(1) / 2) * k / 7) / top for k in range(1, 8)]
        vals += [mpmath.mpf(0)]
        vals.sort()
    ref = []
    for v in vals:
        with mpmath.workprec(24):               # round once to a 24-bit significand (float32)
            r = +v
        ref.append(np.float32(float(r)))
    assert np.array_equal(np.array(ref, np.float32).view(np.uint32), oracle.nf4_levels().view(np.uint32))
    del mp


def test_delta_value():
    assert oracle.NF4_DELTA == (Fraction(31, 32) + Fraction(29, 30)) / 2
    assert abs(float(oracle.NF4_DELTA) - 0.9677083) < 1e-7


def test_midpoints_exact_and_four_representable_ties():
    mid = oracle.nf4_midpoints()
    lv = oracle.nf4_levels().astype(np.float64)
    assert np.all((lv[:-1] < mid) & (mid < lv[1:]))
    representable = [j for j in range(15) if float(np.float32(mid[j])) == mid[j]]
    # ties really occur for float32 inputs at these midpoints
    assert representable == [2, 6, 7, 14]
