"""Pins of the oracle's exact binary32 mean (oracle/exact.py).

* The rational -> binary32 rounding is checked against numpy's float64 ->
  float32 cast (one correctly rounded conversion) on doubles that span the
  normal, subnormal and overflow ranges, including exact midpoints.
* The mean is checked against brute force with Python Fractions.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle.exact import abs_units, mean_abs_f32, round_rational_to_f32


def _f32_from_fraction_by_cast(fr: Fraction) -> np.float32:
    d = float(fr)
    assert Fraction(d) == fr, "helper only valid for values exact in float64"
    with np.errstate(over="ignore"):
        return np.float32(d)


def test_round_matches_numpy_cast_random():
    rng = np.random.default_rng(1)
    for _ in range(20000):
        d = float(np.exp(rng.uniform(-108, 90)))
        fr = Fraction(d)
        got = round_rational_to_f32(fr.numerator, fr.denominator)
        with np.errstate(over="ignore"):
            want = np.float32(d)
        assert got == want or (np.isinf(got) and np.isinf(want)), d


def test_round_exact_midpoints_ties_to_even():
    rng = np.random.default_rng(2)
    a = rng.integers(1, 2**31 - 2**23, size=3000, dtype=np.int64).astype(np.uint32)
    lo = a.view(np.float32)
    hi = (a + 1).view(np.float32)
    for x, y in zip(lo, hi):
        if not (np.isfinite(x) and np.isfinite(y)):
            continue
        mid = (Fraction(float(x)) + Fraction(float(y))) / 2
        got = round_rational_to_f32(mid.numerator, mid.denominator)
        want = _f32_from_fraction_by_cast(mid)
        assert got == want
        even = x if (x.view(np.uint32) & 1) == 0 else y
        assert got == even


def test_round_subnormal_and_overflow():
    tiny = Fraction(1, 2**149)
    assert round_rational_to_f32(tiny.numerator, tiny.denominator) == np.float32(2.0**-149)
    half_tiny = tiny / 2  # exact tie between 0 and 2^-149: rounds to even (0)
    assert round_rational_to_f32(half_tiny.numerator, half_tiny.denominator) == 0.0
    three_halves = tiny * 3 / 2  # tie between 1 and 2 units: even is 2 units
    assert round_rational_to_f32(three_halves.numerator, three_halves.denominator) == np.float32(2.0**-148)
    fmax = Fraction((2**24 - 1) * 2**104)
    assert round_rational_to_f32(fmax.numerator, 1) == np.finfo(np.float32).max
    over = fmax + Fraction(2**103)  # the midpoint to 2^128 rounds away (to inf)
    assert np.isinf(round_rational_to_f32(over.numerator, 1))
    under = fmax + Fraction(2**103) - 1
    assert round_rational_to_f32(under.numerator, 1) == np.finfo(np.float32).max


def _brute_mean_abs(x: np.ndarray) -> Fraction:
    return sum((abs(Fraction(float(v))) for v in x), Fraction(0)) / len(x)


@pytest.mark.parametrize("L", [1, 3, 64, 257])
def test_mean_abs_matches_fractions(L):
    rng = np.random.default_rng(L)
    for trial in range(40):
        scale = 10.0 ** rng.uniform(-40, 35, size=L)
        x = (rng.standard_normal(L) * scale).astype(np.float32)
        if trial % 5 == 0:
            x[: L // 2] = np.float32(1e-45) * rng.integers(0, 50, size=L // 2)  # subnormals
        fr = _brute_mean_abs(x)
        assert abs_units(x) == sum(abs(Fraction(float(v))) for v in x) * 2**149
        got = mean_abs_f32(x)
        want = _f32_from_fraction_by_cast(fr) if Fraction(float(fr)) == fr else None
        if want is not None:
            assert got == want
        # independently: got must be the nearest binary32 to fr
        below = np.nextafter(got, np.float32(-np.inf), dtype=np.float32)
        above = np.nextafter(got, np.float32(np.inf), dtype=np.float32)
        dist = abs(Fraction(float(got)) - fr)
        if np.isfinite(below) and below >= 0:
            assert dist <= abs(Fraction(float(below)) - fr)
        if np.isfinite(above):
            assert dist <= abs(Fraction(float(above)) - fr)


def test_mean_abs_ties():
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2.0), dtype=np.float32)      # 1 + 2^-23
    up2 = np.nextafter(up, np.float32(2.0), dtype=np.float32)      # 1 + 2^-22
    # mean of 1 and 1+2^-23 is the midpoint 1 + 2^-24: ties to even -> 1
    assert mean_abs_f32(np.array([one, -up] * 32, dtype=np.float32)) == one
    # mean of 1+2^-23 and 1+2^-22 is a midpoint whose even neighbour is 1+2^-22
    assert mean_abs_f32(np.array([up, up2] * 32, dtype=np.float32)) == up2
    # just off the midpoint it must round to the nearer neighbour
    x = np.array([one, up] * 32, dtype=np.float32)
    x[0] = np.nextafter(one, np.float32(2.0), dtype=np.float32)
    assert mean_abs_f32(x) == up


def test_mean_abs_specials():
    assert np.isnan(mean_abs_f32(np.array([1, np.nan, np.inf], dtype=np.float32)))
    assert mean_abs_f32(np.array([1, -np.inf], dtype=np.float32)) == np.inf
    assert mean_abs_f32(np.zeros(64, dtype=np.float32)) == 0.0
    z = np.zeros(64, dtype=np.float32)
    z[3] = -0.0
    assert mean_abs_f32(z) == 0.0 and not np.signbit(mean_abs_f32(z))
    big = np.full(64, np.finfo(np.float32).max, dtype=np.float32)
    assert mean_abs_f32(big) == np.finfo(np.float32).max


def test_mean_abs_is_rounded_once_from_the_exact_value():
    """The mean must not pass through binary64. |x| = 3, 3 2^-24 and 2^-100:
    the exact mean 1 + 2^-24 + 2^-100 / 3 lies just above the midpoint
    between 1 and 1 + 2^-23 and rounds up; a binary64 sum drops the 2^-100,
    its quotient is the midpoint itself, and the tie goes to the even 1.
    Mirrored: |y| = 3, 9 2^-24 - 2^-44 and 2^-44 - 2^-68 (binary32 values)
    sum to 3 (1 + 3 2^-24) - 2^-68, whose mean lies just below the midpoint
    between 1 + 2^-23 (odd) and 1 + 2^-22 and rounds down; through binary64
    it ties up."""
    F = np.float32
    x = np.array([3.0, -3.0 * 2.0 ** -24, 2.0 ** -100], dtype=F)
    assert mean_abs_f32(x) == F(1 + 2.0 ** -23)
    y = np.array([3.0, np.nextafter(F(9 * 2.0 ** -24), F(0)),
                  -np.nextafter(F(2.0 ** -44), F(0))], dtype=F)
    assert Fraction(float(y[1])) == Fraction(9, 2 ** 24) - Fraction(1, 2 ** 44)
    assert -Fraction(float(y[2])) == Fraction(1, 2 ** 44) - Fraction(1, 2 ** 68)
    assert mean_abs_f32(y) == F(1 + 2.0 ** -23)
