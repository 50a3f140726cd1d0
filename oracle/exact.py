"""Exact means of binary32 data, rounded once to binary32.

The 1-bit scaled sign takes the mean absolute value of the data it compresses
(gradient-quantisation tutorial, "1-bit gradient quantisation", scaled-sign
variant; applied per chunk of the fused buffer).  The pages do not fix a
summation order, so the oracle uses the order-free definition: the exact real
number sum(|x_j|) / L, rounded to the nearest binary32 (ties to even).

Every finite binary32 value is an integer multiple of 2^-149, so the sum is an
exact Python integer in units of 2^-149.

Pins: Fraction brute force on small inputs, and numpy's own float64 -> float32
cast for the rounding step (tests/test_oracle_exact.py).
"""

from __future__ import annotations

import math

import numpy as np

_TWO24 = 1 << 24
_TWO23 = 1 << 23


def round_rational_to_f32(num: int, den: int) -> np.float32:
    """binary32 value nearest to num/den (num >= 0, den > 0), ties to even.

    Values at or beyond the overflow threshold give +inf."""
    if num < 0 or den <= 0:
        raise ValueError("round_rational_to_f32 expects num >= 0, den > 0")
    if num == 0:
        return np.float32(0.0)
    # choose k so that 2^23 <= num * 2^k / den < 2^24, but never finer than
    # the subnormal spacing 2^-149 (k <= 149)
    k = 23 - (num.bit_length() - den.bit_length())
    while True:
        q = (num << k) // den if k >= 0 else num // (den << -k)
        if q >= _TWO24:
            k -= 1
        elif q < _TWO23 and k < 149:
            k += 1
        else:
            break
    k = min(k, 149)
    if k >= 0:
        q, r = divmod(num << k, den)
        d = den
    else:
        d = den << -k
        q, r = divmod(num, d)
    # round to nearest, ties to even
    if 2 * r > d or (2 * r == d and (q & 1)):
        q += 1
    if q == _TWO24:  # carried into the next binade
        q = _TWO23
        k -= 1
    if k < -104:
        # q < 2^24, so q * 2^-k exceeds the largest finite binary32
        # (2^24 - 1) * 2^104 exactly when the binade is above 2^104
        return np.float32(np.inf)
    return np.float32(math.ldexp(q, -k))


def abs_units(x: np.ndarray) -> int:
    """Exact sum of |x| for finite binary32 x, in integer units of 2^-149.

    Each |x| = M * 2^(E-150) for a normal number (E = biased exponent,
    M = 24-bit significand with the hidden bit) and M * 2^-149 for a
    subnormal one; the significands are summed per exponent (integers below
    2^53, so float64 accumulation is exact) and then combined in Python
    integers."""
    a = np.abs(np.asarray(x, dtype=np.float32)).ravel()
    if a.size >= (1 << 29):
        raise ValueError("too many terms for exact per-exponent accumulation")
    bits = a.view(np.uint32)
    e = (bits >> 23).astype(np.int64)
    m = (bits & 0x7FFFFF).astype(np.int64)
    m = np.where(e > 0, m | 0x800000, m)
    e = np.maximum(e, 1)
    per_exp = np.bincount(e, weights=m.astype(np.float64), minlength=256)
    total = 0
    for ex in range(1, 255):
        c = per_exp[ex]
        if c:
            total += int(c) << (ex - 1)
    return total


def mean_abs_f32(x: np.ndarray) -> np.float32:
    """binary32 nearest to mean(|x|) over all elements (exact, ties to even).

    NaN anywhere gives NaN; otherwise an infinity gives +inf."""
    a = np.asarray(x, dtype=np.float32).ravel()
    if a.size == 0:
        raise ValueError("mean of an empty chunk")
    if np.isnan(a).any():
        return np.float32(np.nan)
    if np.isinf(a).any():
        return np.float32(np.inf)
    return round_rational_to_f32(abs_units(a), a.size << 149)
