"""Test-side exact arithmetic helpers (independent of the oracle).

``nearest_f32`` finds the binary32 nearest to a Fraction by comparing the
exact distances of three candidates around numpy's double-rounded guess; the
true nearest value is always among them because two roundings are off by at
most one binary32 step.
"""

from fractions import Fraction

import numpy as np

F32 = np.float32


def frac(x) -> Fraction:
    return Fraction(float(x))


def nearest_f32(fr: Fraction) -> np.float32:
    with np.errstate(over="ignore"):
        c = np.float32(float(fr))
    cands = [np.nextafter(c, F32(-np.inf), dtype=F32), c, np.nextafter(c, F32(np.inf), dtype=F32)]
    best = None
    for v in cands:
        if not np.isfinite(v):
            continue
        d = abs(Fraction(float(v)) - fr)
        key = (d, int(np.asarray(v, dtype=F32).view(np.uint32)) & 1)  # ties: even mantissa
        if best is None or key < best[0]:
            best = (key, v)
    return F32(best[1])


def rn(fr: Fraction) -> np.float32:
    """Round a Fraction to binary32 (ties to even), returning +-0 as +0."""
    if fr == 0:
        return F32(0.0)
    if fr < 0:
        return F32(-nearest_f32(-fr))
    return nearest_f32(fr)


def ulp(x) -> Fraction:
    """Spacing of binary32 at |x| (Fraction)."""
    x = abs(F32(x))
    nx = np.nextafter(x, F32(np.inf), dtype=F32)
    if not np.isfinite(nx):
        return Fraction(2) ** 104
    return Fraction(float(nx)) - Fraction(float(x))


def _floor_log2(fr: Fraction) -> int:
    """floor(log2(fr)) of a positive Fraction."""
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    elif Fraction(2) ** (e + 1) <= fr:
        e += 1
    return e


def rn64(fr: Fraction) -> Fraction:
    """The binary64 nearest to a positive Fraction (ties to even), as a
    Fraction; normal range only."""
    assert fr > 0
    e = _floor_log2(fr) - 52                  # fr / 2^e in [2^52, 2^53)
    M = fr / Fraction(2) ** e
    q = M.numerator // M.denominator
    rem = M - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return q * Fraction(2) ** e


def sqrt_rn64(fr: Fraction) -> Fraction:
    """The binary64 nearest to the square root of a positive Fraction (ties
    to even, though an exact tie cannot occur for a rational square root of a
    binary64 value), with integer square roots only."""
    import math

    assert fr > 0
    e = (_floor_log2(fr) >> 1) - 52           # sqrt(fr) / 2^e in [2^52, 2^54)
    T = fr / Fraction(4) ** e                 # (sqrt(fr) / 2^e)^2
    q = math.isqrt(T.numerator // T.denominator)   # floor(sqrt(T))
    while q >= 1 << 53:                       # keep 53 significant bits
        e += 1
        T = T / 4
        q = math.isqrt(T.numerator // T.denominator)
    half = Fraction(2 * q + 1, 2)
    if T > half * half or (T == half * half and q % 2 == 1):
        q += 1
    return q * Fraction(2) ** e
