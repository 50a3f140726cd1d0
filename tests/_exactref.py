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
