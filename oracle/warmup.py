"""Warmup phase and the transition to compressed training.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU baseline, never by the library.

Sources:
* 1-bit Adam article, section 2.1: Adam's recursions m_t = beta1 m_{t-1} +
  (1 - beta1) g_t and v_t = beta2 v_{t-1} + (1 - beta2) g_t^2; its
  configuration block: the first warmup_steps steps run without
  quantisation.
* 1-bit LAMB page, algorithm paragraph: v_Tw and the warmup moving average
  c_avg of LAMB's layer coefficient c_t are what the compressed phase keeps;
  layer-scaling paragraph: a fixed per-layer momentum scale k_l is computed
  from the average momentum norm at the end of warmup.

Readings where the pages are silent (each listed in the design notes):
* Adam warmup step: the two recursions with 1 - beta rounded once, then
  x <- x - lr * (m / (sqrt(v) + eps)) with the new m and v; no bias
  correction, no weight decay (the same update as the frozen-variance step).
* LAMB warmup step: the same m and v, u = m / (sqrt(v) + eps), and per layer
  the trust ratio c_l = ||x_l|| / ||u_l|| of LAMB (x before the update),
  c_l = 1 when either norm is zero; x <- x - (lr c_l) u.  The squared norms
  are the exact sums rounded once to binary64, the ratio is
  sqrt(Sx) / sqrt(Su) in binary64, rounded once to binary32.
* c_avg is an exponential moving average of c with factor beta_c, started at
  the first warmup coefficient: c_avg = c_1, then
  c_avg = beta_c c_avg + (1 - beta_c) c (binary32, 1 - beta_c rounded once).
* k_l: the "average momentum norm" of layer l is its root mean square
  a_l = sqrt(||m_l||^2 / d_l); layers are scaled to the mean magnitude,
  k_l = mean_l'(a_l') / a_l, the mean over layers with a_l' > 0; a layer
  with a_l = 0 (or no elements) gets k_l = 1.  Computed in binary64 from
  exact sums, rounded once to binary32.
* Transition: v_Tw = v at the end of warmup; the compressed phase starts with
  r = 1, c = c_avg, fresh variance v_Tw and previous momentum m_Tw.

Parity pins (tests/test_oracle_warmup.py): hand-evaluated steps, the closed
form of the moments under a constant gradient with dyadic betas, beta2 = 1
reducing to the frozen step, the trust ratio against a library norm and its
scale invariance, zero-norm layers, the moving average by hand, and k_l on
layers of constant magnitude.
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Optional

import numpy as np

f32 = np.float32


def _omb(beta: float) -> np.float32:
    return f32(f32(1.0) - f32(beta))


def moments(m: np.ndarray, v: np.ndarray, g: np.ndarray, beta1: float, beta2: float):
    """m_t = beta1 m + (1 - beta1) g and v_t = beta2 v + (1 - beta2) g^2 in
    binary32, one rounding per operation."""
    b1, b2 = f32(beta1), f32(beta2)
    g = np.asarray(g, dtype=f32)
    m_new = ((b1 * np.asarray(m, dtype=f32)).astype(f32) + (_omb(beta1) * g).astype(f32)).astype(f32)
    v_new = ((b2 * np.asarray(v, dtype=f32)).astype(f32)
             + (_omb(beta2) * (g * g).astype(f32)).astype(f32)).astype(f32)
    return m_new, v_new


def adam_direction(m: np.ndarray, v: np.ndarray, eps: float) -> np.ndarray:
    """u = m / (sqrt(v) + eps) in binary32."""
    den = (np.sqrt(np.asarray(v, dtype=f32)) + f32(eps)).astype(f32)
    return (np.asarray(m, dtype=f32) / den).astype(f32)


def adam_warmup_step(x, m, v, g, lr: float, eps: float, beta1: float,
                     beta2: float) -> Dict[str, np.ndarray]:
    """One uncompressed Adam step on the averaged gradient g."""
    m_new, v_new = moments(m, v, g, beta1, beta2)
    u = adam_direction(m_new, v_new, eps)
    x_new = (np.asarray(x, dtype=f32) - (f32(lr) * u).astype(f32)).astype(f32)
    return {"x": x_new, "m": m_new, "v": v_new}


def exact_sumsq(a: np.ndarray) -> float:
    """Sum of squares of binary32 values: exact, rounded once to binary64.
    Each square is exact in binary64 (24 x 24 significand bits), so the
    correctly rounded float sum of the squares is that value."""
    sq = np.asarray(a, dtype=f32).astype(np.float64) ** 2
    return math.fsum(sq.tolist())


def trust_ratio(x_l: np.ndarray, u_l: np.ndarray) -> np.float32:
    """||x_l|| / ||u_l||, or 1 when either norm is zero."""
    sx, su = exact_sumsq(x_l), exact_sumsq(u_l)
    if sx == 0.0 or su == 0.0:
        return f32(1.0)
    return f32(math.sqrt(sx) / math.sqrt(su))


def coefficient_average(c_avg: Optional[np.ndarray], c: np.ndarray, beta_c: float) -> np.ndarray:
    """EMA of the layer coefficients; None (no step yet) starts it at c."""
    c = np.asarray(c, dtype=f32)
    if c_avg is None:
        return c.copy()
    return ((f32(beta_c) * np.asarray(c_avg, dtype=f32)).astype(f32)
            + (_omb(beta_c) * c).astype(f32)).astype(f32)


def lamb_warmup_step(x, m, v, g, seg_off, lr: float, eps: float, beta1: float, beta2: float,
                     c_avg: Optional[np.ndarray] = None,
                     beta_c: float = 0.9) -> Dict[str, np.ndarray]:
    """One uncompressed LAMB step on the averaged gradient g over the fused
    buffer with layer offsets seg_off; also advances the coefficient average."""
    x = np.asarray(x, dtype=f32)
    m_new, v_new = moments(m, v, g, beta1, beta2)
    u = adam_direction(m_new, v_new, eps)
    S = len(seg_off) - 1
    c = np.ones(S, dtype=f32)
    x_new = x.copy()
    for l in range(S):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        c[l] = trust_ratio(x[a:b], u[a:b])
        step = f32(f32(lr) * c[l])
        x_new[a:b] = (x[a:b] - (step * u[a:b]).astype(f32)).astype(f32)
    return {"x": x_new, "m": m_new, "v": v_new, "u": u, "c": c,
            "c_avg": coefficient_average(c_avg, c, beta_c)}


def momentum_scale(m: np.ndarray, seg_off) -> np.ndarray:
    """k_l = mean over layers of the RMS momentum / RMS of layer l."""
    m = np.asarray(m, dtype=f32)
    S = len(seg_off) - 1
    rms = [0.0] * S
    for l in range(S):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        if b > a:
            rms[l] = math.sqrt(exact_sumsq(m[a:b]) / (b - a))
    valid = [r for r in rms if r > 0.0]
    k = np.ones(S, dtype=f32)
    if not valid:
        return k
    mean = math.fsum(valid) / len(valid)
    for l in range(S):
        if rms[l] > 0.0:
            k[l] = f32(mean / rms[l])
    return k


def exact_rms_ratio(m: np.ndarray, seg_off, l: int) -> Fraction:
    """(sum of squares of layer l / d_l) as an exact rational, for pins."""
    a, b = int(seg_off[l]), int(seg_off[l + 1])
    s = sum(Fraction(float(t)) ** 2 for t in np.asarray(m[a:b], dtype=f32))
    return s / (b - a)
