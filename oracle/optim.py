"""Frozen-variance parameter steps of 1-bit Adam and 1-bit LAMB.

Sources:
* 1-bit Adam article, section 2.1: Adam's first and second moment recursions;
  section 6 (tuning): lr 6e-5, betas (0.9, 0.999), eps 1e-6.
* 1-bit LAMB page, algorithm paragraph: after warmup the denominator
  sqrt(v_Tw) is frozen; the layer gradient is reconstructed from two
  consecutive compressed momenta, g_t = (m_t - beta1 m_{t-1}) / (1 - beta1);
  a fresh variance v_t = beta2 v_{t-1} + (1 - beta2) g_t^2 is kept; the
  per-layer ratio r_t = clip(clip(||v_Tw / v_t||_inf, (1-thr) r_{t-1},
  (1+thr) r_{t-1}), r_min, r_max) scales the warmup average coefficient,
  c_t = c_avg r_t.
* 1-bit LAMB page, analysis paragraph: the effective layer learning rate of
  step t is gamma c_{t-1}, so the update of step t uses the coefficient of
  the previous step (default reading); ``use_c_t`` selects the other reading
  (the coefficient computed in the same step).

Readings where the pages are silent:
* Adam step: x <- x - lr * (m / (sqrt(v) + eps)), eps outside the root, no
  bias correction (v is frozen, so it would be a constant folded into lr), no
  weight decay; each operation one binary32 rounding in that order.
* LAMB ratio: elementwise v_Tw / v_t; the layer max skips NaN (0/0) and keeps
  +inf (the soft clip bounds it); of +0 and -0 the max is +0; a layer with no
  valid ratio keeps r_{t-1}.  lo = (1-thr) r_{t-1} and hi = (1+thr) r_{t-1}
  with binary32 constants; clip(x, a, b) = fmin(fmax(x, a), b).
* First compressed step: r = 1 and c = c_avg; the fresh variance starts at
  v_Tw.

Parity pins (tests/test_oracle_optim.py): hand-evaluated points, special
cases (m = 0, lr = 0, eps placement), the momentum round trip of the gradient
reconstruction, r_t bounds, r_min = r_max = 1 (basic 1-bit LAMB: r stays 1),
g^2 = v_Tw giving ratio 1.
"""

from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

f32 = np.float32


def adam_frozen_step(x: np.ndarray, m: np.ndarray, v: np.ndarray, lr: float, eps: float) -> np.ndarray:
    """x - lr * (m / (sqrt(v) + eps)) with frozen v (binary32)."""
    x = np.asarray(x, dtype=f32)
    den = (np.sqrt(np.asarray(v, dtype=f32)) + f32(eps)).astype(f32)
    upd = (np.asarray(m, dtype=f32) / den).astype(f32)
    return (x - (f32(lr) * upd).astype(f32)).astype(f32)


def reconstruct_gradient(m: np.ndarray, m_prev: np.ndarray, beta1: float) -> np.ndarray:
    """g_t = (m_t - beta1 m_{t-1}) / (1 - beta1)."""
    b1 = f32(beta1)
    omb1 = f32(f32(1.0) - b1)
    num = (np.asarray(m, dtype=f32) - (b1 * np.asarray(m_prev, dtype=f32)).astype(f32)).astype(f32)
    return (num / omb1).astype(f32)


def fresh_variance(v_f: np.ndarray, g: np.ndarray, beta2: float) -> np.ndarray:
    """v_t = beta2 v_{t-1} + (1 - beta2) g_t^2."""
    b2 = f32(beta2)
    omb2 = f32(f32(1.0) - b2)
    g = np.asarray(g, dtype=f32)
    return ((b2 * np.asarray(v_f, dtype=f32)).astype(f32)
            + (omb2 * (g * g).astype(f32)).astype(f32)).astype(f32)


def layer_max(vals: np.ndarray, seg_off) -> np.ndarray:
    """Per-segment maximum skipping NaN (+0 beats -0); NaN if no valid value."""
    out = np.full(len(seg_off) - 1, np.nan, dtype=f32)
    for l in range(len(seg_off) - 1):
        seg = np.asarray(vals[int(seg_off[l]):int(seg_off[l + 1])], dtype=f32)
        seg = seg[~np.isnan(seg)]
        if seg.size == 0:
            continue
        mx = seg.max()
        if mx == 0 and np.any((seg == 0) & ~np.signbit(seg)):
            mx = f32(0.0)
        out[l] = mx
    return out


def lamb_ratio_update(R: np.ndarray, r_prev: np.ndarray, c_avg: np.ndarray,
                      thr: float, r_min: float, r_max: float) -> Tuple[np.ndarray, np.ndarray]:
    """r_t = clip(clip(R, (1-thr) r_{t-1}, (1+thr) r_{t-1}), r_min, r_max) and
    c_t = c_avg r_t; R NaN (no valid ratio) keeps r_{t-1}."""
    R = np.asarray(R, dtype=f32)
    r_prev = np.asarray(r_prev, dtype=f32)
    R = np.where(np.isnan(R), r_prev, R).astype(f32)
    lo = (f32(f32(1.0) - f32(thr)) * r_prev).astype(f32)
    hi = (f32(f32(1.0) + f32(thr)) * r_prev).astype(f32)
    r = np.fmin(np.fmax(R, lo), hi).astype(f32)
    r = np.fmin(np.fmax(r, f32(r_min)), f32(r_max)).astype(f32)
    c = (np.asarray(c_avg, dtype=f32) * r).astype(f32)
    return r, c


def lamb_apply(x: np.ndarray, m: np.ndarray, v_tw: np.ndarray, seg_off, c_used: np.ndarray,
               lr: float, eps: float) -> np.ndarray:
    """x - (lr c_l) * (m / (sqrt(v_Tw) + eps)), per segment l."""
    x = np.asarray(x, dtype=f32)
    den = (np.sqrt(np.asarray(v_tw, dtype=f32)) + f32(eps)).astype(f32)
    upd = (np.asarray(m, dtype=f32) / den).astype(f32)
    out = np.empty_like(x)
    for l in range(len(seg_off) - 1):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        step = f32(f32(lr) * f32(c_used[l]))
        out[a:b] = (x[a:b] - (step * upd[a:b]).astype(f32)).astype(f32)
    return out


def lamb_frozen_step(x, m, m_prev, v_f, v_tw, seg_off, c_avg, r_prev, c_prev,
                     lr: float, eps: float, beta1: float, beta2: float,
                     thr: float, r_min: float, r_max: float,
                     use_c_t: bool = False) -> Dict[str, np.ndarray]:
    """One 1-bit LAMB step over the fused buffer.  Returns the new x, fresh
    variance, per-layer max ratio R, r_t and c_t."""
    g = reconstruct_gradient(m, m_prev, beta1)
    v_new = fresh_variance(v_f, g, beta2)
    ratio = (np.asarray(v_tw, dtype=f32) / v_new).astype(f32)
    R = layer_max(ratio, seg_off)
    r, c = lamb_ratio_update(R, r_prev, c_avg, thr, r_min, r_max)
    c_used = c if use_c_t else np.asarray(c_prev, dtype=f32)
    x_new = lamb_apply(x, m, v_tw, seg_off, c_used, lr, eps)
    # factor for the next step's error feedback: c_{t-1} / c_t of each layer
    rho = (np.asarray(c_prev, dtype=f32) / c).astype(f32)
    return {"x": x_new, "v": v_new, "R": R, "r": r, "c": c, "g": g, "err_ratio": rho}
