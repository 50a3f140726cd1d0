"""Block-wise INT8 stochastic rounding with error feedback.

Sources (gradient-quantisation tutorial):
* "FP32 -> INT8", step 1: scale = max|g| / 127, dequantised value q * scale,
  codes in [-127, 127];
* step 2: one scale per block;
* step 3 and the PyTorch example: stochastic rounding -- floor of g/scale,
  plus one with probability equal to the fractional part -- then the clamp
  to [-127, 127] and the dequantisation q * scale;
* "1-bit gradient quantisation" (error feedback) and "accuracy recovery":
  keep the residual and add it before the next quantisation.

Readings:
* the quantised value is the error-compensated g' = g + e; M = max(0, max
  |g'| over the block's non-NaN elements); scale = M / 127 by a correctly
  rounded division; scale == 0 gives code 0 and dequantised 0;
* x = g' / scale by true division (never a reciprocal), f = floor(x),
  p = x - f, code = f + (u < p), clamped by fmin/fmax to [-127, 127] (a NaN
  x therefore gives -127);
* u is the Philox uniform of ``philox.uniforms`` (keyed by seed, element
  index and step);
* new error e = g' - q * scale.

Variants: a per-tensor scale (block 0) and deterministic rounding to the
nearest integer, halves away from zero.

Parity pins (tests/test_oracle_int8.py): codes in range, |deq - g'| < scale
away from the clamp, integral x gives a deterministic code, all-zero blocks,
the block maximum's code, unbiasedness over seeds, the comparison u < p
(a fraction equal to its own uniform rounds down: of the 2^24 grid values of
u exactly p 2^24 lie below such a p), the clamp reached from -128 and +128
(a scale that rounds down puts the maximum just past 127), and a NaN left
out of the block maximum.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .philox import uniforms

f32 = np.float32


def round_half_away(x: np.ndarray) -> np.ndarray:
    """Nearest integer, halves away from zero (the ordinary rounding the
    tutorial's step 1 names); exact on binary32."""
    x = np.asarray(x, dtype=f32)
    t = np.trunc(x).astype(f32)
    frac = np.abs((x - t).astype(f32))
    return np.where(frac >= f32(0.5), (t + np.sign(x)).astype(f32), t).astype(f32)


def int8_sr(g: np.ndarray, e: Optional[np.ndarray], seed: int, step: int,
            block: int = 256, J0: int = 0, rounding: str = "stochastic") -> Dict[str, np.ndarray]:
    """Quantise g (+ e when given).  ``J0`` is the global index of g[0] for
    the Philox counter (so a slice can be checked on its own).

    block = 0 takes one scale for the whole tensor (the PyTorch example's
    max over the tensor); rounding = "nearest" replaces the stochastic draw
    by rounding to the nearest integer, halves away from zero ("FP32 ->
    INT8" step 1)."""
    g = np.asarray(g, dtype=f32).ravel()
    N = g.size
    if block == 0:
        block = N
    if N % block:
        raise ValueError("length must be a multiple of the block")
    gc = g if e is None else (g + np.asarray(e, dtype=f32).ravel()).astype(f32)
    a = np.abs(gc).reshape(-1, block)
    a = np.where(np.isnan(a), f32(0.0), a)
    M = a.max(axis=1).astype(f32)
    M = np.fmax(M, f32(0.0))
    scale = (M / f32(127.0)).astype(f32)
    sc = np.repeat(scale, block)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = (gc / sc).astype(f32)
        if rounding == "nearest":
            q = round_half_away(x)
        else:
            u = uniforms(J0, N, seed, step)
            f = np.floor(x).astype(f32)
            p = (x - f).astype(f32)
            q = (f + np.where(u < p, f32(1.0), f32(0.0))).astype(f32)
        q = np.fmin(np.fmax(q, f32(-127.0)), f32(127.0))
    zero = sc == 0
    q = np.where(zero, f32(0.0), q)
    codes = q.astype(np.int8)
    with np.errstate(invalid="ignore", over="ignore"):
        deq = np.where(zero, f32(0.0), (q * sc).astype(f32)).astype(f32)
        e_new = (gc - deq).astype(f32)
    return {"gc": gc, "codes": codes, "scales": scale, "deq": deq, "e": e_new}
