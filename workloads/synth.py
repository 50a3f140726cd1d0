"""Seeded synthetic inputs (torch; CPU or device).

Recipes follow the workload descriptions: momentum ~ N(0, sigma) with sigma
fixed per segment (per 2^20-element block, or per tensor) and drawn once,
log-uniformly, from the workload's range; a fresh momentum draw per (worker,
step); frozen variance |N(0, 1e-6)| + 1e-8; parameters N(0, 0.02); INT8
gradients Laplace(0, 1e-3) with a 1e-4 share of x100 outliers.  The pad
segment of a padded buffer is all zero momentum, unit variance, unit
coefficients.

Nothing here computes any step of the compression method; the outputs are
handed unchanged to both the HIP path and the CPU oracle.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np
import torch

from .configs import Workload

# stream tags keep the draws of different tensors independent
TAG_SIGMA, TAG_M, TAG_V, TAG_X, TAG_G, TAG_MPREV, TAG_CAVG = range(7)


def _gen(seed: int, tag: int, step: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 7919 + step * 104_729) & 0x7FFF_FFFF_FFFF)
    return g


def _range_of(mode: str) -> Tuple[float, float]:
    if mode == "loguniform_1e-5_1e-2":
        return 1e-5, 1e-2
    if mode == "loguniform_1e-6_1e-1":
        return 1e-6, 1e-1
    raise ValueError(mode)


def segment_sigmas(wl: Workload) -> np.ndarray:
    """One standard deviation per segment (float64), drawn once from the
    workload seed.  A trailing pad segment gets sigma 0."""
    nseg = len(wl.segments)
    if wl.sigma_mode == "const1e-3":
        sig = np.full(nseg, 1e-3)
    else:
        lo, hi = _range_of(wl.sigma_mode)
        rng = np.random.Generator(np.random.Philox(key=wl.seed * 31 + TAG_SIGMA))
        sig = np.exp(rng.uniform(math.log(lo), math.log(hi), size=nseg))
    if wl.pad:
        sig[-1] = 0.0
    return sig


def per_element(values: np.ndarray, wl: Workload, device, dtype=torch.float32) -> torch.Tensor:
    """Expand one value per segment into an [N] tensor."""
    counts = torch.tensor(wl.segments, dtype=torch.int64, device=device)
    v = torch.tensor(values, dtype=dtype, device=device)
    return torch.repeat_interleave(v, counts)


def momentum(wl: Workload, step: int, device="cpu", rows: Optional[int] = None,
             sigma_elem: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None
             ) -> torch.Tensor:
    """Worker momentum draw for one step: float32 [rows, N], rows defaults
    to the worker count.  ``out`` may pass a preallocated buffer."""
    rows = wl.n if rows is None else rows
    if sigma_elem is None:
        sigma_elem = per_element(segment_sigmas(wl), wl, device)
    if out is None:
        out = torch.empty((rows, wl.N), dtype=torch.float32, device=device)
    g = _gen(wl.seed, TAG_M, step, device)
    for r in range(rows):
        out[r].normal_(0.0, 1.0, generator=g)
        out[r].mul_(sigma_elem)
    return out


def frozen_variance(wl: Workload, device="cpu") -> torch.Tensor:
    g = _gen(wl.seed, TAG_V, 0, device)
    v = torch.empty(wl.N, dtype=torch.float32, device=device)
    v.normal_(0.0, 1e-6, generator=g).abs_().add_(1e-8)
    if wl.pad:
        v[wl.N - wl.pad:] = 1.0
    return v


def params(wl: Workload, device="cpu") -> torch.Tensor:
    g = _gen(wl.seed, TAG_X, 0, device)
    x = torch.empty(wl.N, dtype=torch.float32, device=device)
    x.normal_(0.0, 0.02, generator=g)
    if wl.pad:
        x[wl.N - wl.pad:] = 0.0
    return x


def lamb_c_avg(wl: Workload) -> np.ndarray:
    """Per-segment warmup averages c_avg of LAMB's layer coefficient
    (float32), log-uniform in [0.5, 2]; the pad segment gets 1."""
    rng = np.random.Generator(np.random.Philox(key=wl.seed * 31 + TAG_CAVG))
    c_avg = np.exp(rng.uniform(math.log(0.5), math.log(2.0),
                               size=len(wl.segments))).astype(np.float32)
    if wl.pad:
        c_avg[-1] = 1.0
    return c_avg


def lamb_tables(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Per-segment fixed momentum coefficients k and warmup averages c_avg
    (float32) for the small tests.  k is the reciprocal of the segment's
    generating sigma, the coefficient that brings the segment to unit scale
    (a stand-in for the coefficient from the warmup momentum, which the
    full-size runs take from ``lamb_prev_momentum`` with the library's
    momentum scale); the pad segment gets k = 1."""
    sig = segment_sigmas(wl)
    k = np.ones(len(sig), dtype=np.float32)
    nz = sig > 0
    k[nz] = (1.0 / sig[nz]).astype(np.float32)
    return k, lamb_c_avg(wl)


def lamb_prev_momentum(wl: Workload, device="cpu", sigma_elem=None) -> torch.Tensor:
    """The global momentum at the end of warmup, m_Tw: N(0, sigma_l) per
    segment.  It is the previous momentum of the first compressed LAMB step
    and the momentum the per-layer coefficients k_l are taken from."""
    if sigma_elem is None:
        sigma_elem = per_element(segment_sigmas(wl), wl, device)
    g = _gen(wl.seed, TAG_MPREV, 0, device)
    m = torch.empty(wl.N, dtype=torch.float32, device=device)
    m.normal_(0.0, 1.0, generator=g).mul_(sigma_elem)
    return m


def laplace_gradient(N: int, step: int, seed: int, device="cpu", b: float = 1e-3,
                     outlier_p: float = 1e-4, outlier_x: float = 100.0,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Laplace(0, b) gradient with independent x100 outliers (prob 1e-4)."""
    g = _gen(seed, TAG_G, step, device)
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=device)
    piece = 1 << 26
    for a in range(0, N, piece):
        z = min(piece, N - a)
        u = torch.rand(z, generator=g, device=device, dtype=torch.float64) - 0.5
        lap = -b * torch.sign(u) * torch.log1p(-2.0 * u.abs())
        o = torch.rand(z, generator=g, device=device) < outlier_p
        lap = torch.where(o, lap * outlier_x, lap)
        out[a:a + z] = lap.to(torch.float32)
    return out
