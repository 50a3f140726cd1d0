"""Worker and server sides of error-compensated 1-bit compression.

Sources:
* 1-bit Adam article, section 2.1 (error compensation): the compensated value
  g' = g + e_prev, the 1-bit quantisation q = sign(g') and the new error
  e = g' - q.  Here, as in 1-bit LAMB, the compressed quantity is the
  momentum (1-bit LAMB page, layer-scaling paragraph: the local momentum is
  what is compressed and communicated).
* gradient-quantisation tutorial, "1-bit gradient quantisation": the scaled
  sign mean(|g'|) * sign(g') and error feedback.  The scale is taken per
  chunk of the fused buffer (one chunk per worker, each chunk owned by one
  server rank).
* 1-bit Adam article, section 4.1 (convergence fixes, code example): the
  periodic error reset (before compensation) and the clamp of the
  compensated value.
* 1-bit LAMB page, layer-scaling paragraph: the fixed per-layer coefficient
  multiplies the local momentum before compression and divides the global
  compressed momentum after it.
* 1-bit LAMB page, experiments paragraph: the compressed backend's two phases
  -- each worker's chunk c goes to server c (all-to-all), which averages the
  n chunks, error-compensates and re-compresses them; every worker then
  receives all server chunks (all-gather) and decompresses.

Readings where the pages are silent (the same ones the HIP path follows):
* chunk = N / n consecutive elements of a worker row; scale s[i][c] is the
  exact mean |g'| of worker i's chunk c, rounded once to binary32;
* the server keeps its own error buffer, reset at the same steps as the
  worker errors; the clamp applies to the worker's compensated value only;
* the server average sums the n decoded chunks in ascending worker order in
  binary32, starting from +0, then divides by n;
* clamp(x) = fmin(fmax(x, -clip), clip), so NaN becomes -clip;
* the step-ratio factor of the 1-bit LAMB analysis multiplies the carried
  error of both levels (worker and server) by the factor of its layer, so
  that the two-level momentum identity keeps the ratio.

Parity pins (tests/test_oracle_onebit.py): brute force with Fractions on tiny
inputs, the error identity, exact telescoping of the error feedback on dyadic
inputs, optimality of the mean-|.| scale, |e| <= clip, the n = 1 and
unanimous-sign server cases, and the two-level momentum identity.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import bits as B
from .exact import mean_abs_f32

f32 = np.float32


def clamp(x: np.ndarray, clip: float) -> np.ndarray:
    """fmin(fmax(x, -clip), clip); clip <= 0 or inf disables it."""
    c = f32(clip)
    if not (c > 0) or np.isinf(c):
        return x
    return np.fmin(np.fmax(x, -c), c).astype(f32)


def error_from(gc: np.ndarray, s: np.float32) -> np.ndarray:
    """e = g' - q with q = s * sign(g'), one binary32 rounding."""
    s = f32(s)
    return np.where(B.sign_bit(gc), gc - s, gc + s).astype(f32)


def worker_compress(m: np.ndarray, e: np.ndarray, clip: float = 0.0,
                    reset: bool = False, k: Optional[np.ndarray] = None,
                    unit_scale: bool = False,
                    err_ratio: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One worker-side compression of all n workers.

    m, e : float32 [n, N] momentum and carried error (N a multiple of 64 n)
    k    : optional float32 [N] per-element layer coefficient (x k before
           compensation)
    unit_scale : the unscaled 1-bit sign q = +-1 of the 1-bit Adam article,
           section 2.1 (s = 1 instead of the chunk mean)
    err_ratio : optional float32 [N] per-element factor on the carried error,
           the step-ratio-scaled error feedback of the 1-bit LAMB page
           (analysis paragraph: the error is multiplied by c_{t-2}/c_{t-1}
           of its layer before it is added)
    Returns gc (compensated, clamped) [n, N], bits uint32 [n, N/32],
    s float32 [n, n] (s[i][c] for worker i, chunk c) and the new error
    e [n, N]."""
    m = np.asarray(m, dtype=f32)
    n, N = m.shape
    if N % (64 * n):
        raise ValueError("N must be a multiple of 64 n")
    L = N // n
    e_in = np.zeros_like(m) if reset else np.asarray(e, dtype=f32)
    if err_ratio is not None and not reset:
        e_in = (np.asarray(err_ratio, dtype=f32)[None, :] * e_in).astype(f32)
    gc = np.empty_like(m)
    e_out = np.empty_like(m)
    s = np.empty((n, n), dtype=f32)
    bits = np.empty((n, N // 32), dtype=np.uint32)
    for i in range(n):
        mi = m[i] if k is None else (np.asarray(k, dtype=f32) * m[i]).astype(f32)
        gi = clamp((mi + e_in[i]).astype(f32), clip)
        gc[i] = gi
        for c in range(n):
            sl = slice(c * L, (c + 1) * L)
            s[i, c] = f32(1.0) if unit_scale else mean_abs_f32(gi[sl])
            e_out[i, sl] = error_from(gi[sl], s[i, c])
        bits[i] = B.pack(B.sign_bit(gi))
    return {"gc": gc, "bits": bits, "s": s, "e": e_out}


def server_chunk(bits_c: np.ndarray, s_c: np.ndarray, E_c: np.ndarray,
                 reset: bool = False, unit_scale: bool = False,
                 err_ratio_c: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Server side of one chunk.

    bits_c : uint32 [n, L/32] -- this chunk's sign words of every worker
    s_c    : float32 [n]      -- this chunk's scale of every worker
    E_c    : float32 [L]      -- the server error of this chunk
    The decoded values +-s_c[i] are summed in ascending worker order in
    binary32 from +0, then divided by n once; the server error is added and
    the result compressed like a worker chunk."""
    bits_c = np.asarray(bits_c, dtype=np.uint32)
    s_c = np.asarray(s_c, dtype=f32)
    n = s_c.shape[0]
    L = bits_c.shape[1] * 32
    acc = np.zeros(L, dtype=f32)
    for i in range(n):
        acc = (acc + B.signed(B.unpack(bits_c[i]), s_c[i])).astype(f32)
    avg = (acc / f32(n)).astype(f32)
    E_in = np.zeros(L, dtype=f32) if reset else np.asarray(E_c, dtype=f32)
    if err_ratio_c is not None and not reset:
        E_in = (np.asarray(err_ratio_c, dtype=f32) * E_in).astype(f32)
    g2 = (avg + E_in).astype(f32)
    S = f32(1.0) if unit_scale else mean_abs_f32(g2)
    return {"avg": avg, "g2": g2, "bits": B.pack(B.sign_bit(g2)), "S": S,
            "E": error_from(g2, S)}


def server_reduce(bits: np.ndarray, s: np.ndarray, E: np.ndarray,
                  reset: bool = False, unit_scale: bool = False,
                  err_ratio: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Server side for every chunk c (server rank c).

    bits : uint32 [n, N/32] worker sign words; s : float32 [n, n] worker scales
    E    : float32 [N] server error (chunk c owned by server c)
    Returns avg [N], g2 (compensated) [N], bits uint32 [N/32], S float32 [n]
    and the new server error E [N]."""
    bits = np.asarray(bits, dtype=np.uint32)
    s = np.asarray(s, dtype=f32)
    n = s.shape[0]
    N = bits.shape[1] * 32
    L = N // n
    out = {"avg": np.empty(N, dtype=f32), "g2": np.empty(N, dtype=f32),
           "E": np.empty(N, dtype=f32), "S": np.empty(n, dtype=f32),
           "bits": np.empty(N // 32, dtype=np.uint32)}
    E = np.zeros(N, dtype=f32) if reset else np.asarray(E, dtype=f32)
    for c in range(n):
        sl = slice(c * L, (c + 1) * L)
        r = server_chunk(bits[:, c * L // 32:(c + 1) * L // 32], s[:, c], E[sl], reset,
                         unit_scale, None if err_ratio is None else np.asarray(err_ratio)[sl])
        for key in ("avg", "g2", "E"):
            out[key][sl] = r[key]
        out["S"][c] = r["S"]
        out["bits"][c * L // 32:(c + 1) * L // 32] = r["bits"]
    return out


def decompress(sbits: np.ndarray, S: np.ndarray, k: Optional[np.ndarray] = None) -> np.ndarray:
    """Global momentum every worker reconstructs: +S[c] / -S[c] per bit of
    chunk c; divided by the layer coefficient k (per element) when given."""
    S = np.asarray(S, dtype=f32)
    n = S.shape[0]
    b = B.unpack(sbits)
    N = b.size
    L = N // n
    out = np.empty(N, dtype=f32)
    for c in range(n):
        sl = slice(c * L, (c + 1) * L)
        out[sl] = B.signed(b[sl], S[c])
    if k is not None:
        out = (out / np.asarray(k, dtype=f32)).astype(f32)
    return out


def local_momentum(g: np.ndarray, mbar_prev: np.ndarray, beta1: float) -> np.ndarray:
    """Each worker's momentum from its gradient and the previous global
    momentum (1-bit Adam article, section 2.1: m_t = beta1 m_{t-1} +
    (1 - beta1) g_t; the previous momentum is the decompressed global one,
    identical on every worker): fl(fl(beta1 m) + fl((1 - beta1) g)) with
    1 - beta1 rounded once.  g: [n, N]; mbar_prev: [N]."""
    b1 = f32(beta1)
    omb1 = f32(f32(1.0) - b1)
    a = (b1 * np.asarray(mbar_prev, dtype=f32)).astype(f32)
    return (a[None, :] + (omb1 * np.asarray(g, dtype=f32)).astype(f32)).astype(f32)


def layer_scale(buf: np.ndarray, seg_off, k: np.ndarray, divide: bool) -> np.ndarray:
    """Segment-wise x * k_l (or x / k_l) over the last axis of ``buf``."""
    buf = np.asarray(buf, dtype=f32)
    out = np.empty_like(buf)
    k = np.asarray(k, dtype=f32)
    for l in range(len(seg_off) - 1):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        out[..., a:b] = (buf[..., a:b] / k[l]) if divide else (buf[..., a:b] * k[l])
    return out


def per_element_k(seg_off, k: np.ndarray) -> np.ndarray:
    """Expand per-segment coefficients to one per element."""
    k = np.asarray(k, dtype=f32)
    sizes = np.diff(np.asarray(seg_off, dtype=np.int64))
    return np.repeat(k, sizes).astype(f32)
