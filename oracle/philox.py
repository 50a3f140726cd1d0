"""Philox4x32-10 counter-based generator.

Definition from Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3" (SC'11), section 4 (the Philox S-box): a 4-word counter and a
2-word key; each of 10 rounds multiplies words 0 and 2 by two fixed 32-bit
constants, forms the new words from the high halves xored with the other
words and the round key and from the low halves, and the key is bumped by two
Weyl constants (golden ratio and sqrt(3) - 1, scaled to 32 bits) between
rounds.

The INT8 stochastic rounding of the gradient-quantisation tutorial ("FP32 ->
INT8", stochastic rounding; PyTorch example) draws one uniform per element.
Here element J uses counter (J>>2 low word, J>>2 high word, step, 0) and key
(seed low word, seed high word); output word J&3, shifted right by 8, times
2^-24, is the uniform in [0, 1).

Pin: rocRAND's Philox4x32-10 engine, an independent implementation, compiled
on the host (tests/test_oracle_philox.py).
"""

from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """ctr: uint32 [..., 4]; key: uint32 [..., 2] (broadcastable).
    Returns uint32 [..., 4]."""
    x = np.asarray(ctr, dtype=np.uint32).astype(np.uint64)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint32), x.shape[:-1] + (2,)).astype(np.uint64)
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & _MASK
            k1 = (k1 + W1) & _MASK
        p0 = M0 * x0  # < 2^64, exact in uint64
        p1 = M1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def uniforms(J0: int, count: int, seed: int, step: int) -> np.ndarray:
    """Uniforms u_J for J = J0 .. J0+count-1 (float32, multiples of 2^-24)."""
    J = np.arange(J0, J0 + count, dtype=np.uint64)
    blk = J >> np.uint64(2)
    ctr = np.stack([blk & _MASK, blk >> np.uint64(32),
                    np.full_like(blk, np.uint64(step) & _MASK), np.zeros_like(blk)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    words = philox4x32_10(ctr.astype(np.uint32), key)
    w = words[np.arange(count), (J & np.uint64(3)).astype(np.int64)]
    return ((w >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)
