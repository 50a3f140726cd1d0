"""Sign bits and their packing into 32-bit words.

The 1-bit Adam article (section 3.1, sign aggregation) packs the sign of each
gradient element into bits before communication.  Convention used here:
bit = 1 for x >= 0 (so sign(0) = +1 for both zeros), bit = 0 for x < 0 and
for NaN; element j lands in word j >> 5 at bit position j & 31
(least-significant bit first).

Pins: numpy.packbits(..., bitorder='little') viewed as little-endian uint32,
and round trips (tests/test_oracle_bits.py).
"""

from __future__ import annotations

import numpy as np


def sign_bit(x: np.ndarray) -> np.ndarray:
    """bool array: True where x >= 0 (+1), False where x < 0 or NaN (-1)."""
    return np.asarray(x) >= 0


def pack(b: np.ndarray) -> np.ndarray:
    """Pack a bool vector (length a multiple of 32) into uint32 words."""
    b = np.asarray(b, dtype=bool).ravel()
    if b.size % 32:
        raise ValueError("bit count must be a multiple of 32")
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    words = (b.reshape(-1, 32).astype(np.uint64) * weights).sum(axis=1)
    return words.astype(np.uint32)


def unpack(words: np.ndarray, count: int | None = None) -> np.ndarray:
    """Inverse of ``pack``: bool vector of 32 * len(words) (or ``count``)."""
    w = np.asarray(words, dtype=np.uint32).ravel()
    pos = np.arange(32, dtype=np.uint32)
    b = ((w[:, None] >> pos[None, :]) & np.uint32(1)).astype(bool).ravel()
    return b if count is None else b[:count]


def signed(b: np.ndarray, s: np.float32) -> np.ndarray:
    """The scaled sign q = s * sign: +s where the bit is set, -s elsewhere."""
    s = np.float32(s)
    return np.where(b, s, -s).astype(np.float32)
