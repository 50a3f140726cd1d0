"""Pins of the oracle's sign-bit packing (oracle/bits.py) against numpy."""

import numpy as np

from oracle import bits as B


def test_pack_matches_numpy_packbits_little():
    rng = np.random.default_rng(0)
    for n in (32, 64, 96, 1024, 32 * 77):
        b = rng.random(n) < 0.5
        want = np.packbits(b, bitorder="little").view("<u4")
        assert np.array_equal(B.pack(b), want)


def test_pack_unpack_exhaustive_16bit_windows():
    pats = np.arange(1 << 16, dtype=np.uint32)
    for shift in (0, 5, 16):
        words = (pats << np.uint32(shift)).astype(np.uint32)
        b = B.unpack(words)
        assert np.array_equal(B.pack(b), words)
        # bit j of word w is element 32 w + j
        bb = b.reshape(-1, 32)
        for j in range(16):
            assert np.array_equal(bb[:, shift + j], ((pats >> j) & 1).astype(bool))


def test_sign_convention():
    x = np.array([0.0, -0.0, 1e-45, -1e-45, np.inf, -np.inf, np.nan, 3.0], dtype=np.float32)
    assert list(B.sign_bit(x)) == [True, True, True, False, True, False, False, True]
    q = B.signed(B.sign_bit(x), np.float32(0.5))
    assert list(q) == [0.5, 0.5, 0.5, -0.5, 0.5, -0.5, -0.5, 0.5]
