"""Pin of the oracle's Philox4x32-10 (oracle/philox.py) against rocRAND's
Philox4x32-10 engine, an independent implementation shipped as source in the
ROCm headers, compiled here for the host (no GPU is touched).

rocRAND's engine initialised with (seed, subsequence, offset) uses key =
seed and counter words (offset/4 low, offset/4 high, subsequence low,
subsequence high), starting at word offset % 4; so the oracle's uniform for
element J at step t is word 0 of rocRAND's output at (seed, t, J).
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle.philox import philox4x32_10, uniforms

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "xcheck", "rocrand_philox.cpp")


def build_rocrand_dump():
    """Compile the rocRAND cross-check for the host; returns a function from
    (seed, subsequence, offset) triples to rocRAND's output words, or None
    when hipcc is not available."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        return None
    out = os.path.join(tempfile.mkdtemp(prefix="philox_xcheck_"), "rocrand_philox")
    subprocess.run([hipcc, "-O1", "-o", out, SRC], check=True, capture_output=True, timeout=300)

    def run(triples):
        text = "".join(f"{s} {q} {o}\n" for s, q, o in triples)
        res = subprocess.run([out], input=text, capture_output=True, text=True, check=True, timeout=120)
        return np.array([[int(w, 16) for w in line.split()] for line in res.stdout.splitlines()],
                        dtype=np.uint64).astype(np.uint32)

    return run


@pytest.fixture(scope="module")
def rocrand_dump():
    run = build_rocrand_dump()
    if run is None:
        pytest.skip("hipcc not available to build the rocRAND cross-check")
    return run


def test_raw_blocks_match_rocrand(rocrand_dump):
    rng = np.random.default_rng(0)
    triples, ctrs, keys = [], [], []
    for _ in range(500):
        seed = int(rng.integers(0, 2**63))
        sub = int(rng.integers(0, 2**63))
        blk = int(rng.integers(0, 2**62))
        triples.append((seed, sub, 4 * blk))
        ctrs.append([blk & 0xFFFFFFFF, blk >> 32, sub & 0xFFFFFFFF, sub >> 32])
        keys.append([seed & 0xFFFFFFFF, seed >> 32])
    want = rocrand_dump(triples)
    c32 = np.array(ctrs, dtype=np.uint64).astype(np.uint32)
    k32 = np.array(keys, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(philox4x32_10(c32, k32), want)
    from oracle import cref

    got_cpp = np.stack([cref.philox4x32_10(c32[i], k32[i])[0] for i in range(len(c32))])
    assert np.array_equal(got_cpp, want)  # the C++ oracle's generator, pinned the same way


def test_element_uniforms_match_rocrand(rocrand_dump):
    rng = np.random.default_rng(1)
    for _ in range(5):
        seed = int(rng.integers(0, 2**40))
        step = int(rng.integers(0, 1000))
        J0 = int(rng.integers(0, 2**33))
        count = 37
        want = rocrand_dump([(seed, step, J0 + j) for j in range(count)])[:, 0]
        u = uniforms(J0, count, seed, step)
        expect = ((want >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)
        assert np.array_equal(u, expect)
        from oracle import cref

        assert np.array_equal(cref.uniforms(J0, count, seed, step), expect)
