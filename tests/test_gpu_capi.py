"""The plain C test program (tests/capi/capi_roundtrip.c) on the GPU: one
reset step of compress, server, decompression and Adam through the C ABI
with hipMalloc'd buffers, checked against values derived by hand in the
program (dyadic inputs: every result exact)."""

import os
import subprocess

import pytest

from momentum_compression_amd import build as B

pytestmark = pytest.mark.gpu


def test_c_program_round_trip():
    if not os.path.exists(B.CAPI_BIN):
        pytest.fail("the C test program is not built: run python -m momentum_compression_amd.build")
    print("[capi] running the C program", flush=True)
    res = subprocess.run([B.CAPI_BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip() == "capi ok"
