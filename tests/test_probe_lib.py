"""Host-side checks of the benchmark's probe library (libonebit_probe.so):
it is built next to libonebit.so, exports its five probes, and rejects
invalid sizes before any HIP call (no GPU needed)."""

import ctypes
import os

import pytest

from momentum_compression_amd import build as B

P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.PROBE_LIB):
        pytest.skip("libonebit_probe.so is not built")
    L = ctypes.CDLL(B.PROBE_LIB)
    L.onebit_probe_stream.restype = I32
    L.onebit_probe_stream.argtypes = [P, P, P, P, I64, I32, I32, P]
    L.onebit_probe_server.restype = I32
    L.onebit_probe_server.argtypes = [P, P, P, P, I64, I32, I64, P]
    L.onebit_probe_int8.restype = I32
    L.onebit_probe_int8.argtypes = [P, P, P, P, P, I64, P]
    L.onebit_probe_basic.restype = I32
    L.onebit_probe_basic.argtypes = [P, P, I64, I32, P]
    L.onebit_probe_mix.restype = I32
    L.onebit_probe_mix.argtypes = [P, P, P, P, I64, I32, I32, P]
    return L


def test_probe_sizes_rejected_before_launch(lib):
    # compression probe: N a positive multiple of 64 n, 1 <= n <= 64, mode 0..3
    assert lib.onebit_probe_stream(None, None, None, None, 0, 4, 0, None) == -2
    assert lib.onebit_probe_stream(None, None, None, None, 1000, 4, 0, None) == -2
    assert lib.onebit_probe_stream(None, None, None, None, 4096, 0, 0, None) == -2
    assert lib.onebit_probe_stream(None, None, None, None, 4096, 65, 0, None) == -2
    assert lib.onebit_probe_stream(None, None, None, None, 4096, 4, 4, None) == -2
    assert lib.onebit_probe_stream(None, None, None, None, 4096, 4, -1, None) == -2
    # server probe
    assert lib.onebit_probe_server(None, None, None, None, 0, 16, 0, None) == -2
    assert lib.onebit_probe_server(None, None, None, None, 64 * 16 + 64, 16, 0, None) == -2
    assert lib.onebit_probe_server(None, None, None, None, 4096, 65, 0, None) == -2
    assert lib.onebit_probe_server(None, None, None, None, 4096, 16, 127, None) == -2  # < N/32
    # INT8 probe: N a positive multiple of 256
    assert lib.onebit_probe_int8(None, None, None, None, None, 0, None) == -2
    assert lib.onebit_probe_int8(None, None, None, None, None, 1000, None) == -2
    # plain streams: N a positive multiple of 1024, N / 4 below 2^32, mode 0..3
    assert lib.onebit_probe_basic(None, None, 0, 0, None) == -2
    assert lib.onebit_probe_basic(None, None, 1000, 0, None) == -2
    assert lib.onebit_probe_basic(None, None, 1 << 34, 0, None) == -2
    assert lib.onebit_probe_basic(None, None, 4096, 4, None) == -2
    assert lib.onebit_probe_basic(None, None, 4096, -1, None) == -2
    # read/write mixes: (3, 2) or (4, 3) only, N as above
    assert lib.onebit_probe_mix(None, None, None, None, 4096, 2, 1, None) == -2
    assert lib.onebit_probe_mix(None, None, None, None, 4096, 3, 3, None) == -2
    assert lib.onebit_probe_mix(None, None, None, None, 1000, 3, 2, None) == -2
    assert lib.onebit_probe_mix(None, None, None, None, 1 << 34, 4, 3, None) == -2


def test_probe_library_is_not_the_product_library():
    # the product library exports no probe (the probes are the benchmark's)
    prod = ctypes.CDLL(os.path.join(os.path.dirname(B.PROBE_LIB), "libonebit.so"))
    for name in ("onebit_probe_stream", "onebit_probe_server", "onebit_probe_int8",
                 "onebit_probe_basic", "onebit_probe_mix"):
        assert not hasattr(prod, name)
