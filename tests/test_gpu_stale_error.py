"""An error that an earlier HIP call left on the calling thread is not taken
for a failure of the library's own launches: every entry point drops it
before it launches, so its status reflects only its own work.

The stale error is made on the host: hipSetDevice with an ordinal that no
machine has is refused, leaves the current device as it was, and leaves
hipErrorInvalidDevice as the thread's last error.  No kernel is involved.
Nothing else runs between that call and the library call (torch's own
launch checks would report the error first)."""

import ctypes

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import OneBitGroup
from oracle import int8 as I
from oracle import onebit as O
from oracle import optim as P
from tests._gpu import device, gen, host

pytestmark = pytest.mark.gpu


def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipPeekAtLastError.restype = ctypes.c_int
    return hip


def _leave_stale_error(hip) -> None:
    assert hip.hipSetDevice(1 << 20) != 0
    assert hip.hipPeekAtLastError() != 0


def test_stale_thread_error_does_not_fail_the_step():
    hip = _hip()
    dev = device()
    N, n = 4 * 3136, 4  # chunks of 3 tiles and a ragged 64
    print(f"[stale error] N={N} n={n}", flush=True)
    grp = OneBitGroup(N, n, dev)
    g = gen(4711, dev)
    m = torch.randn((n, N), generator=g, device=dev) * 1e-3
    x = torch.randn(N, generator=g, device=dev) * 0.02
    v = torch.rand(N, generator=g, device=dev) * 1e-6 + 1e-8
    x_h, v_h = host(x).copy(), host(v)
    gg = torch.randn(256 * 40, generator=g, device=dev) * 1e-3
    codes = torch.empty(gg.numel(), dtype=torch.int8, device=dev)
    sc = torch.empty(40, device=dev)
    torch.cuda.synchronize()

    _leave_stale_error(hip)
    grp.compress(m, 1, first=True)
    _leave_stale_error(hip)
    grp.server(1, first=True, decompress=False)
    _leave_stale_error(hip)
    grp.adam_step_packed(x, v, 6e-5, 1e-6, decompress=True)
    _leave_stale_error(hip)
    ob.int8_sr_quantize(gg, None, codes, sc, None, gg.numel(), 256, 99, 1)
    assert hip.hipPeekAtLastError() == 0  # the last entry point took the stale error away
    torch.cuda.synchronize()

    w = O.worker_compress(host(m), np.zeros((n, N), np.float32), reset=True)
    sv = O.server_reduce(w["bits"], w["s"], np.zeros(N, np.float32), reset=True)
    mbar = O.decompress(sv["bits"], sv["S"])
    x_h = P.adam_frozen_step(x_h, mbar, v_h, 6e-5, 1e-6)
    assert np.array_equal(host(grp.bits), w["bits"])
    assert np.array_equal(host(grp.scales).view(np.uint32), w["s"].view(np.uint32))
    assert np.array_equal(host(grp.sv_bits), sv["bits"])
    assert np.array_equal(host(grp.sv_scales).view(np.uint32), sv["S"].view(np.uint32))
    assert np.array_equal(host(grp.mbar).view(np.uint32), mbar.view(np.uint32))
    assert np.array_equal(host(x).view(np.uint32), x_h.view(np.uint32))
    o = I.int8_sr(host(gg), None, 99, 1, 256)
    assert np.array_equal(host(codes), o["codes"])
    assert np.array_equal(host(sc).view(np.uint32), o["scales"].view(np.uint32))
