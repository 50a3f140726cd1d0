"""C ABI checks that need no GPU: the library loads, exports every function
include/onebit.h declares, sizes its workspace, and rejects invalid calls
with the documented status before touching the HIP runtime (the fake
device addresses below are never dereferenced)."""

import ctypes

import pytest

from momentum_compression_amd import onebit as ob

P = 0x10000  # a 16-byte aligned fake device address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return ob.load()


def test_every_declared_symbol_is_exported(lib):
    names = ob.declared_functions()
    assert {"onebit_compress", "onebit_server_reduce", "lamb_layer_scale", "frozen_v_step",
            "int8_sr_quantize", "onebit_workspace_bytes", "frozen_v_workspace_bytes",
            "onebit_strerror"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_strerror_covers_codes(lib):
    for code in range(0, -7, -1):
        assert ob.strerror(code) != "unknown status"
    assert ob.strerror(-99) == "unknown status"


def test_workspace_bytes(lib):
    assert ob.workspace_bytes(1 << 20, 4) > 0
    assert ob.workspace_bytes(1000, 4) == 0           # not a multiple of 64 n
    assert ob.workspace_bytes(1 << 20, 0) == 0
    assert ob.workspace_bytes(1 << 20, 65) == 0
    # one binary64 partial per workgroup of the compression (one 1024-element
    # tile each, 16 x 16 chunks of 81,970,560) dominates: 80,049 x 256 x 8 B
    big = ob.workspace_bytes(1_311_528_960, 16, 291)
    assert 80_049 * 256 * 8 <= big < 80_049 * 256 * 8 + (1 << 20)


def test_frozen_v_workspace_bytes(lib):
    # layer keys (rounded to 256 bytes) + one 4-byte slot per 4096 elements
    assert ob.frozen_v_workspace_bytes(4096 * 300 - 16, 8) == 256 + 1280
    assert ob.frozen_v_workspace_bytes(336_226_304, 303) == 1280 + 328_448
    assert ob.frozen_v_workspace_bytes(0, 1) == 256
    assert ob.frozen_v_workspace_bytes(1022, 4) == 0
    assert ob.frozen_v_workspace_bytes(1024, 0) == 0


def _compress(lib, m=P, ef=P, sc=P, bits=P, N=1 << 12, n=4, clip=0.0, off=None, k=None, nseg=0,
              ws=P, wsb=1 << 30):
    return lib.onebit_compress(m, ef, sc, bits, N, n, clip, 0, off, k, nseg, ws, wsb, None)


def test_compress_validation(lib):
    assert _compress(lib, m=None) == ob.ONEBIT_E_NULL
    assert _compress(lib, N=4 * 63) == ob.ONEBIT_E_SIZE
    assert _compress(lib, n=0) == ob.ONEBIT_E_SIZE
    assert _compress(lib, n=65, N=65 * 64) == ob.ONEBIT_E_SIZE
    assert _compress(lib, N=-64 * 4) == ob.ONEBIT_E_SIZE
    assert _compress(lib, m=P + 4) == ob.ONEBIT_E_ALIGN
    assert _compress(lib, ws=None) == ob.ONEBIT_E_WORKSPACE
    assert _compress(lib, wsb=16) == ob.ONEBIT_E_WORKSPACE
    assert _compress(lib, ws=P + 16) == ob.ONEBIT_E_ALIGN
    assert _compress(lib, off=P) == ob.ONEBIT_E_NULL         # offsets without coefficients
    assert _compress(lib, off=P, k=P, nseg=0) == ob.ONEBIT_E_ARG
    assert _compress(lib, clip=float("nan")) == ob.ONEBIT_E_ARG
    assert _compress(lib, N=0) == ob.ONEBIT_OK              # empty: no-op, no launch


def test_server_and_other_validation(lib):
    f = lib.onebit_server_reduce
    assert f(None, P, P, P, P, None, None, None, 0, 1 << 12, 4, 0, P, 1 << 30, None) == ob.ONEBIT_E_NULL
    assert f(P, P, P, P, P, P + 4, None, None, 0, 1 << 12, 4, 0, P, 1 << 30, None) == ob.ONEBIT_E_ALIGN
    assert f(P, P, P, P, P, None, None, None, 0, 100, 4, 0, P, 1 << 30, None) == ob.ONEBIT_E_SIZE
    assert f(P, P, P, P, P, None, None, None, 0, 1 << 12, 4, 0, P, 8, None) == ob.ONEBIT_E_WORKSPACE
    assert lib.onebit_decompress(P, P, None, None, None, 0, 1 << 12, 4, None) == ob.ONEBIT_E_NULL
    assert lib.onebit_error_materialize(P, P, P, 1 << 12, 0, 4, None) == ob.ONEBIT_E_SIZE
    assert lib.lamb_layer_scale(P, 1 << 12, 1, P, P, 0, 0, None) == ob.ONEBIT_E_ARG
    assert lib.lamb_layer_scale(P, 6, 1, P, P, 1, 0, None) == ob.ONEBIT_E_SIZE
    i8 = lib.int8_sr_quantize
    assert i8(P, None, P, P, None, 1 << 12, 100, 1, 1, None) == ob.ONEBIT_E_SIZE
    assert i8(P, None, P, P, None, 256 * 3 + 64, 256, 1, 1, None) == ob.ONEBIT_E_SIZE
    assert i8(P, P + 8, P, P, None, 256, 256, 1, 1, None) == ob.ONEBIT_E_ALIGN
    assert i8(None, None, P, P, None, 256, 256, 1, 1, None) == ob.ONEBIT_E_NULL


def test_server_noalloc_validation(lib):
    """The allocation-free server refuses what the workspace form refuses,
    with the same codes, and refuses sizes whose partial sums would not fit
    its fixed 2^20-double scratch with ONEBIT_E_WORKSPACE, all before any
    HIP call (N = 0 is a no-op)."""
    f = lib.onebit_server_reduce_noalloc

    def call(bits=P, sc=P, ef=P, svs=P, svb=P, m=None, off=None, k=None, r=None, nseg=0,
             N=1 << 12, n=4, reset=0, flags=0):
        return f(bits, sc, ef, svs, svb, m, off, k, r, nseg, N, n, reset, flags, None)

    assert call(bits=None) == ob.ONEBIT_E_NULL
    assert call(m=P + 4) == ob.ONEBIT_E_ALIGN
    assert call(N=100) == ob.ONEBIT_E_SIZE
    assert call(n=65, N=65 * 64) == ob.ONEBIT_E_SIZE
    assert call(flags=4) == ob.ONEBIT_E_ARG
    assert call(r=P) == ob.ONEBIT_E_ARG          # a step-ratio factor needs a layer table
    assert call(off=P, k=None, nseg=2) == ob.ONEBIT_E_NULL
    assert call(N=0) == ob.ONEBIT_OK
    # n <= 8: one partial per 2048 elements, so 2^20 of them end at N = 2^31
    # (sizes that fit are not called here: they would launch)
    assert call(N=(1 << 31) + 8 * 2048, n=8) == ob.ONEBIT_E_WORKSPACE
    # n > 8: one partial per 8192 elements
    assert call(N=(1 << 33) + 16 * 8192 * 64, n=16) == ob.ONEBIT_E_WORKSPACE


def test_compress_grad_validation(lib):
    f = lib.onebit_compress_grad
    args = [P, P, P, 0.9, P, P, P, 1 << 12, 4, 0.0, 0, None, None, 0, P, 1 << 30, None]
    bad = list(args); bad[1] = None
    assert f(*bad) == ob.ONEBIT_E_NULL
    bad = list(args); bad[3] = float("nan")
    assert f(*bad) == ob.ONEBIT_E_ARG
    bad = list(args); bad[0] = P + 4
    assert f(*bad) == ob.ONEBIT_E_ALIGN
    bad = list(args); bad[14] = None
    assert f(*bad) == ob.ONEBIT_E_WORKSPACE


def test_frozen_v_validation(lib):
    a = ob.FrozenVArgs(mode=0, N=1024, x=P, m=P, v=None, lr=1e-3, eps=1e-6)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL
    a = ob.FrozenVArgs(mode=4, N=1024, x=P, m=P, v=P)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_ARG
    a = ob.FrozenVArgs(mode=1, N=1024, x=P, m=P, v=P, m_prev=P, v_fresh=P, seg_off=P, c_avg=P,
                       r_prev=P, c_prev=P, n_seg=4)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_WORKSPACE
    a.n_seg = 0
    assert lib.frozen_v_step(ctypes.byref(a), P, 1 << 20, None) == ob.ONEBIT_E_ARG
    a = ob.FrozenVArgs(mode=2, N=1024, x=P, m=None, v=P, m_bits=None, m_scales=P, m_chunks=4)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL
    a = ob.FrozenVArgs(mode=2, N=1024 + 64, x=P, m=None, v=P, m_bits=P, m_scales=P, m_chunks=4)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_SIZE
    a = ob.FrozenVArgs(mode=2, N=1024, x=P, m=None, v=P, m_bits=P, m_scales=P, m_chunks=4,
                       m_out=P + 4)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_ALIGN
    lamb = dict(mode=3, N=1024, x=P, m=None, v=P, m_prev=P, v_fresh=P, seg_off=P, c_avg=P,
                r_prev=P, c_prev=P, n_seg=4, m_bits=P, m_scales=P, m_chunks=4, m_seg_k=P)
    a = ob.FrozenVArgs(**{**lamb, "m_seg_k": None})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL
    a = ob.FrozenVArgs(**{**lamb, "use_c_t": 1})          # the second pass reads m_out
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL
    a = ob.FrozenVArgs(**{**lamb, "m_chunks": 3})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_SIZE
    a = ob.FrozenVArgs(**{**lamb, "m_out": P + 64})       # overlaps m_prev
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_ARG
    a = ob.FrozenVArgs(**{**lamb, "m_out": P + 4 * 1024})  # adjacent: accepted up to the workspace
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_WORKSPACE
    # m_{t-1} packed: words and scales both or neither; m_prev then not needed
    a = ob.FrozenVArgs(**{**lamb, "mp_bits": P})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL
    a = ob.FrozenVArgs(**{**lamb, "m_prev": None})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL
    a = ob.FrozenVArgs(**{**lamb, "m_prev": None, "mp_bits": P, "mp_scales": P})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_WORKSPACE
    a = ob.FrozenVArgs(**{**lamb, "m_prev": None, "mp_bits": P + 2, "mp_scales": P})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_ALIGN
    a = ob.FrozenVArgs(**{**lamb, "m_out": P + 64, "mp_bits": P, "mp_scales": P})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_WORKSPACE  # m_prev unread
    a = ob.FrozenVArgs(**{**lamb, "mode": 1, "m": P, "m_prev": None, "mp_bits": P, "mp_scales": P})
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_NULL  # mode 1 reads m_prev
    a = ob.FrozenVArgs(mode=0, N=1022, x=P, m=P, v=P)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_SIZE
    assert lib.frozen_v_step(None, None, 0, None) == ob.ONEBIT_E_NULL


def test_struct_layout_matches_header():
    # offsets implied by the C declaration on x86-64 / amdgcn (LP64)
    assert ob.FrozenVArgs.N.offset == 8
    assert ob.FrozenVArgs.n_seg.offset == 44
    assert ob.FrozenVArgs.x.offset == 48
    assert ob.FrozenVArgs.m_bits.offset == 128
    assert ob.FrozenVArgs.m_chunks.offset == 144
    assert ob.FrozenVArgs.err_ratio.offset == 152
    assert ob.FrozenVArgs.m_out.offset == 160
    assert ob.FrozenVArgs.m_seg_k.offset == 168
    assert ob.FrozenVArgs.mp_bits.offset == 176
    assert ob.FrozenVArgs.mp_scales.offset == 184
    assert ctypes.sizeof(ob.FrozenVArgs) == 192


def test_extended_entries_validation(lib):
    cx = lib.onebit_compress_ex
    base = [P, None, None, 0.0, P, P, P, 1 << 12, 4, 0.0, 0, None, None, None, 0, 0, P, 1 << 30, None]
    bad = list(base); bad[18 - 2] = None  # no workspace
    assert cx(*bad) == ob.ONEBIT_E_WORKSPACE
    bad = list(base); bad[15] = ob.ONEBIT_KEEP_PREV  # a server-only flag
    assert cx(*bad) == ob.ONEBIT_E_ARG
    bad = list(base); bad[13] = P         # error ratio without a layer table
    assert cx(*bad) == ob.ONEBIT_E_ARG
    bad = list(base); bad[1] = P          # words without scales
    assert cx(*bad) == ob.ONEBIT_E_NULL
    sx = lib.onebit_server_reduce_ex
    sbase = [P, P, P, P, P, None, None, None, None, 0, 1 << 12, 4, 0, 0, P, 1 << 30, None]
    bad = list(sbase); bad[13] = 4
    assert sx(*bad) == ob.ONEBIT_E_ARG
    ok = list(sbase); ok[13] = ob.ONEBIT_UNIT_SCALE | ob.ONEBIT_KEEP_PREV; ok[10] = 0
    assert sx(*ok) == ob.ONEBIT_OK                 # both flags accepted (empty: no launch)
    bad = list(sbase); bad[8] = P
    assert sx(*bad) == ob.ONEBIT_E_ARG
    q = lib.int8_quantize
    assert q(P, None, P, P, None, 4096, 0, 0, 1, 1, None, 0, None) == ob.ONEBIT_E_WORKSPACE
    assert q(P, None, P, P, None, 4096, 256, 2, 1, 1, None, 0, None) == ob.ONEBIT_E_ARG
    assert q(P, None, P, P, None, 4098, 0, 0, 1, 1, P, 256, None) == ob.ONEBIT_E_SIZE
    assert lib.int8_sr_quantize(P, None, P, P, None, 4096, 0, 1, 1, None) == ob.ONEBIT_E_SIZE


def test_warmup_validation(lib):
    """Only argument errors (no launch): P is not a device address."""
    f = lib.warmup_adam_step
    assert f(P, P, P, P, 1022, 1e-3, 1e-6, 0.9, 0.999, None) == ob.ONEBIT_E_SIZE
    assert f(P, None, P, P, 1024, 1e-3, 1e-6, 0.9, 0.999, None) == ob.ONEBIT_E_NULL
    assert f(P, P, P, P + 4, 1024, 1e-3, 1e-6, 0.9, 0.999, None) == ob.ONEBIT_E_ALIGN
    assert f(P, P, P, P, 0, 1e-3, 1e-6, 0.9, 0.999, None) == ob.ONEBIT_OK  # empty: no launch

    def lamb(**kw):
        a = dict(x=P, m=P, v=P, g=P, N=4096, off=P, nseg=3, first=1, c=P, cavg=P, ws=P,
                 wsb=1 << 30)
        a.update(kw)
        return lib.warmup_lamb_step(a["x"], a["m"], a["v"], a["g"], a["N"], a["off"], a["nseg"],
                                    1e-3, 1e-6, 0.9, 0.999, 0.9, a["first"], a["c"], a["cavg"],
                                    a["ws"], a["wsb"], None)
    assert lamb(N=4098) == ob.ONEBIT_E_SIZE
    assert lamb(off=None) == ob.ONEBIT_E_NULL
    assert lamb(c=None) == ob.ONEBIT_E_NULL
    assert lamb(nseg=0) == ob.ONEBIT_E_ARG
    assert lamb(first=2) == ob.ONEBIT_E_ARG
    assert lamb(off=P + 4) == ob.ONEBIT_E_ALIGN
    assert lamb(ws=None) == ob.ONEBIT_E_WORKSPACE
    assert lamb(wsb=256) == ob.ONEBIT_E_WORKSPACE
    assert lamb(ws=P + 128) == ob.ONEBIT_E_ALIGN

    g = lib.lamb_momentum_scale
    assert g(P, 4098, P, 3, P, P, 1 << 30, None) == ob.ONEBIT_E_SIZE
    assert g(P, 4096, None, 3, P, P, 1 << 30, None) == ob.ONEBIT_E_NULL
    assert g(P, 4096, P, 0, P, P, 1 << 30, None) == ob.ONEBIT_E_ARG
    assert g(P, 4096, P, 3, P, P, 64, None) == ob.ONEBIT_E_WORKSPACE


def test_warmup_workspace_bytes(lib):
    # plan (n_seg + 1 int64), one binary64 pair per workgroup of the upper
    # bound ceil(N / 4096) + 2 n_seg + 1, layer RMS (n_seg binary64), the
    # exact path's marks (n_seg + 1 int32), exact RMS (n_seg binary64) and
    # two 640-bit integers per workgroup; each part rounded up to 256 bytes
    def rup(x):
        return (x + 255) // 256 * 256
    for N, S in [(4096, 3), (336_226_304, 303), (0, 1)]:
        grid = -(-N // 4096) + 2 * S + 1
        want = (rup(8 * (S + 1)) + rup(16 * grid) + rup(8 * S) + rup(4 * (S + 1)) + rup(8 * S)
                + rup(grid * 2 * 10 * 8))
        assert ob.warmup_workspace_bytes(N, S) == want
    assert ob.warmup_workspace_bytes(1022, 3) == 0
    assert ob.warmup_workspace_bytes(1024, 0) == 0


def test_grid_limit_refused(lib):
    """Sizes whose launch would pass 2^32 work-items along x are refused before
    any launch (the hardware would cut the grid short without an error)."""
    a = ob.FrozenVArgs(mode=0, N=1 << 37, x=P, m=P, v=P, lr=1e-3, eps=1e-6)
    assert lib.frozen_v_step(ctypes.byref(a), None, 0, None) == ob.ONEBIT_E_SIZE
    assert lib.int8_quantize(P, P, P, P, P, 1 << 36, 256, 0, 1, 1, None, 0, None) == ob.ONEBIT_E_SIZE
    # 2^35 elements in 64 chunks of 2^29: a valid chunking, but 2^25 workgroups
    assert lib.onebit_error_materialize(P, P, P, 1 << 35, 64, 64, None) == ob.ONEBIT_E_SIZE
    assert lib.warmup_adam_step(P, P, P, P, 1 << 37, 1e-3, 1e-6, 0.9, 0.999, None) == ob.ONEBIT_E_SIZE


def test_chunk_length_limit(lib):
    """Chunks below 2^31 elements keep the fp64 sums' depth inside the bound
    the finalize certifies; longer chunks are refused."""
    assert ob.workspace_bytes((1 << 31) - 64, 1) > 0
    assert ob.workspace_bytes(1 << 31, 1) == 0
    assert ob.workspace_bytes(1 << 32, 2) == 0
    assert _compress(lib, N=1 << 32, n=2) == ob.ONEBIT_E_SIZE


def test_binding_refuses_host_short_and_mistyped_tensors(monkeypatch):
    """The Python binding checks what the C ABI cannot see: tensors must live
    on the device, carry the element type of their buffer and hold enough
    elements.  Every call below fails in Python, before the library is
    entered (no call here reaches a kernel)."""
    import torch

    N, n = 4096, 4
    host = torch.zeros((n, N))
    with pytest.raises(ValueError, match="device tensor"):
        ob.onebit_compress(host, host, torch.zeros((n, n)), torch.zeros((n, N // 32),
                           dtype=torch.int32), N, n, ws=torch.zeros(1 << 20, dtype=torch.uint8))
    # pretend host tensors are device tensors to reach the size and type checks
    monkeypatch.setattr(ob, "_on_gpu", lambda t: True)
    scales = torch.zeros((n, n))
    bits = torch.zeros((n, N // 32), dtype=torch.int32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="needs"):
        ob.onebit_compress(torch.zeros((n, N - 64)), host, scales, bits, N, n, ws=ws)
    with pytest.raises(ValueError, match="float32"):
        ob.onebit_compress(host.double(), host, scales, bits, N, n, ws=ws)
    with pytest.raises(ValueError, match="int32 or uint32"):
        ob.onebit_compress(host, host, scales, bits.long(), N, n, ws=ws)
    with pytest.raises(ValueError, match="needs"):
        ob.onebit_server_reduce(bits, scales, torch.zeros(N - 4), torch.zeros(n),
                                torch.zeros(N // 32, dtype=torch.int32), None, N, n, ws=ws)
    with pytest.raises(ValueError, match="int8"):
        ob.int8_sr_quantize(torch.zeros(N), None, torch.zeros(N, dtype=torch.uint8),
                            torch.zeros(N // 256), None, N, 256, 1, 1)
    with pytest.raises(ValueError, match="needs"):
        ob.frozen_v_step(mode=0, N=N, x=torch.zeros(N), m=torch.zeros(N // 2), v=torch.zeros(N),
                         lr=1e-3, eps=1e-6)
    with pytest.raises(ValueError, match="int64"):
        ob.lamb_layer_scale(torch.zeros(N), N, 1, torch.zeros(3, dtype=torch.int32),
                            torch.zeros(2), 2, False)


def test_binding_shares_torchs_hip_runtime():
    """Loading the library through the binding before torch leaves one HIP
    runtime in the process, torch's (the binding imports torch first): a
    second runtime beside torch's would report no device to the library's
    calls.  Checked in a fresh interpreter from the mapped files; nothing
    is initialised, so no GPU is needed."""
    import ast
    import os
    import subprocess
    import sys

    code = ("from momentum_compression_amd import onebit as ob\n"
            "ob.load()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    runtimes = ast.literal_eval(out.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes
