"""Python access to the C++ oracle (oracle/cpp/onebit_ref.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU baseline use it; the GPU library never does.

The C++ oracle computes what the numpy oracle computes, as plain loops, fast
enough for whole full-size buffers. The functions below only marshal numpy
arrays into it and have the numpy oracle's names and return keys. Rows
(workers) and server chunks are independent, so ``threads`` > 1 runs them in
parallel Python threads (ctypes releases the interpreter lock during each
call); that changes no arithmetic.
"""

from __future__ import annotations

import ctypes as ct
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "onebit_ref.cpp")
LIB = os.path.join(HERE, "cpp", "libonebit_ref.so")
# -fno-math-errno only stops sqrt from setting errno; no flag here changes a
# binary32 result
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-fno-math-errno", "-Wall", "-Wextra", "-Werror"]

_lib = None
f32 = np.float32
_P = ct.c_void_p
_I64, _I32, _U32, _U64, _F = ct.c_int64, ct.c_int32, ct.c_uint32, ct.c_uint64, ct.c_float


def build(verbose: bool = False) -> str:
    """Compile the C++ oracle with g++ (plain binary32 arithmetic, nothing
    contracted or reassociated) and return the library path."""
    tmp = LIB + ".tmp"
    cmd = ["g++", *FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ct.CDLL(LIB)
    sig = {
        "ref_mean_abs": (_F, [_P, _I64]),
        "ref_worker_compress_row": (_I32, [_P, _P, _P, _P, _I64, _I32, _F, _I32, _I32,
                                           _P, _P, _P, _P]),
        "ref_local_momentum": (None, [_P, _P, _F, _I64, _P]),
        "ref_server_chunk": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                    _P, _P, _P, _P, _P]),
        "ref_decompress": (_I32, [_P, _P, _P, _I64, _I32, _P]),
        "ref_adam_frozen_step": (None, [_P, _P, _P, _I64, _F, _F]),
        "ref_lamb_frozen_step": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _P, _P,
                                        _F, _F, _F, _F, _F, _F, _F, _I32, _P, _P, _P, _P]),
        "ref_philox4x32_10": (None, [_P, _P, _P]),
        "ref_uniform": (_F, [_U64, _U64, _U32]),
        "ref_int8_quantize": (_I32, [_P, _P, _I64, _I64, _I32, _U64, _U32, _I64,
                                     _P, _P, _P, _P]),
        "ref_adam_warmup_step": (None, [_P, _P, _P, _P, _I64, _F, _F, _F, _F]),
        "ref_lamb_warmup_step": (_I32, [_P, _P, _P, _P, _P, _I32, _F, _F, _F, _F, _P, _F,
                                        _P, _P]),
        "ref_momentum_scale": (_I32, [_P, _P, _I32, _P]),
        "ref_exact_sumsq": (ct.c_double, [_P, _I64]),
        "ref_exact_sum_f64": (ct.c_double, [_P, _I64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _arr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _ok(rc: int, what: str) -> None:
    if rc:
        raise ValueError(f"C++ oracle rejected the arguments of {what}")


def _run(fn, items, threads: int) -> None:
    if threads <= 1:
        for it in items:
            fn(it)
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for _ in ex.map(fn, items):
            pass


def mean_abs_f32(x) -> np.float32:
    x = _arr(x, f32).ravel()
    if x.size == 0:
        raise ValueError("mean of an empty chunk")
    if x.size >= 1 << 39:
        raise ValueError("too many terms for the per-exponent accumulation")
    return f32(load().ref_mean_abs(_p(x), x.size))


def worker_compress(m, e, clip: float = 0.0, reset: bool = False, k=None,
                    unit_scale: bool = False, err_ratio=None, threads: int = 1,
                    keep_gc: bool = True) -> Dict[str, np.ndarray]:
    """Same contract as ``oracle.onebit.worker_compress``. With
    ``keep_gc=False`` the compensated values are not returned (one row of
    scratch instead of n)."""
    lib = load()
    m = _arr(m, f32)
    n, N = m.shape
    e = None if reset else _arr(e, f32)
    k = None if k is None else _arr(k, f32)
    ratio = None if err_ratio is None else _arr(err_ratio, f32)
    e_out = np.empty((n, N), dtype=f32)
    bits = np.zeros((n, N // 32), dtype=np.uint32)
    s = np.empty((n, n), dtype=f32)
    gc = np.empty((n, N), dtype=f32) if keep_gc else None

    def row(i):
        g_i = gc[i] if keep_gc else np.empty(N, dtype=f32)
        rc = lib.ref_worker_compress_row(_p(m[i]), None if e is None else _p(e[i]), _p(k),
                                         _p(ratio), N, n, float(clip), int(bool(reset)),
                                         int(bool(unit_scale)), _p(g_i), _p(e_out[i]),
                                         _p(bits[i]), _p(s[i]))
        _ok(rc, "worker_compress")

    _run(row, range(n), threads)
    out = {"bits": bits, "s": s, "e": e_out}
    if keep_gc:
        out["gc"] = gc
    return out


def worker_compress_row(m_row, e_row, n: int, clip: float = 0.0, reset: bool = False, k=None,
                        unit_scale: bool = False, err_ratio=None, threads: int = 1,
                        gc_out: Optional[np.ndarray] = None,
                        e_out: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One worker's row of ``worker_compress`` (the row holds n chunks):
    gc, bits (N/32), s (n) and the new error, which is written over ``e_row``
    when that is a contiguous float32 array (a copy otherwise), or into
    ``e_out`` when given (needed with ``reset``, where ``e_row`` is not read).
    ``gc_out`` may pass the buffer for the compensated values.

    With ``threads`` > 1 the row's n chunks run in parallel, each as a row of
    one chunk: every step of the worker compression is per element except the
    scale, which is per chunk, so the results are the same."""
    lib = load()
    m_row = _arr(m_row, f32)
    N = m_row.size
    e = None if reset else _arr(e_row, f32)
    if e_out is None:
        e_out = e if e is not None else np.empty(N, dtype=f32)
    k = None if k is None else _arr(k, f32)
    ratio = None if err_ratio is None else _arr(err_ratio, f32)
    gc = np.empty(N, dtype=f32) if gc_out is None else gc_out
    for buf in (gc, e_out):
        if buf.dtype != f32 or buf.size != N or not buf.flags.c_contiguous:
            raise ValueError("output buffers must be contiguous float32 rows of N elements")
    bits = np.zeros(N // 32, dtype=np.uint32)
    s = np.empty(n, dtype=f32)
    if N % (64 * n):
        raise ValueError("N must be a multiple of 64 n")
    L = N // n

    def at(a, c, per=1):
        return None if a is None else a[c * L // per:]

    def chunk(c):
        rc = lib.ref_worker_compress_row(_p(at(m_row, c)), _p(at(e, c)), _p(at(k, c)),
                                         _p(at(ratio, c)), L, 1, float(clip), int(bool(reset)),
                                         int(bool(unit_scale)), _p(at(gc, c)), _p(at(e_out, c)),
                                         _p(at(bits, c, 32)), _p(s[c:]))
        _ok(rc, "worker_compress_row")

    if threads > 1:
        _run(chunk, range(n), min(threads, n))
    else:
        rc = lib.ref_worker_compress_row(_p(m_row), _p(e), _p(k), _p(ratio), N, n, float(clip),
                                         int(bool(reset)), int(bool(unit_scale)), _p(gc),
                                         _p(e_out), _p(bits), _p(s))
        _ok(rc, "worker_compress_row")
    return {"gc": gc, "bits": bits, "s": s, "e": e_out}


def local_momentum(g, mbar_prev, beta1: float) -> np.ndarray:
    lib = load()
    g = _arr(g, f32)
    mb = _arr(mbar_prev, f32)
    out = np.empty_like(g)
    for i in range(g.shape[0]):
        lib.ref_local_momentum(_p(g[i]), _p(mb), float(beta1), g.shape[1], _p(out[i]))
    return out


def server_reduce(bits, s, E, reset: bool = False, unit_scale: bool = False, err_ratio=None,
                  threads: int = 1) -> Dict[str, np.ndarray]:
    """Same contract as ``oracle.onebit.server_reduce``."""
    lib = load()
    bits = _arr(bits, np.uint32)
    s = _arr(s, f32)
    n = s.shape[0]
    N = bits.shape[1] * 32
    E = None if reset else _arr(E, f32)
    ratio = None if err_ratio is None else _arr(err_ratio, f32)
    out = {"avg": np.empty(N, dtype=f32), "g2": np.empty(N, dtype=f32),
           "E": np.empty(N, dtype=f32), "S": np.empty(n, dtype=f32),
           "bits": np.zeros(N // 32, dtype=np.uint32)}

    def chunk(c):
        rc = lib.ref_server_chunk(_p(bits), _p(s), _p(E), _p(ratio), N, n, c, int(bool(reset)),
                                  int(bool(unit_scale)), _p(out["avg"]), _p(out["g2"]),
                                  _p(out["E"]), _p(out["bits"]), _p(out["S"]))
        _ok(rc, "server_reduce")

    _run(chunk, range(n), threads)
    return out


def server_reduce_chunk(bits, s, E, c: int, reset: bool = False, unit_scale: bool = False,
                        err_ratio=None) -> Dict[str, np.ndarray]:
    """The server of chunk c alone: ``server_reduce`` restricted to one chunk.
    bits [n, N/32] and s [n, n] as there; E (not read with ``reset``) and
    err_ratio need only the elements up to the chunk's end. The outputs
    cover elements [0, (c + 1) L), of which only chunk c is written, and
    S[c]."""
    lib = load()
    bits = _arr(bits, np.uint32)
    s = _arr(s, f32)
    n = s.shape[0]
    N = bits.shape[1] * 32
    if N % (64 * n) or not 0 <= c < n:
        raise ValueError("bad chunk or buffer size")
    end = (c + 1) * (N // n)
    E = None if reset else _arr(E, f32)
    ratio = None if err_ratio is None else _arr(err_ratio, f32)
    for a in (E, ratio):
        if a is not None and a.size < end:
            raise ValueError("E and err_ratio must cover the chunk")
    out = {"avg": np.empty(end, dtype=f32), "g2": np.empty(end, dtype=f32),
           "E": np.empty(end, dtype=f32), "S": np.zeros(n, dtype=f32),
           "bits": np.zeros(end // 32, dtype=np.uint32)}
    rc = lib.ref_server_chunk(_p(bits), _p(s), _p(E), _p(ratio), N, n, c, int(bool(reset)),
                              int(bool(unit_scale)), _p(out["avg"]), _p(out["g2"]),
                              _p(out["E"]), _p(out["bits"]), _p(out["S"]))
    _ok(rc, "server_reduce_chunk")
    return out


def decompress(sbits, S, k=None, threads: int = 1) -> np.ndarray:
    """Same contract as ``oracle.onebit.decompress``. With ``threads`` > 1
    the chunks run in parallel, each as a buffer of one chunk (every output
    element depends only on its own bit, its chunk's scale and its k)."""
    lib = load()
    sbits = _arr(sbits, np.uint32)
    S = _arr(S, f32)
    N = sbits.size * 32
    n = S.size
    k = None if k is None else _arr(k, f32)
    out = np.empty(N, dtype=f32)
    if threads <= 1 or n == 1:
        _ok(lib.ref_decompress(_p(sbits), _p(S), _p(k), N, n, _p(out)), "decompress")
        return out
    if N % (64 * n):
        raise ValueError("N must be a multiple of 64 n")
    L = N // n

    def chunk(c):
        rc = lib.ref_decompress(_p(sbits[c * L // 32:]), _p(S[c:]),
                                None if k is None else _p(k[c * L:]), L, 1, _p(out[c * L:]))
        _ok(rc, "decompress")

    _run(chunk, range(n), min(threads, n))
    return out


def adam_frozen_step(x, m, v, lr: float, eps: float, threads: int = 1) -> np.ndarray:
    """Same contract as ``oracle.optim.adam_frozen_step``; with ``threads`` > 1
    the (elementwise) step runs over that many slices in parallel."""
    lib = load()
    x = _arr(x, f32).copy()
    m, v = _arr(m, f32), _arr(v, f32)
    N = x.size
    parts = max(1, min(threads, N // 4096))
    cuts = [N * p // parts for p in range(parts + 1)]

    def part(p):
        a, b = cuts[p], cuts[p + 1]
        lib.ref_adam_frozen_step(_p(x[a:]), _p(m[a:]), _p(v[a:]), b - a, float(lr), float(eps))

    _run(part, range(parts), parts)
    return x


def lamb_frozen_step(x, m, m_prev, v_f, v_tw, seg_off, c_avg, r_prev, c_prev,
                     lr: float, eps: float, beta1: float, beta2: float,
                     thr: float, r_min: float, r_max: float,
                     use_c_t: bool = False) -> Dict[str, np.ndarray]:
    """Same contract as ``oracle.optim.lamb_frozen_step`` (without ``g``)."""
    lib = load()
    x = _arr(x, f32).copy()
    v = _arr(v_f, f32).copy()
    m, m_prev, v_tw = _arr(m, f32), _arr(m_prev, f32), _arr(v_tw, f32)
    off = _arr(seg_off, np.int64)
    L = off.size - 1
    c_avg, r_prev, c_prev = _arr(c_avg, f32), _arr(r_prev, f32), _arr(c_prev, f32)
    R, r, c, rho = (np.empty(L, dtype=f32) for _ in range(4))
    rc = lib.ref_lamb_frozen_step(_p(x), _p(m), _p(m_prev), _p(v), _p(v_tw), _p(off), L,
                                  _p(c_avg), _p(r_prev), _p(c_prev), float(lr), float(eps),
                                  float(beta1), float(beta2), float(thr), float(r_min),
                                  float(r_max), int(bool(use_c_t)), _p(R), _p(r), _p(c), _p(rho))
    _ok(rc, "lamb_frozen_step")
    return {"x": x, "v": v, "R": R, "r": r, "c": c, "err_ratio": rho}


def philox4x32_10(ctr, key) -> np.ndarray:
    lib = load()
    ctr = _arr(ctr, np.uint32).reshape(-1, 4)
    key = np.broadcast_to(_arr(key, np.uint32), (ctr.shape[0], 2)).copy()
    out = np.empty_like(ctr)
    for i in range(ctr.shape[0]):
        lib.ref_philox4x32_10(_p(ctr[i]), _p(key[i]), _p(out[i]))
    return out


def uniforms(J0: int, count: int, seed: int, step: int) -> np.ndarray:
    lib = load()
    return np.array([lib.ref_uniform(J0 + j, seed, step) for j in range(count)], dtype=f32)


def int8_sr(g, e, seed: int, step: int, block: int = 256, J0: int = 0,
            rounding: str = "stochastic", threads: int = 1) -> Dict[str, np.ndarray]:
    """Same contract as ``oracle.int8.int8_sr`` (without ``gc``). With
    ``threads`` > 1 and a block size, whole blocks are split into that many
    slices, each keyed by its own first global index."""
    lib = load()
    g = _arr(g, f32).ravel()
    e = None if e is None else _arr(e, f32).ravel()
    N = g.size
    if block and N % block:
        raise ValueError("length must be a multiple of the block")
    nb = 1 if block == 0 else N // block
    codes = np.empty(N, dtype=np.int8)
    scales = np.empty(nb, dtype=f32)
    deq = np.empty(N, dtype=f32)
    e_out = np.empty(N, dtype=f32)
    mode = {"stochastic": 0, "nearest": 1}[rounding]
    parts = 1 if block == 0 else max(1, min(threads, nb))
    cuts = [(nb * p // parts) * (block or N) for p in range(parts + 1)]

    def part(p):
        a, b = cuts[p], cuts[p + 1]
        if a == b:
            return
        rc = lib.ref_int8_quantize(_p(g[a:b]), None if e is None else _p(e[a:b]), b - a, block,
                                   mode, seed, step, J0 + a, _p(codes[a:b]),
                                   _p(scales[a // (block or N):]), _p(deq[a:b]), _p(e_out[a:b]))
        _ok(rc, "int8_sr")

    _run(part, range(parts), threads)
    return {"codes": codes, "scales": scales, "deq": deq, "e": e_out}


def adam_warmup_step(x, m, v, g, lr: float, eps: float, beta1: float,
                     beta2: float) -> Dict[str, np.ndarray]:
    """Same contract as ``oracle.warmup.adam_warmup_step``."""
    lib = load()
    x, m, v = (_arr(a, f32).copy() for a in (x, m, v))
    g = _arr(g, f32)
    lib.ref_adam_warmup_step(_p(x), _p(m), _p(v), _p(g), x.size, float(lr), float(eps),
                             float(beta1), float(beta2))
    return {"x": x, "m": m, "v": v}


def lamb_warmup_step(x, m, v, g, seg_off, lr: float, eps: float, beta1: float, beta2: float,
                     c_avg=None, beta_c: float = 0.9) -> Dict[str, np.ndarray]:
    """Same contract as ``oracle.warmup.lamb_warmup_step`` (without ``u``)."""
    lib = load()
    x, m, v = (_arr(a, f32).copy() for a in (x, m, v))
    g = _arr(g, f32)
    off = _arr(seg_off, np.int64)
    S = off.size - 1
    c = np.empty(S, dtype=f32)
    c_out = np.empty(S, dtype=f32)
    c_in = None if c_avg is None else _arr(c_avg, f32)
    rc = lib.ref_lamb_warmup_step(_p(x), _p(m), _p(v), _p(g), _p(off), S, float(lr), float(eps),
                                  float(beta1), float(beta2), _p(c_in), float(beta_c), _p(c),
                                  _p(c_out))
    _ok(rc, "lamb_warmup_step")
    return {"x": x, "m": m, "v": v, "c": c, "c_avg": c_out}


def momentum_scale(m, seg_off) -> np.ndarray:
    """Same contract as ``oracle.warmup.momentum_scale``."""
    lib = load()
    m = _arr(m, f32)
    off = _arr(seg_off, np.int64)
    k = np.empty(off.size - 1, dtype=f32)
    _ok(lib.ref_momentum_scale(_p(m), _p(off), off.size - 1, _p(k)), "momentum_scale")
    return k


def exact_sumsq(x) -> float:
    x = _arr(x, f32).ravel()
    return load().ref_exact_sumsq(_p(x), x.size)


def exact_sum_f64(x) -> float:
    x = _arr(x, np.float64).ravel()
    return load().ref_exact_sum_f64(_p(x), x.size)
