"""ctypes binding of libonebit.so (the C ABI declared in include/onebit.h).

Argument marshalling only: tensors become device pointers, the stream
defaults to torch's current HIP stream, and a nonzero status raises
``OnebitError``.  Every step of the compression stage runs in the library's
HIP kernels; nothing here computes.  The library must have been built
(``python -m momentum_compression_amd.build``); a missing library is an
error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libonebit.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "onebit.h")

ONEBIT_OK = 0
ONEBIT_E_NULL = -1
ONEBIT_E_SIZE = -2
ONEBIT_E_ALIGN = -3
ONEBIT_E_WORKSPACE = -4
ONEBIT_E_ARG = -5
ONEBIT_E_HIP = -6
ONEBIT_UNIT_SCALE = 1
ONEBIT_KEEP_PREV = 2

_c_i32, _c_i64, _c_u32, _c_u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
_c_f, _c_p, _c_sz = ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class FrozenVArgs(ctypes.Structure):
    """Mirror of onebit_frozen_v_args."""

    _fields_ = [
        ("mode", _c_i32), ("use_c_t", _c_i32), ("N", _c_i64),
        ("lr", _c_f), ("eps", _c_f), ("beta1", _c_f), ("beta2", _c_f),
        ("r_threshold", _c_f), ("r_min", _c_f), ("r_max", _c_f),
        ("n_seg", _c_i32),
        ("x", _c_p), ("m", _c_p), ("v", _c_p), ("m_prev", _c_p), ("v_fresh", _c_p),
        ("seg_off", _c_p), ("c_avg", _c_p), ("r_prev", _c_p), ("c_prev", _c_p),
        ("ratio_max", _c_p),
        ("m_bits", _c_p), ("m_scales", _c_p), ("m_chunks", _c_i32),
        ("err_ratio", _c_p),
        ("m_out", _c_p), ("m_seg_k", _c_p),
        ("mp_bits", _c_p), ("mp_scales", _c_p),
    ]


_SIGNATURES = {
    "onebit_compress": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_f, _c_i32, _c_p, _c_p,
                                 _c_i32, _c_p, _c_sz, _c_p]),
    "onebit_compress_grad": (_c_i32, [_c_p, _c_p, _c_p, _c_f, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_f,
                                      _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_sz, _c_p]),
    "onebit_compress_ex": (_c_i32, [_c_p, _c_p, _c_p, _c_f, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_f,
                                    _c_i32, _c_p, _c_p, _c_p, _c_i32, _c_u32, _c_p, _c_sz, _c_p]),
    "onebit_server_reduce_ex": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                         _c_i32, _c_i64, _c_i32, _c_i32, _c_u32, _c_p, _c_sz,
                                         _c_p]),
    "onebit_server_reduce_noalloc": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                              _c_p, _c_i32, _c_i64, _c_i32, _c_i32, _c_u32, _c_p]),
    "int8_quantize": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_u64, _c_u32,
                               _c_p, _c_sz, _c_p]),
    "onebit_server_reduce": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64,
                                      _c_i32, _c_i32, _c_p, _c_sz, _c_p]),
    "onebit_decompress": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_i32, _c_p]),
    "onebit_error_materialize": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_p]),
    "lamb_layer_scale": (_c_i32, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_i32, _c_i32, _c_p]),
    "frozen_v_step": (_c_i32, [ctypes.POINTER(FrozenVArgs), _c_p, _c_sz, _c_p]),
    "int8_sr_quantize": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_u64, _c_u32, _c_p]),
    "onebit_workspace_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32]),
    "frozen_v_workspace_bytes": (_c_sz, [_c_i64, _c_i32]),
    "warmup_adam_step": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_f, _c_f, _c_f, _c_f, _c_p]),
    "warmup_lamb_step": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i32, _c_f, _c_f, _c_f,
                                  _c_f, _c_f, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "lamb_momentum_scale": (_c_i32, [_c_p, _c_i64, _c_p, _c_i32, _c_p, _c_p, _c_sz, _c_p]),
    "warmup_workspace_bytes": (_c_sz, [_c_i64, _c_i32]),
    "onebit_strerror": (ctypes.c_char_p, [_c_i32]),
}

_lib: Optional[ctypes.CDLL] = None


class OnebitError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libonebit.so (raises if it has not been built).

    torch is imported first.  Its wheel carries its own HIP runtime, whose
    soname (libamdhip64.so.7) the library's dependency then resolves to, so
    the process holds one runtime, the one torch's tensors and streams
    belong to.  Loaded before torch, the library would bind to the system's
    runtime and torch would then load its own beside it: two runtimes, and
    the library's calls fail (a runtime that finds the device already taken
    reports no device)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (before the library: one HIP runtime)

        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m momentum_compression_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def declared_functions() -> list:
    """Function names declared in include/onebit.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def strerror(status: int) -> str:
    return load().onebit_strerror(status).decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr()


def _on_gpu(t) -> bool:
    return t.device.type == "cuda"


# element kinds of the C ABI's buffers and the tensor dtypes that carry them
_KINDS = {"f32": ("float32",), "u32": ("int32", "uint32"), "i64": ("int64",),
          "i8": ("int8",), "u8": ("uint8",)}


def _buf(x, count: int, kind: str, name: str) -> Optional[int]:
    """Device pointer of a tensor argument that must hold at least ``count``
    elements of ``kind``.  Plain integers (raw device addresses) pass as they
    are; a host tensor, a wrong dtype or a short buffer raises ValueError
    before the library sees the call (the C ABI cannot check sizes)."""
    if x is None or isinstance(x, int):
        return x
    if not _on_gpu(x):
        raise ValueError(f"{name} must be a device tensor (got {x.device})")
    if str(x.dtype).replace("torch.", "") not in _KINDS[kind]:
        raise ValueError(f"{name} must be {' or '.join(_KINDS[kind])} (got {x.dtype})")
    if x.numel() < count:
        raise ValueError(f"{name} holds {x.numel()} elements, the call needs {count}")
    return _ptr(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int) -> None:
    if st != ONEBIT_OK:
        raise OnebitError(fn, st)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def workspace_bytes(N: int, n: int, n_seg: int = 0) -> int:
    return int(load().onebit_workspace_bytes(N, n, n_seg))


def frozen_v_workspace_bytes(N: int, n_seg: int) -> int:
    return int(load().frozen_v_workspace_bytes(N, n_seg))


def onebit_compress(m, ef, scales, bits, N: int, n: int, clip: float = 0.0, reset: bool = False,
                    seg_off=None, seg_k=None, n_seg: int = 0, ws=None, stream=None) -> None:
    _check("onebit_compress", load().onebit_compress(
        _buf(m, n * N, "f32", "m"), _buf(ef, n * N, "f32", "ef"), _buf(scales, n * n, "f32", "scales"),
        _buf(bits, n * N // 32, "u32", "bits"), N, n, clip, int(bool(reset)),
        _buf(seg_off, n_seg + 1, "i64", "seg_off"), _buf(seg_k, n_seg, "f32", "seg_k"), n_seg,
        _buf(ws, 0, "u8", "ws"), _nbytes(ws) if ws is not None else 0, _stream(stream)))


def onebit_compress_grad(g, mb_bits, mb_scales, beta1: float, ef, scales, bits, N: int, n: int,
                         clip: float = 0.0, reset: bool = False, seg_off=None, seg_k=None,
                         n_seg: int = 0, ws=None, stream=None) -> None:
    _check("onebit_compress_grad", load().onebit_compress_grad(
        _buf(g, n * N, "f32", "g"), _buf(mb_bits, N // 32, "u32", "mb_bits"),
        _buf(mb_scales, n, "f32", "mb_scales"), beta1, _buf(ef, n * N, "f32", "ef"),
        _buf(scales, n * n, "f32", "scales"), _buf(bits, n * N // 32, "u32", "bits"), N, n,
        clip, int(bool(reset)), _buf(seg_off, n_seg + 1, "i64", "seg_off"),
        _buf(seg_k, n_seg, "f32", "seg_k"), n_seg, _buf(ws, 0, "u8", "ws"),
        _nbytes(ws) if ws is not None else 0, _stream(stream)))


def onebit_compress_ex(m, ef, scales, bits, N: int, n: int, mb_bits=None, mb_scales=None,
                       beta1: float = 0.0, clip: float = 0.0, reset: bool = False, seg_off=None,
                       seg_k=None, seg_err_ratio=None, n_seg: int = 0, flags: int = 0, ws=None,
                       stream=None) -> None:
    _check("onebit_compress_ex", load().onebit_compress_ex(
        _buf(m, n * N, "f32", "m"), _buf(mb_bits, N // 32, "u32", "mb_bits"),
        _buf(mb_scales, n, "f32", "mb_scales"), beta1, _buf(ef, n * N, "f32", "ef"),
        _buf(scales, n * n, "f32", "scales"), _buf(bits, n * N // 32, "u32", "bits"), N, n,
        clip, int(bool(reset)), _buf(seg_off, n_seg + 1, "i64", "seg_off"),
        _buf(seg_k, n_seg, "f32", "seg_k"), _buf(seg_err_ratio, n_seg, "f32", "seg_err_ratio"),
        n_seg, flags, _buf(ws, 0, "u8", "ws"), _nbytes(ws) if ws is not None else 0,
        _stream(stream)))


def onebit_server_reduce_ex(bits, scales, ef, sv_scales, sv_bits, m_out, N: int, n: int,
                            reset: bool = False, seg_off=None, seg_k=None, seg_err_ratio=None,
                            n_seg: int = 0, flags: int = 0, ws=None, stream=None) -> None:
    _check("onebit_server_reduce_ex", load().onebit_server_reduce_ex(
        _buf(bits, n * N // 32, "u32", "bits"), _buf(scales, n * n, "f32", "scales"),
        _buf(ef, N, "f32", "ef"),
        _buf(sv_scales, 2 * n if flags & ONEBIT_KEEP_PREV else n, "f32", "sv_scales"),
        _buf(sv_bits, N // 32, "u32", "sv_bits"), _buf(m_out, N, "f32", "m_out"),
        _buf(seg_off, n_seg + 1, "i64", "seg_off"), _buf(seg_k, n_seg, "f32", "seg_k"),
        _buf(seg_err_ratio, n_seg, "f32", "seg_err_ratio"), n_seg, N, n, int(bool(reset)), flags,
        _buf(ws, 0, "u8", "ws"), _nbytes(ws) if ws is not None else 0, _stream(stream)))


def onebit_server_reduce_noalloc(bits, scales, ef, sv_scales, sv_bits, m_out, N: int, n: int,
                                 reset: bool = False, seg_off=None, seg_k=None,
                                 seg_err_ratio=None, n_seg: int = 0, flags: int = 0,
                                 stream=None) -> None:
    """``onebit_server_reduce_ex`` without a workspace (the library's fixed
    per-device scratch)."""
    _check("onebit_server_reduce_noalloc", load().onebit_server_reduce_noalloc(
        _buf(bits, n * N // 32, "u32", "bits"), _buf(scales, n * n, "f32", "scales"),
        _buf(ef, N, "f32", "ef"),
        _buf(sv_scales, 2 * n if flags & ONEBIT_KEEP_PREV else n, "f32", "sv_scales"),
        _buf(sv_bits, N // 32, "u32", "sv_bits"), _buf(m_out, N, "f32", "m_out"),
        _buf(seg_off, n_seg + 1, "i64", "seg_off"), _buf(seg_k, n_seg, "f32", "seg_k"),
        _buf(seg_err_ratio, n_seg, "f32", "seg_err_ratio"), n_seg, N, n, int(bool(reset)), flags,
        _stream(stream)))


def onebit_server_reduce(bits, scales, ef, sv_scales, sv_bits, m_out, N: int, n: int,
                         reset: bool = False, seg_off=None, seg_k=None, n_seg: int = 0, ws=None,
                         stream=None) -> None:
    _check("onebit_server_reduce", load().onebit_server_reduce(
        _buf(bits, n * N // 32, "u32", "bits"), _buf(scales, n * n, "f32", "scales"),
        _buf(ef, N, "f32", "ef"), _buf(sv_scales, n, "f32", "sv_scales"),
        _buf(sv_bits, N // 32, "u32", "sv_bits"), _buf(m_out, N, "f32", "m_out"),
        _buf(seg_off, n_seg + 1, "i64", "seg_off"), _buf(seg_k, n_seg, "f32", "seg_k"), n_seg, N,
        n, int(bool(reset)), _buf(ws, 0, "u8", "ws"), _nbytes(ws) if ws is not None else 0,
        _stream(stream)))


def onebit_decompress(sv_bits, sv_scales, m_out, N: int, n: int, seg_off=None, seg_k=None,
                      n_seg: int = 0, stream=None) -> None:
    _check("onebit_decompress", load().onebit_decompress(
        _buf(sv_bits, N // 32, "u32", "sv_bits"), _buf(sv_scales, n, "f32", "sv_scales"),
        _buf(m_out, N, "f32", "m_out"), _buf(seg_off, n_seg + 1, "i64", "seg_off"),
        _buf(seg_k, n_seg, "f32", "seg_k"), n_seg, N, n, _stream(stream)))


def onebit_error_materialize(ef, scales, e_out, N: int, rows: int, n: int, stream=None) -> None:
    _check("onebit_error_materialize", load().onebit_error_materialize(
        _buf(ef, rows * N, "f32", "ef"), _buf(scales, rows * n, "f32", "scales"),
        _buf(e_out, rows * N, "f32", "e_out"), N, rows, n, _stream(stream)))


def lamb_layer_scale(buf, N: int, batch: int, seg_off, seg_k, n_seg: int, divide: bool,
                     stream=None) -> None:
    _check("lamb_layer_scale", load().lamb_layer_scale(
        _buf(buf, batch * N, "f32", "buf"), N, batch, _buf(seg_off, n_seg + 1, "i64", "seg_off"),
        _buf(seg_k, n_seg, "f32", "seg_k"), n_seg, int(bool(divide)), _stream(stream)))


def frozen_v_step(*, mode: int, N: int, x, m, v, lr: float, eps: float, beta1: float = 0.9,
                  beta2: float = 0.999, m_prev=None, v_fresh=None, seg_off=None, n_seg: int = 0,
                  c_avg=None, r_prev=None, c_prev=None, ratio_max=None, r_threshold: float = 0.1,
                  r_min: float = 0.5, r_max: float = 4.0, use_c_t: bool = False, m_bits=None,
                  m_scales=None, m_chunks: int = 0, err_ratio=None, m_out=None, m_seg_k=None,
                  mp_bits=None, mp_scales=None, ws=None, stream=None) -> None:
    a = FrozenVArgs(mode=mode, use_c_t=int(bool(use_c_t)), N=N, lr=lr, eps=eps, beta1=beta1,
                    beta2=beta2, r_threshold=r_threshold, r_min=r_min, r_max=r_max, n_seg=n_seg,
                    x=_buf(x, N, "f32", "x"), m=_buf(m, N, "f32", "m"), v=_buf(v, N, "f32", "v"),
                    m_prev=_buf(m_prev, N, "f32", "m_prev"),
                    v_fresh=_buf(v_fresh, N, "f32", "v_fresh"),
                    seg_off=_buf(seg_off, n_seg + 1, "i64", "seg_off"),
                    c_avg=_buf(c_avg, n_seg, "f32", "c_avg"), r_prev=_buf(r_prev, n_seg, "f32", "r_prev"),
                    c_prev=_buf(c_prev, n_seg, "f32", "c_prev"),
                    ratio_max=_buf(ratio_max, n_seg, "f32", "ratio_max"),
                    m_bits=_buf(m_bits, N // 32, "u32", "m_bits"),
                    m_scales=_buf(m_scales, m_chunks, "f32", "m_scales"), m_chunks=m_chunks,
                    err_ratio=_buf(err_ratio, n_seg, "f32", "err_ratio"),
                    m_out=_buf(m_out, N, "f32", "m_out"), m_seg_k=_buf(m_seg_k, n_seg, "f32", "m_seg_k"),
                    mp_bits=_buf(mp_bits, N // 32, "u32", "mp_bits"),
                    mp_scales=_buf(mp_scales, m_chunks, "f32", "mp_scales"))
    _check("frozen_v_step", load().frozen_v_step(
        ctypes.byref(a), _buf(ws, 0, "u8", "ws"), _nbytes(ws) if ws is not None else 0,
        _stream(stream)))


def int8_sr_quantize(g, err, codes, block_scales, deq, N: int, block: int, seed: int, step: int,
                     stream=None) -> None:
    nsc = N // block if block > 0 else 1
    _check("int8_sr_quantize", load().int8_sr_quantize(
        _buf(g, N, "f32", "g"), _buf(err, N, "f32", "err"), _buf(codes, N, "i8", "codes"),
        _buf(block_scales, nsc, "f32", "block_scales"), _buf(deq, N, "f32", "deq"), N, block,
        seed & 0xFFFFFFFFFFFFFFFF, step & 0xFFFFFFFF, _stream(stream)))


def int8_quantize(g, err, codes, block_scales, deq, N: int, block: int, rounding: int, seed: int,
                  step: int, ws=None, stream=None) -> None:
    nsc = N // block if block > 0 else 1
    _check("int8_quantize", load().int8_quantize(
        _buf(g, N, "f32", "g"), _buf(err, N, "f32", "err"), _buf(codes, N, "i8", "codes"),
        _buf(block_scales, nsc, "f32", "block_scales"), _buf(deq, N, "f32", "deq"), N, block,
        rounding, seed & 0xFFFFFFFFFFFFFFFF, step & 0xFFFFFFFF, _buf(ws, 0, "u8", "ws"),
        _nbytes(ws) if ws is not None else 0, _stream(stream)))


def warmup_workspace_bytes(N: int, n_seg: int) -> int:
    return int(load().warmup_workspace_bytes(N, n_seg))


def warmup_adam_step(x, m, v, g, N: int, lr: float, eps: float, beta1: float, beta2: float,
                     stream=None) -> None:
    _check("warmup_adam_step", load().warmup_adam_step(
        _buf(x, N, "f32", "x"), _buf(m, N, "f32", "m"), _buf(v, N, "f32", "v"),
        _buf(g, N, "f32", "g"), N, lr, eps, beta1, beta2, _stream(stream)))


def warmup_lamb_step(x, m, v, g, N: int, seg_off, n_seg: int, lr: float, eps: float, beta1: float,
                     beta2: float, beta_c: float, first: bool, c, c_avg, ws, stream=None) -> None:
    _check("warmup_lamb_step", load().warmup_lamb_step(
        _buf(x, N, "f32", "x"), _buf(m, N, "f32", "m"), _buf(v, N, "f32", "v"),
        _buf(g, N, "f32", "g"), N, _buf(seg_off, n_seg + 1, "i64", "seg_off"), n_seg, lr, eps,
        beta1, beta2, beta_c, 1 if first else 0, _buf(c, n_seg, "f32", "c"),
        _buf(c_avg, n_seg, "f32", "c_avg"), _buf(ws, 0, "u8", "ws"), _nbytes(ws), _stream(stream)))


def lamb_momentum_scale(m, N: int, seg_off, n_seg: int, k, ws, stream=None) -> None:
    _check("lamb_momentum_scale", load().lamb_momentum_scale(
        _buf(m, N, "f32", "m"), N, _buf(seg_off, n_seg + 1, "i64", "seg_off"), n_seg,
        _buf(k, n_seg, "f32", "k"), _buf(ws, 0, "u8", "ws"), _nbytes(ws), _stream(stream)))
