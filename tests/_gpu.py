"""Helpers for the GPU parity tests (device handling, comparisons).

A GPU test never falls back to anything: if the library is missing the
binding raises, and the test fails."""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob


def device() -> torch.device:
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ob.load()  # raises if libonebit.so is missing
    return torch.device("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int32:
        a = a.view(np.uint32)
    return a


def gen(seed: int, dev) -> torch.Generator:
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


def same_f32(got: np.ndarray, want: np.ndarray, name: str, rtol: float = 1e-6,
             atol: float = 1e-9) -> None:
    """Parity bar for binary32 values: within |a - b| <= atol + rtol |b|
    (NaN matching NaN), and -- the design target -- bit-identical."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{name}: NaN positions differ ({np.sum(gn != wn)})"
    ok = ~gn
    g64, w64 = got[ok].astype(np.float64), want[ok].astype(np.float64)
    with np.errstate(invalid="ignore"):
        inf_ok = np.isinf(w64) & (g64 == w64)
        diff = np.abs(g64 - w64)
        close = inf_ok | (diff <= atol + rtol * np.abs(w64))
    assert close.all(), f"{name}: {np.sum(~close)} of {close.size} outside tolerance"
    bits_eq = got[ok].view(np.uint32) == want[ok].view(np.uint32)
    assert bits_eq.all(), f"{name}: {np.sum(~bits_eq)} of {bits_eq.size} not bit-identical"


def same_bits(got: np.ndarray, want: np.ndarray, name: str) -> None:
    got = np.asarray(got).view(np.uint32) if np.asarray(got).dtype == np.int32 else np.asarray(got)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    neq = got != want
    assert not neq.any(), f"{name}: {int(neq.sum())} of {neq.size} words differ"


def same_whole(got: np.ndarray, want: np.ndarray, name: str) -> None:
    """Bit identity of a whole (large) buffer, checked without float64
    copies; on a mismatch the differing elements go through ``same_f32`` (or
    are counted, for integer data), which names how many differ and where."""
    got, want = np.ascontiguousarray(got), np.ascontiguousarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.dtype == np.float32:
        gb, wb = got.view(np.uint32), want.view(np.uint32)
        if np.array_equal(gb, wb):
            return
        bad = np.flatnonzero(gb != wb)
        same_f32(got.ravel()[bad], want.ravel()[bad],
                 f"{name}: {bad.size} of {got.size} differ, first at {bad[0]}")
    else:
        got = got.view(np.uint32) if got.dtype == np.int32 else got
        neq = got != want
        assert not neq.any(), (f"{name}: {int(neq.sum())} of {neq.size} differ, first at "
                               f"{np.flatnonzero(neq)[0]}")


def same_whole_par(got: np.ndarray, want: np.ndarray, name: str, threads: int = 16) -> None:
    """``same_whole`` with the comparison split over slices that run in
    parallel threads (numpy releases the interpreter lock while it compares);
    a slice that differs goes through ``same_whole`` to name the elements."""
    got, want = np.ascontiguousarray(got).ravel(), np.ascontiguousarray(want).ravel()
    assert got.shape == want.shape and got.dtype == want.dtype, (name, got.shape, want.shape)
    if got.dtype in (np.float32, np.int32):
        gb, wb = got.view(np.uint32), want.view(np.uint32)
    else:
        gb, wb = got, want
    parts = max(1, min(threads, gb.size // (1 << 20)))
    cuts = [gb.size * p // parts for p in range(parts + 1)]

    def equal(p):
        return np.array_equal(gb[cuts[p]:cuts[p + 1]], wb[cuts[p]:cuts[p + 1]])

    with ThreadPoolExecutor(max_workers=parts) as ex:
        eq = list(ex.map(equal, range(parts)))
    for p, ok in enumerate(eq):
        if not ok:
            a, b = cuts[p], cuts[p + 1]
            same_whole(got[a:b], want[a:b], f"{name} (elements {a}..{b - 1})")
