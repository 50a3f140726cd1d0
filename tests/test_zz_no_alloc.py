"""The allocation-free server entry point against the workspace form.

onebit_server_reduce_noalloc keeps the server's partial sums in the
library's fixed per-device scratch instead of a caller workspace. On the same
inputs it must give exactly what onebit_server_reduce_ex gives: sign words,
scales (and the kept previous scales), compensated values and the
decompressed momentum, bit for bit. Two calls in a row, the second on a
smaller input, check that the scratch's leftover contents from the first
call do not leak into the second.
"""

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from tests._gpu import device, gen

pytestmark = pytest.mark.gpu


def _inputs(N, n, seed, dev):
    g = gen(seed, dev)
    bits = torch.randint(-(1 << 31), (1 << 31) - 1, (n, N // 32), generator=g, device=dev,
                         dtype=torch.int32)
    scales = torch.rand((n, n), generator=g, device=dev) * 1e-3
    ef = torch.randn(N, generator=g, device=dev) * 1e-3
    sv_scales = torch.rand(2 * n, generator=g, device=dev) * 1e-3
    return bits, scales, ef, sv_scales


def _run(fn, bits, scales, ef, sv_scales, N, n, **kw):
    ef, sv_scales = ef.clone(), sv_scales.clone()
    sv_bits = torch.zeros(N // 32, dtype=torch.int32, device=ef.device)
    m_out = torch.empty(N, device=ef.device)
    fn(bits, scales, ef, sv_scales, sv_bits, m_out, N, n, **kw)
    return {"ef": ef, "sv_scales": sv_scales, "sv_bits": sv_bits, "m_out": m_out}


def _same(a, b, what):
    for key in a:
        assert torch.equal(a[key].view(torch.int32), b[key].view(torch.int32)), f"{what}: {key}"


def test_noalloc_server_equals_workspace_server_two_calls():
    dev = device()
    cases = [
        # 16 workers, chunks of 30,016 elements (a ragged last tile, several
        # groups per workgroup), layer table with the step-ratio factor,
        # previous scales kept
        dict(N=16 * 30016, n=16, seed=1, layers=True, flags=ob.ONEBIT_KEEP_PREV, reset=False),
        # then a smaller input: 8 workers, 4,160 elements per chunk
        dict(N=8 * 4160, n=8, seed=2, layers=False, flags=0, reset=False),
    ]
    for c in cases:
        N, n = c["N"], c["n"]
        print(f"[noalloc] N={N} n={n} layers={c['layers']} flags={c['flags']}", flush=True)
        bits, scales, ef, sv_scales = _inputs(N, n, c["seed"], dev)
        kw = dict(reset=c["reset"], flags=c["flags"])
        if c["layers"]:
            n_seg = 7
            off = np.sort(np.random.default_rng(c["seed"]).integers(1, N, n_seg - 1))
            off = torch.tensor(np.concatenate([[0], off, [N]]), dtype=torch.int64, device=dev)
            kw.update(seg_off=off, seg_k=torch.ones(n_seg, device=dev),
                      seg_err_ratio=torch.rand(n_seg, generator=gen(9, dev), device=dev) + 0.5,
                      n_seg=n_seg)
        ws = torch.empty(ob.workspace_bytes(N, n, kw.get("n_seg", 0)), dtype=torch.uint8,
                         device=dev)
        want = _run(lambda *a, **k: ob.onebit_server_reduce_ex(*a, ws=ws, **k), bits, scales,
                    ef, sv_scales, N, n, **kw)
        got = _run(ob.onebit_server_reduce_noalloc, bits, scales, ef, sv_scales, N, n, **kw)
        torch.cuda.synchronize()
        _same(got, want, f"N={N} n={n}")
        # a reset step as well (the carried error is not read)
        kw["reset"] = True
        want = _run(lambda *a, **k: ob.onebit_server_reduce_ex(*a, ws=ws, **k), bits, scales,
                    ef, sv_scales, N, n, **kw)
        got = _run(ob.onebit_server_reduce_noalloc, bits, scales, ef, sv_scales, N, n, **kw)
        torch.cuda.synchronize()
        _same(got, want, f"N={N} n={n} reset")


def _random_case(rng, dev, seed):
    n = int(rng.choice([1, 3, 4, 8, 16, 33, 64]))
    L = 64 * int(rng.integers(1, 2000))
    N = n * L
    kw = dict(reset=bool(rng.integers(0, 4) == 0),
              flags=int(rng.choice([0, ob.ONEBIT_KEEP_PREV, ob.ONEBIT_UNIT_SCALE])))
    if rng.integers(0, 2):
        n_seg = int(rng.integers(1, 12))
        off = np.sort(rng.integers(0, N + 1, n_seg - 1))
        off = torch.tensor(np.concatenate([[0], off, [N]]), dtype=torch.int64, device=dev)
        k = torch.from_numpy(np.exp(rng.uniform(-1, 1, n_seg)).astype(np.float32)).to(dev)
        kw.update(seg_off=off, seg_k=k, n_seg=n_seg)
        if rng.integers(0, 2):
            kw["seg_err_ratio"] = torch.rand(n_seg, generator=gen(seed, dev), device=dev) + 0.5
    return N, n, kw


@pytest.mark.parametrize("seed", range(6))
def test_noalloc_random_call_sequences(seed):
    """Four calls in a row of random shapes (n 1..64, ragged chunks, larger
    and smaller than the previous call) and options (a layer table with ÷k
    and the step-ratio factor, kept previous scales, the unscaled sign,
    reset), each equal to the workspace form bit for bit."""
    dev = device()
    rng = np.random.default_rng(300 + seed)
    for call in range(4):
        N, n, kw = _random_case(rng, dev, 10 * seed + call)
        print(f"[noalloc random] seed={seed} call={call} N={N} n={n} "
              f"layers={kw.get('n_seg', 0)} flags={kw['flags']} reset={kw['reset']}", flush=True)
        bits, scales, ef, sv_scales = _inputs(N, n, 100 * seed + call, dev)
        ws = torch.empty(ob.workspace_bytes(N, n, kw.get("n_seg", 0)), dtype=torch.uint8,
                         device=dev)
        want = _run(lambda *a, **k: ob.onebit_server_reduce_ex(*a, ws=ws, **k), bits, scales,
                    ef, sv_scales, N, n, **kw)
        got = _run(ob.onebit_server_reduce_noalloc, bits, scales, ef, sv_scales, N, n, **kw)
        torch.cuda.synchronize()
        _same(got, want, f"seed={seed} call={call}")


def test_noalloc_at_the_scratch_limit():
    """16 workers with chunks of 2^27 elements need exactly 2^20 partial sums,
    the scratch's whole size: the call is accepted and equals the workspace
    form (a chunk one 64-element group longer is refused on the host)."""
    dev = device()
    n, L = 16, 1 << 27
    N = n * L
    free = torch.cuda.mem_get_info()[0]
    if free < 60 * (1 << 30):
        pytest.skip("not enough device memory for two 2^31-element server calls")
    print(f"[noalloc limit] N={N} n={n}", flush=True)
    bits, scales, ef, sv_scales = _inputs(N, n, 77, dev)
    ws = torch.empty(ob.workspace_bytes(N, n, 0), dtype=torch.uint8, device=dev)
    want = _run(lambda *a, **k: ob.onebit_server_reduce_ex(*a, ws=ws, **k), bits, scales, ef,
                sv_scales, N, n, reset=False, flags=0)
    del ws
    got = _run(ob.onebit_server_reduce_noalloc, bits, scales, ef, sv_scales, N, n, reset=False,
               flags=0)
    torch.cuda.synchronize()
    _same(got, want, "at the limit")
