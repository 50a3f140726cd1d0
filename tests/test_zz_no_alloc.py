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
