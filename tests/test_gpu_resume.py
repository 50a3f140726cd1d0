"""Checkpoint and resume on the GPU: T steps in one run equal k steps, a
checkpoint written to disk, a fresh state loaded from it and T - k more
steps, bit for bit (error states, scales, packed global momentum,
parameters, LAMB tables).  The Adam run crosses an error reset after the
resume; the LAMB run takes its momentum from the server's sign words."""

import numpy as np
import pytest
import torch

from momentum_compression_amd import checkpoint as ck
from momentum_compression_amd.state import LambState, OneBitGroup
from tests._gpu import device, gen, host
from workloads import configs as C
from workloads import synth as S

pytestmark = pytest.mark.gpu


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


def _adam_steps(grp, x, v, t0, t1, dev, N, n):
    for t in range(t0, t1):
        m = torch.randn((n, N), generator=gen(100 + t, dev), device=dev) * 1e-3
        grp.compress(m, t, first=t == 1)
        grp.server(t, first=t == 1, decompress=False)
        grp.adam_step_packed(x, v, 1e-3, 1e-6, decompress=True)


def test_adam_resume_bit_exact(tmp_path):
    dev = device()
    N, n, T, k = 8 * 3136, 8, 7, 3
    print(f"[resume adam] N={N} n={n} T={T} k={k}", flush=True)
    cfg = dict(clip=2.5e-3, reset_interval=5)
    v = torch.rand(N, generator=gen(1, dev), device=dev) * 1e-6
    x0 = torch.randn(N, generator=gen(2, dev), device=dev)
    a = OneBitGroup(N, n, dev, **cfg)
    xa = x0.clone()
    _adam_steps(a, xa, v, 1, T + 1, dev, N, n)
    b = OneBitGroup(N, n, dev, **cfg)
    xb = x0.clone()
    _adam_steps(b, xb, v, 1, k + 1, dev, N, n)
    ck.save(str(tmp_path), {**b.state_dict(), "x": xb}, meta={"t": k, "group": b.config()})
    del b, xb
    tens, meta = ck.load(str(tmp_path), dev)
    c = OneBitGroup.from_state(tens, meta["group"], dev)
    xc = tens["x"]
    _adam_steps(c, xc, v, meta["t"] + 1, T + 1, dev, N, n)
    torch.cuda.synchronize()
    assert _same(xa, xc), "parameters"
    for name in OneBitGroup._STATE:
        assert _same(getattr(a, name), getattr(c, name)), name


@pytest.mark.parametrize("keep_prev", [False, True])
def test_lamb_resume_bit_exact(tmp_path, keep_prev):
    """keep_prev: from the second step on the LAMB step reads m_{t-1} as the
    previous step's server words, which the checkpoint carries."""
    dev = device()
    wl = C.scaled_lamb(n=16, target_elems=1 << 20)
    N, n, T, k = wl.N, wl.n, 5, 2
    print(f"[resume lamb] N={N} n={n} segments={len(wl.segments)} T={T} k={k} "
          f"keep_prev={keep_prev}", flush=True)
    off = torch.from_numpy(np.array(C.segment_offsets(wl.segments), dtype=np.int64)).to(dev)
    kk, c_avg = S.lamb_tables(wl)
    k_d, c_d = torch.from_numpy(kk).to(dev), torch.from_numpy(c_avg).to(dev)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    hp = dict(lr=wl.lr, eps=wl.eps, beta1=wl.beta1, beta2=wl.beta2, thr=wl.r_threshold,
              r_min=wl.r_min, r_max=wl.r_max)
    x0, v0 = S.params(wl, dev), S.frozen_variance(wl, dev)
    mp0 = S.lamb_prev_momentum(wl, dev, sig)

    def run(grp, st, t0, t1):
        for t in range(t0, t1):
            m = S.momentum(wl, t, dev, sigma_elem=sig)
            grp.seg_err_ratio = st.err_ratio if t > 1 else None
            grp.compress(m, t, first=t == 1)
            grp.server(t, first=t == 1, decompress=False)
            prev = {}
            if grp.keep_prev and t > 1:
                prev = dict(prev_bits=grp.sv_bits_prev, prev_scales=grp.sv_scales_prev)
            st.step_packed(grp.sv_bits, grp.sv_scales, k_d, n, **hp, **prev)

    a = OneBitGroup(N, n, dev, seg_off=off, seg_k=k_d, keep_prev=keep_prev)
    sa = LambState.create(x0.clone(), v0, mp0.clone(), off, c_d.clone())
    run(a, sa, 1, T + 1)
    b = OneBitGroup(N, n, dev, seg_off=off, seg_k=k_d, keep_prev=keep_prev)
    sb = LambState.create(x0.clone(), v0, mp0.clone(), off, c_d.clone())
    run(b, sb, 1, k + 1)
    b.seg_err_ratio = None  # the ratio lives in the LAMB state
    ck.save(str(tmp_path / "group"), b.state_dict(), meta={"t": k, "group": b.config()})
    ck.save(str(tmp_path / "lamb"), sb.state_dict())
    del b, sb
    tg, meta = ck.load(str(tmp_path / "group"), dev)
    tl, _ = ck.load(str(tmp_path / "lamb"), dev)
    c = OneBitGroup.from_state(tg, meta["group"], dev)
    sc = LambState.from_state(tl)
    run(c, sc, meta["t"] + 1, T + 1)
    torch.cuda.synchronize()
    assert c.keep_prev == keep_prev
    for name in a._state_names():
        assert _same(getattr(a, name), getattr(c, name)), name
    for name in LambState._STATE:
        assert _same(getattr(sa, name), getattr(sc, name)), name
