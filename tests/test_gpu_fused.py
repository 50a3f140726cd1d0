"""GPU parity of the fused entry points: compression fed with gradients (the
local momentum update formed from the previous packed global momentum) and
the Adam step reading the global momentum packed."""

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import LambState, OneBitGroup
from oracle import onebit as O
from oracle import optim as P
from tests._gpu import device, gen, host, same_bits, same_f32
from workloads import configs as C
from workloads import synth as S

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.mark.parametrize("n,L,clip", [(4, 3 * 1024 + 64, 0.0), (8, 1024, 1e-3), (3, 2368, 0.0)])
def test_adam_from_gradients_free_running(n, L, clip):
    dev = device()
    N, beta1, lr, eps = n * L, 0.9, 6e-5, 1e-6
    print(f"[fused adam] N={N} n={n} clip={clip}", flush=True)
    grp = OneBitGroup(N, n, dev, clip=clip)
    g0 = gen(31 + n, dev)
    x = torch.randn(N, generator=g0, device=dev) * 0.02
    v = torch.randn(N, generator=g0, device=dev).abs() * 1e-6 + 1e-8
    x_h, v_h = host(x).copy(), host(v)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    mbar = np.zeros(N, dtype=F32)
    for t in range(1, 6):
        gr = torch.randn((n, N), generator=g0, device=dev) * 1e-3
        first = t == 1
        grp.compress_grad(gr, t, beta1, first=first)
        grp.server(t, first=first, decompress=False)
        grp.adam_step_packed(x, v, lr, eps)
        torch.cuda.synchronize()
        m = O.local_momentum(host(gr), mbar, beta1)
        w = O.worker_compress(m, e, clip=clip, reset=first)
        sv = O.server_reduce(w["bits"], w["s"], E, reset=first)
        mbar = O.decompress(sv["bits"], sv["S"])
        x_h = P.adam_frozen_step(x_h, mbar, v_h, lr, eps)
        tag = f"t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.scales), w["s"], f"{tag} worker scales")
        same_f32(host(grp.ef), w["gc"], f"{tag} worker compensated")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        same_f32(host(x), x_h, f"{tag} parameters")
        e, E = w["e"], sv["E"]


def test_packed_adam_equals_decompress_then_adam():
    dev = device()
    N, n = 8 * 2048, 8
    grp = OneBitGroup(N, n, dev)
    g0 = gen(5, dev)
    grp.compress(torch.randn((n, N), generator=g0, device=dev) * 1e-3, 1, first=True)
    grp.server(1, first=True, decompress=True)
    x = torch.randn(N, generator=g0, device=dev)
    v = torch.rand(N, generator=g0, device=dev) * 1e-6
    x2 = x.clone()
    x3 = x.clone()
    grp.adam_step(x, v, 1e-3, 1e-6)
    grp.adam_step_packed(x2, v, 1e-3, 1e-6)
    mbar = grp.mbar.clone()
    grp.mbar.fill_(float("nan"))
    grp.adam_step_packed(x3, v, 1e-3, 1e-6, decompress=True)   # also writes mbar
    torch.cuda.synchronize()
    assert np.array_equal(host(x).view(np.uint32), host(x2).view(np.uint32))
    assert np.array_equal(host(x).view(np.uint32), host(x3).view(np.uint32))
    assert np.array_equal(host(grp.mbar).view(np.uint32), host(mbar).view(np.uint32))
    sv_bits, S = host(grp.sv_bits), host(grp.sv_scales)
    same_f32(host(grp.mbar), O.decompress(sv_bits, S), "decompressed by the step")


def test_lamb_from_gradients():
    """1-bit LAMB fed with gradients: the previous global momentum is
    decompressed with / k_l, updated with the gradient, scaled by k_l."""
    dev = device()
    wl = C.scaled_lamb(n=8, target_elems=1 << 20, seed=6)
    N, n, beta1 = wl.N, wl.n, wl.beta1
    print(f"[fused lamb] N={N} n={n} segments={len(wl.segments)}", flush=True)
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    k, c_avg = S.lamb_tables(wl)
    k_el = O.per_element_k(off, k)
    off_d, k_d = torch.from_numpy(off).to(dev), torch.from_numpy(k).to(dev)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    grp = OneBitGroup(N, n, dev, seg_off=off_d, seg_k=k_d)
    st = LambState.create(S.params(wl, dev), S.frozen_variance(wl, dev),
                          torch.zeros(N, device=dev), off_d, torch.from_numpy(c_avg).to(dev))
    x_h, v_h, vf_h = host(st.x).copy(), host(st.v_frozen), host(st.v_frozen).copy()
    r_h, c_h = np.ones(len(k), dtype=F32), c_avg.copy()
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    mbar = np.zeros(N, dtype=F32)
    for t in range(1, 4):
        gr = S.momentum(wl, t, dev, sigma_elem=sig)  # gradient stand-in, same recipe
        first = t == 1
        grp.compress_grad(gr, t, beta1, first=first)
        grp.server(t, first=first, decompress=True)
        st.step(grp.mbar, wl.lr, wl.eps, wl.beta1, wl.beta2, wl.r_threshold, wl.r_min, wl.r_max)
        torch.cuda.synchronize()
        m = O.local_momentum(host(gr), mbar, beta1)
        w = O.worker_compress(m, e, reset=first, k=k_el)
        sv = O.server_reduce(w["bits"], w["s"], E, reset=first)
        mbar_new = O.decompress(sv["bits"], sv["S"], k=k_el)
        out = P.lamb_frozen_step(x_h, mbar_new, mbar, vf_h, v_h, off, c_avg, r_h, c_h, wl.lr,
                                 wl.eps, wl.beta1, wl.beta2, wl.r_threshold, wl.r_min, wl.r_max)
        tag = f"t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.scales), w["s"], f"{tag} worker scales")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.mbar), mbar_new, f"{tag} m / k")
        same_f32(host(st.x), out["x"], f"{tag} parameters")
        same_f32(host(st.c), out["c"], f"{tag} c_t")
        x_h, vf_h, r_h, c_h = out["x"], out["v"], out["r"], out["c"]
        e, E, mbar = w["e"], sv["E"], mbar_new
        st.m_prev.copy_(grp.mbar)


def test_invalid_fused_arguments():
    dev = device()
    grp = OneBitGroup(4 * 1024, 4, dev)
    g = torch.zeros((4, 4 * 1024), device=dev)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress_grad(g, None, grp.sv_scales, 0.9, grp.ef, grp.scales, grp.bits,
                                4 * 1024, 4, ws=grp.ws)
    assert ei.value.status == ob.ONEBIT_E_NULL
