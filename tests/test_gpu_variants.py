"""GPU parity of the variants: unscaled +-1 signs, step-ratio-scaled error
feedback chained from the LAMB step, INT8 round-to-nearest and per-tensor
scale."""

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import LambState, OneBitGroup
from oracle import onebit as O
from oracle import optim as P
from oracle.int8 import int8_sr
from tests._gpu import device, gen, host, same_bits, same_f32
from workloads import configs as C
from workloads import synth as S

pytestmark = pytest.mark.gpu
F32 = np.float32


def test_unit_scale_free_running():
    dev = device()
    n, L = 4, 2048 + 320
    N = n * L
    print(f"[unit scale] N={N} n={n}", flush=True)
    grp = OneBitGroup(N, n, dev, unit_scale=True)
    g0 = gen(41, dev)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    for t in range(1, 5):
        m = torch.randn((n, N), generator=g0, device=dev) * 0.5
        first = t == 1
        grp.compress(m, t, first=first)
        grp.server(t, first=first)
        torch.cuda.synchronize()
        w = O.worker_compress(host(m), e, reset=first, unit_scale=True)
        sv = O.server_reduce(w["bits"], w["s"], E, reset=first, unit_scale=True)
        same_bits(host(grp.bits), w["bits"], f"t={t} worker bits")
        same_f32(host(grp.scales), w["s"], f"t={t} worker scales")
        same_f32(host(grp.worker_error()), w["e"], f"t={t} worker error")
        same_bits(host(grp.sv_bits), sv["bits"], f"t={t} server bits")
        same_f32(host(grp.server_error()), sv["E"], f"t={t} server error")
        same_f32(host(grp.mbar), O.decompress(sv["bits"], sv["S"]), f"t={t} decompressed")
        e, E = w["e"], sv["E"]


@pytest.mark.parametrize("n", [8, 16, 5])
def test_lamb_step_ratio_error_feedback_chained(n):
    """The LAMB step writes c_{t-1}/c_t per layer; the next compression and
    server reduce scale the carried errors by it.  n = 8 and 16 run the
    server kernels specialised for those worker counts, n = 5 the general
    one."""
    dev = device()
    wl = C.scaled_lamb(n=n, target_elems=1 << 20, seed=9)
    N, n = wl.N, wl.n
    print(f"[step-ratio EF] N={N} n={n} segments={len(wl.segments)}", flush=True)
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    k, c_avg = S.lamb_tables(wl)
    k_el = O.per_element_k(off, k)
    off_d, k_d = torch.from_numpy(off).to(dev), torch.from_numpy(k).to(dev)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    st = LambState.create(S.params(wl, dev), S.frozen_variance(wl, dev),
                          S.lamb_prev_momentum(wl, dev, sig), off_d, torch.from_numpy(c_avg).to(dev))
    grp = OneBitGroup(N, n, dev, seg_off=off_d, seg_k=k_d, seg_err_ratio=st.err_ratio)
    x_h, v_h, vf_h, mp_h = host(st.x).copy(), host(st.v_frozen), host(st.v_frozen).copy(), \
        host(st.m_prev).copy()
    r_h, c_h = np.ones(len(k), dtype=F32), c_avg.copy()
    rho = np.ones(len(k), dtype=F32)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    # r_min/r_max wide and thr large so that c_t moves and the ratio differs from 1
    hp = dict(lr=wl.lr, eps=wl.eps, beta1=wl.beta1, beta2=wl.beta2, thr=0.5, r_min=0.1, r_max=10.0)
    for t in range(1, 5):
        m = S.momentum(wl, t, dev, sigma_elem=sig)
        first = t == 1
        grp.compress(m, t, first=first)
        grp.server(t, first=first)
        st.step(grp.mbar, **hp)
        torch.cuda.synchronize()
        rho_el = O.per_element_k(off, rho)
        w = O.worker_compress(host(m), e, reset=first, k=k_el, err_ratio=rho_el)
        sv = O.server_reduce(w["bits"], w["s"], E, reset=first, err_ratio=rho_el)
        mbar = O.decompress(sv["bits"], sv["S"], k=k_el)
        out = P.lamb_frozen_step(x_h, mbar, mp_h, vf_h, v_h, off, c_avg, r_h, c_h, hp["lr"],
                                 hp["eps"], hp["beta1"], hp["beta2"], hp["thr"], hp["r_min"],
                                 hp["r_max"])
        tag = f"t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.worker_error()), w["e"], f"{tag} worker error")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.server_error()), sv["E"], f"{tag} server error")
        same_f32(host(st.x), out["x"], f"{tag} parameters")
        same_f32(host(st.err_ratio), out["err_ratio"], f"{tag} error ratio")
        if t >= 2:
            assert np.any(out["err_ratio"] != 1)
        x_h, vf_h, r_h, c_h, rho = out["x"], out["v"], out["r"], out["c"], out["err_ratio"]
        e, E, mp_h = w["e"], sv["E"], mbar
        st.m_prev.copy_(grp.mbar)


@pytest.mark.parametrize("block,rounding", [(256, 1), (1024, 1), (0, 0), (0, 1), (64, 1)])
def test_int8_variants(block, rounding):
    dev = device()
    N = 256 * 997 if block <= 256 else block * 251  # not a multiple of the 1024-element tile
    print(f"[int8 variant] N={N} block={block} rounding={rounding}", flush=True)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(max(1, N // block) if block else 1, device=dev)
    deq = torch.empty(N, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    e_h = np.zeros(N, dtype=F32)
    for step in range(1, 4):
        g = S.laplace_gradient(N, step, 8, dev)
        if step == 2:
            g[100:140] = torch.arange(40, device=dev, dtype=torch.float32) * 0.5  # halves
        ob.int8_quantize(g, err, codes, scales, deq, N, block, rounding, 77, step, ws=ws)
        torch.cuda.synchronize()
        o = int8_sr(host(g), e_h, 77, step, block=block,
                    rounding="nearest" if rounding else "stochastic")
        assert np.array_equal(host(codes), o["codes"]), f"step {step} codes"
        same_f32(host(scales), o["scales"], f"step {step} scales")
        same_f32(host(deq), o["deq"], f"step {step} deq")
        same_f32(host(err), o["e"], f"step {step} residual")
        e_h = o["e"]


@pytest.mark.parametrize("with_err", [True, False])
def test_int8_tensor_scale_grid_stride(with_err):
    """Per-tensor scale on a tensor long enough that every workgroup of the
    max pass strides over it more than once; the maximum sits in the ragged
    last span."""
    dev = device()
    N = 2 * 2048 * 4096 + 4 * 333
    print(f"[int8 tensor scale] N={N} err={with_err}", flush=True)
    g = S.laplace_gradient(N, 3, 8, dev)
    g[N - 3] = -4.0  # far above the x100 outliers of the Laplace(1e-3) draw
    g[N // 2] = 2.0
    err = torch.zeros(N, device=dev) if with_err else None
    if with_err:
        err[N - 7] = 3.875  # g' = 3.875 + g, below 4
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(1, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    e_h = host(err) if with_err else None
    ob.int8_quantize(g, err, codes, scales, None, N, 0, 1, 5, 1, ws=ws)
    torch.cuda.synchronize()
    o = int8_sr(host(g), e_h, 5, 1, block=0, rounding="nearest")
    assert host(scales)[0] == o["scales"][0] == np.float32(4.0) / np.float32(127)
    assert np.array_equal(host(codes), o["codes"])
    if with_err:
        same_f32(host(err), o["e"], "residual")
