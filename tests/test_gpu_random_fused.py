"""GPU parity of the fused paths over seeded random shapes and options: the
compression fed with gradients (each worker's momentum formed from its
gradient and the previous packed global momentum, 1-bit Adam article,
section 2.1), then the server and the decompression inside the Adam pass;
or, with a random layer table and coefficients, the 1-bit LAMB step on the
decompressed momentum divided by k_l (1-bit LAMB page, algorithm and
layer-scaling paragraphs). Worker counts 1..64, ragged chunk lengths,
clamp, periodic reset, the unscaled sign and random beta1; four
free-running steps each, against the oracle."""

import os

import numpy as np
import pytest
import torch

from momentum_compression_amd.state import LambState, OneBitGroup
from oracle import onebit as O
from oracle import optim as P
from tests._gpu import device, gen, host, same_bits, same_f32

pytestmark = pytest.mark.gpu
F32 = np.float32
STEPS = 4


def _seeds(default: int) -> range:
    """`default` seeds, or more when ONEBIT_RANDOM_SEEDS asks for a wider
    campaign."""
    return range(max(default, int(os.environ.get("ONEBIT_RANDOM_SEEDS", "0"))))


def _config(seed):
    rng = np.random.default_rng(9000 + seed)
    n = [1, 2, 3, 4, 5, 8, 12, 16, 33, 64][seed % 10]
    L = 64 * int(rng.integers(1, 64))
    N = n * L
    lamb = bool(rng.integers(0, 2))
    off = k = None
    if lamb:
        cuts = np.sort(rng.integers(0, N + 1, size=int(rng.integers(1, 12))))
        off = np.concatenate([[0], cuts, [N]]).astype(np.int64)
        k = np.exp(rng.uniform(-2, 2, len(off) - 1)).astype(F32)
    return dict(n=n, L=L, N=N, lamb=lamb, off=off, k=k,
                clip=0.0 if lamb else float(rng.choice([0.0, 0.0, 2e-3])),
                R=int(rng.choice([0, 2, 3])), unit=seed % 6 == 4,
                beta1=float(rng.choice([0.9, 0.5, 0.99])),
                scale=float(10.0 ** rng.uniform(-4, -2)))


@pytest.mark.parametrize("seed", _seeds(16))
def test_random_fused(seed):
    cfg = _config(seed)
    n, N, off, k, beta1 = cfg["n"], cfg["N"], cfg["off"], cfg["k"], cfg["beta1"]
    dev = device()
    print(f"[random fused] seed={seed} n={n} L={cfg['L']} lamb={cfg['lamb']} "
          f"layers={None if off is None else len(off) - 1} clip={cfg['clip']} R={cfg['R']} "
          f"unit={cfg['unit']} beta1={beta1}", flush=True)
    k_el = None if k is None else O.per_element_k(off, k)
    off_d = None if off is None else torch.from_numpy(off).to(dev)
    k_d = None if k is None else torch.from_numpy(k).to(dev)
    grp = OneBitGroup(N, n, dev, clip=cfg["clip"], reset_interval=cfg["R"], seg_off=off_d,
                      seg_k=k_d, unit_scale=cfg["unit"])
    g0 = gen(seed + 700, dev)
    x = torch.randn(N, generator=g0, device=dev) * 0.02
    v = torch.rand(N, generator=g0, device=dev) * 1e-6 + 1e-8
    lr, eps = 6e-5, 1e-6
    hp = (lr, eps, beta1, 0.999, 0.1, 0.5, 4.0)
    if cfg["lamb"]:
        c_avg = np.exp(np.random.default_rng(seed).uniform(-0.5, 0.5, len(k))).astype(F32)
        st = LambState.create(x.clone(), v.clone(), torch.zeros(N, device=dev), off_d,
                              torch.from_numpy(c_avg).to(dev))
        x_h, v_h, vf_h = host(st.x).copy(), host(st.v_frozen), host(st.v_frozen).copy()
        r_h, c_h = np.ones(len(k), dtype=F32), c_avg.copy()
    else:
        x_h, v_h = host(x).copy(), host(v)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    mbar = np.zeros(N, dtype=F32)
    for t in range(1, STEPS + 1):
        gr = torch.randn((n, N), generator=g0, device=dev) * cfg["scale"]
        first = t == 1
        reset = first or grp.is_reset(t)
        grp.compress_grad(gr, t, beta1, first=first)
        if cfg["lamb"]:
            grp.server(t, first=first, decompress=True)
            st.step(grp.mbar, *hp)
        else:
            grp.server(t, first=first, decompress=False)
            grp.adam_step_packed(x, v, lr, eps)
        torch.cuda.synchronize()
        m = O.local_momentum(host(gr), mbar, beta1)
        w = O.worker_compress(m, e, clip=cfg["clip"], reset=reset, k=k_el,
                              unit_scale=cfg["unit"])
        sv = O.server_reduce(w["bits"], w["s"], E, reset=reset, unit_scale=cfg["unit"])
        mbar_new = O.decompress(sv["bits"], sv["S"], k=k_el)
        tag = f"seed={seed} t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.scales), w["s"], f"{tag} worker scales")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        if cfg["lamb"]:
            out = P.lamb_frozen_step(x_h, mbar_new, mbar, vf_h, v_h, off, c_avg, r_h, c_h, *hp)
            same_f32(host(grp.mbar), mbar_new, f"{tag} m / k")
            same_f32(host(st.x), out["x"], f"{tag} parameters")
            same_f32(host(st.c), out["c"], f"{tag} c_t")
            x_h, vf_h, r_h, c_h = out["x"], out["v"], out["r"], out["c"]
            st.m_prev.copy_(grp.mbar)  # this step's momentum is the next step's m_{t-1}
        else:
            x_h = P.adam_frozen_step(x_h, mbar_new, v_h, lr, eps)
            same_f32(host(x), x_h, f"{tag} parameters")
        mbar, e, E = mbar_new, w["e"], sv["E"]
