"""GPU parity over seeded random configurations of the 1-bit LAMB path and of
INT8, whole buffers against the C++ oracle.

LAMB: random worker counts, chunk lengths and layer tables (up to 60 cuts,
empty layers, edges inside a float4 and a sign word), coefficients k_l and
c_avg, both readings of the coefficient (c_{t-1} or c_t), the step-ratio
error chained from the LAMB step into both compression levels, and the LAMB
step from the sign words with m_{t-1} packed from the second step on. Four
free-running steps: the workers, the server, x, the fresh variance and every
layer's R, r_t, c_t and c_{t-1}/c_t.

INT8: random lengths, every block size and the per-tensor scale, both
roundings, with and without error feedback, random 64-bit seeds and steps;
two steps, every code, scale, dequantised value and residual.
"""

import os

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import LambState, OneBitGroup
from oracle import cref as R
from tests._gpu import device, gen, host, same_whole

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]
F32 = np.float32


def _seeds(default: int) -> range:
    """The seeds of this family: `default` of them, or more when
    ONEBIT_RANDOM_SEEDS asks for a wider campaign."""
    return range(max(default, int(os.environ.get("ONEBIT_RANDOM_SEEDS", "0"))))


def _lamb_config(seed):
    rng = np.random.default_rng(2000 + seed)
    n = [1, 3, 4, 8, 13, 16, 32, 64][seed % 8]
    L = 64 * int(np.exp(rng.uniform(np.log(16), np.log(1 << 13))))
    while n * n * L > (1 << 27):
        L //= 2
    L -= L % 64
    N = n * L
    cuts = np.sort(rng.integers(0, N + 1, size=int(rng.integers(1, 61))))
    off = np.concatenate([[0], cuts, [N]]).astype(np.int64)
    return dict(n=n, L=L, N=N, off=off, use_c_t=bool(rng.integers(0, 2)),
                scale=float(10.0 ** rng.uniform(-5, -2)))


@pytest.mark.parametrize("seed", _seeds(16))
def test_random_lamb(seed):
    cfg = _lamb_config(seed)
    n, N, off = cfg["n"], cfg["N"], cfg["off"]
    S = len(off) - 1
    dev = device()
    print(f"[random lamb] seed={seed} n={n} L={cfg['L']} layers={S} use_c_t={cfg['use_c_t']}",
          flush=True)
    rng = np.random.default_rng(seed + 11)
    k = np.exp(rng.uniform(-2, 2, S)).astype(F32)
    k_el = np.repeat(k, np.diff(off)).astype(F32)
    c_avg = np.exp(rng.uniform(-1, 1, S)).astype(F32)
    off_d, k_d = torch.from_numpy(off).to(dev), torch.from_numpy(k).to(dev)
    grp = OneBitGroup(N, n, dev, seg_off=off_d, seg_k=k_d, keep_prev=True)
    gx = gen(seed + 300, dev)
    x = torch.randn(N, generator=gx, device=dev) * 0.02
    v_tw = torch.rand(N, generator=gx, device=dev) * 1e-6 + 1e-9
    m_prev = torch.randn(N, generator=gx, device=dev) * cfg["scale"]
    st = LambState.create(x, v_tw, m_prev.clone(), off_d, torch.from_numpy(c_avg).to(dev))
    x_h, vf_h, vtw_h, mp_h = host(x).copy(), host(v_tw).copy(), host(v_tw), host(m_prev).copy()
    r_h, c_h = np.ones(S, dtype=F32), c_avg.copy()
    e = E = None
    rho_el = None
    hp = (1e-3, 1e-6, 0.9, 0.999, 0.1, 0.5, 4.0)
    for t in range(1, 5):
        first = t == 1
        grp.seg_err_ratio = None if first else st.err_ratio
        m = torch.randn((n, N), generator=gen(seed * 100 + t, dev), device=dev) * cfg["scale"]
        grp.compress(m, t, first=first)
        grp.server(t, first=first, decompress=False)
        prev = {} if first else dict(prev_bits=grp.sv_bits_prev, prev_scales=grp.sv_scales_prev)
        st.step_packed(grp.sv_bits, grp.sv_scales, k_d, n, *hp, use_c_t=cfg["use_c_t"], **prev)
        torch.cuda.synchronize()
        w = R.worker_compress(host(m), e, reset=first, k=k_el, err_ratio=rho_el, threads=16)
        sv = R.server_reduce(w["bits"], w["s"], E, reset=first, err_ratio=rho_el, threads=16)
        mbar = R.decompress(sv["bits"], sv["S"], k_el)
        out = R.lamb_frozen_step(x_h, mbar, mp_h, vf_h, vtw_h, off, c_avg, r_h, c_h, *hp,
                                 use_c_t=cfg["use_c_t"])
        tag = f"seed={seed} t={t}"
        same_whole(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_whole(host(grp.scales), w["s"], f"{tag} worker scales")
        same_whole(host(grp.ef), w["gc"], f"{tag} worker state")
        same_whole(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_whole(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        same_whole(host(grp.sv_ef), sv["g2"], f"{tag} server state")
        same_whole(host(st.x), out["x"], f"{tag} parameters")
        same_whole(host(st.v_fresh), out["v"], f"{tag} fresh variance")
        same_whole(host(st.ratio_max), out["R"], f"{tag} layer max ratio")
        same_whole(host(st.r), out["r"], f"{tag} r_t")
        same_whole(host(st.c), out["c"], f"{tag} c_t")
        same_whole(host(st.err_ratio), out["err_ratio"], f"{tag} c_(t-1)/c_t")
        if first or cfg["use_c_t"]:  # the decompressed momentum is written
            same_whole(host(st.m_prev), mbar, f"{tag} decompressed momentum / k")
        x_h, vf_h, r_h, c_h, mp_h = out["x"], out["v"], out["r"], out["c"], mbar
        e, E = w["e"], sv["E"]
        rho_el = np.repeat(out["err_ratio"], np.diff(off)).astype(F32)


def _int8_config(seed):
    rng = np.random.default_rng(3000 + seed)
    block = [0, 64, 128, 256, 512, 1024][seed % 6]
    unit = block or 4
    N = unit * int(np.exp(rng.uniform(np.log(1), np.log((1 << 24) // unit))))
    return dict(N=N, block=block, rounding=int(rng.integers(0, 2)), ef=bool(rng.integers(0, 3)),
                seed=int(rng.integers(0, 2**63)), step=int(rng.integers(0, 2**32)))


@pytest.mark.parametrize("seed", _seeds(24))
def test_random_int8(seed):
    cfg = _int8_config(seed)
    N, block = cfg["N"], cfg["block"]
    dev = device()
    print(f"[random int8] seed={seed} N={N} block={block} rounding={cfg['rounding']} "
          f"ef={cfg['ef']}", flush=True)
    nb = N // block if block else 1
    err = torch.zeros(N, device=dev) if cfg["ef"] else None
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(nb, device=dev)
    deq = torch.empty(N, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    e_ref = np.zeros(N, dtype=F32) if cfg["ef"] else None
    g_gen = gen(seed + 40, dev)
    for i in range(2):
        step = (cfg["step"] + i) & 0xFFFFFFFF
        g = torch.randn(N, generator=g_gen, device=dev) * 1e-3
        g[:: 997] *= 100  # outliers
        ob.int8_quantize(g, err, codes, scales, deq, N, block, cfg["rounding"], cfg["seed"], step,
                         ws=ws)
        torch.cuda.synchronize()
        o = R.int8_sr(host(g), e_ref, cfg["seed"], step, block,
                      rounding=("stochastic", "nearest")[cfg["rounding"]], threads=16)
        tag = f"seed={seed} step={i}"
        same_whole(host(codes), o["codes"], f"{tag} codes")
        same_whole(host(scales), o["scales"], f"{tag} scales")
        same_whole(host(deq), o["deq"], f"{tag} dequantised")
        if cfg["ef"]:
            same_whole(host(err), o["e"], f"{tag} residual")
            e_ref = o["e"]
