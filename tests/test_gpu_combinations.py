"""GPU parity over the option combinations of the 1-bit stage: layer table
(x k_l before compression, / k_l after), step-ratio-scaled error feedback
(needs the layer table), clamp, compression fed with gradients (local
momentum from the previous packed global momentum) and the unscaled sign.
Every combination the entry points accept runs three free-running steps
against the oracle on a small ragged buffer whose layer edges fall inside
float4 quads and inside sign words."""

import itertools

import numpy as np
import pytest
import torch

from momentum_compression_amd.state import OneBitGroup
from oracle import onebit as O
from tests._gpu import device, gen, host, same_bits, same_f32

pytestmark = pytest.mark.gpu
F32 = np.float32

N_WORKERS = 4
L = 3 * 1024 + 64          # chunk: three tiles and a ragged tail
N = N_WORKERS * L
OFF = np.array([0, 6, 1030, 1031 + 1, 5000, 5002, 9999 + 1, N], dtype=np.int64)
BETA1 = 0.9
CLIP = 2.5e-3              # binds for a few percent of the elements


def _combos():
    for seg, ers, clamp, mom, unit in itertools.product([False, True], repeat=5):
        if ers and not seg:
            continue  # the step-ratio factor is per layer
        yield seg, ers, clamp, mom, unit


@pytest.mark.parametrize("seg,ers,clamp,mom,unit", list(_combos()))
def test_option_combination(seg, ers, clamp, mom, unit):
    dev = device()
    tag0 = f"seg={seg} ers={ers} clamp={clamp} mom={mom} unit={unit}"
    print(f"[combination] N={N} n={N_WORKERS} {tag0}", flush=True)
    g0 = gen(1000 + 32 * seg + 16 * ers + 8 * clamp + 4 * mom + 2 * unit, dev)
    S_ = len(OFF) - 1
    k = np.exp(np.linspace(-3.0, 3.0, S_)).astype(F32)
    rho = np.linspace(0.5, 2.0, S_).astype(F32)
    k_el = O.per_element_k(OFF, k)
    rho_el = O.per_element_k(OFF, rho)
    grp = OneBitGroup(N, N_WORKERS, dev, clip=CLIP if clamp else 0.0,
                      seg_off=torch.from_numpy(OFF).to(dev) if seg else None,
                      seg_k=torch.from_numpy(k).to(dev) if seg else None,
                      unit_scale=unit,
                      seg_err_ratio=torch.from_numpy(rho).to(dev) if ers else None)
    e = np.zeros((N_WORKERS, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    mbar = np.zeros(N, dtype=F32)
    for t in range(1, 4):
        x = (torch.randn((N_WORKERS, N), generator=g0, device=dev) * 1e-3).contiguous()
        first = t == 1
        if mom:
            grp.compress_grad(x, t, BETA1, first=first)
            m = O.local_momentum(host(x), mbar, BETA1)
        else:
            grp.compress(x, t, first=first)
            m = host(x)
        grp.server(t, first=first)
        torch.cuda.synchronize()
        w = O.worker_compress(m, e, clip=CLIP if clamp else 0.0, reset=first,
                              k=k_el if seg else None, unit_scale=unit,
                              err_ratio=rho_el if ers else None)
        sv = O.server_reduce(w["bits"], w["s"], E, reset=first, unit_scale=unit,
                             err_ratio=rho_el if ers else None)
        mbar = O.decompress(sv["bits"], sv["S"], k=k_el if seg else None)
        tag = f"{tag0} t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.scales), w["s"], f"{tag} worker scales")
        same_f32(host(grp.ef), w["gc"], f"{tag} worker state")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        same_f32(host(grp.sv_ef), sv["g2"], f"{tag} server state")
        same_f32(host(grp.mbar), mbar, f"{tag} decompressed")
        e, E = w["e"], sv["E"]
