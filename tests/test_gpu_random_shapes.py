"""GPU parity over seeded random shapes and options: worker counts 1..64
(the compile-time 8 and 16 and the general form), chunk lengths from one
64-element group to several tiles with a ragged tail, random layer tables
(empty layers, edges inside a float4 and a sign word), clamp, reset, the
unscaled sign, the layer coefficient, and the decompression inside the Adam
pass.  Three free-running steps each, against the oracle."""

import os

import numpy as np
import pytest
import torch

from momentum_compression_amd.state import OneBitGroup
from oracle import onebit as O
from oracle import optim as P
from tests._gpu import device, gen, host, same_bits, same_f32

pytestmark = pytest.mark.gpu
F32 = np.float32


def _seeds(default: int) -> range:
    """The seeds of this family: `default` of them, or more when
    ONEBIT_RANDOM_SEEDS asks for a wider campaign."""
    return range(max(default, int(os.environ.get("ONEBIT_RANDOM_SEEDS", "0"))))


def _config(seed):
    rng = np.random.default_rng(seed)
    n = [1, 2, 3, 5, 7, 8, 11, 16, 24, 33, 64, 8, 16, 4, 6, 13][seed % 16]
    L = 64 * int(rng.integers(1, 3 * 16 + 7))  # 64 .. about 3.4 tiles
    N = n * L
    seg = bool(rng.integers(0, 2))
    off = None
    if seg:
        cuts = np.sort(rng.integers(0, N + 1, size=int(rng.integers(1, 9))))
        off = np.concatenate([[0], cuts, [N]]).astype(np.int64)
    return dict(n=n, L=L, N=N, seg=seg, off=off,
                clip=float(rng.choice([0.0, 0.0, 1.5e-3])),
                R=int(rng.choice([0, 2])),
                unit=seed % 5 == 3,
                scale=float(10.0 ** rng.uniform(-5, -1)))


@pytest.mark.parametrize("seed", _seeds(16))
def test_random_shape(seed):
    cfg = _config(seed)
    n, N, off = cfg["n"], cfg["N"], cfg["off"]
    dev = device()
    print(f"[random shape] seed={seed} n={n} L={cfg['L']} layers="
          f"{None if off is None else len(off) - 1} clip={cfg['clip']} R={cfg['R']} "
          f"unit={cfg['unit']}", flush=True)
    k = k_el = None
    if off is not None:
        k = np.exp(np.random.default_rng(seed + 100).uniform(-2, 2, len(off) - 1)).astype(F32)
        k_el = O.per_element_k(off, k)
    grp = OneBitGroup(N, n, dev, clip=cfg["clip"], reset_interval=cfg["R"],
                      seg_off=None if off is None else torch.from_numpy(off).to(dev),
                      seg_k=None if k is None else torch.from_numpy(k).to(dev),
                      unit_scale=cfg["unit"])
    gx = gen(seed + 500, dev)
    x = torch.randn(N, generator=gx, device=dev) * 0.02
    v = torch.rand(N, generator=gx, device=dev) * 1e-6 + 1e-8
    x_h, v_h = host(x).copy(), host(v)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    for t in range(1, 4):
        m = torch.randn((n, N), generator=gen(seed * 100 + t, dev), device=dev) * cfg["scale"]
        grp.compress(m, t, first=t == 1)
        grp.server(t, first=t == 1, decompress=False)
        grp.adam_step_packed(x, v, 6e-5, 1e-6, decompress=True)
        torch.cuda.synchronize()
        reset = t == 1 or (cfg["R"] > 0 and t % cfg["R"] == 0)
        w = O.worker_compress(host(m), e, clip=cfg["clip"], reset=reset, k=k_el,
                              unit_scale=cfg["unit"])
        sv = O.server_reduce(w["bits"], w["s"], E, reset=reset, unit_scale=cfg["unit"])
        mbar = O.decompress(sv["bits"], sv["S"], k=k_el)
        # the Adam step reads the global momentum before / k (the x k of the
        # compress side is undone only for the LAMB path)
        x_h = P.adam_frozen_step(x_h, O.decompress(sv["bits"], sv["S"]), v_h, 6e-5, 1e-6)
        tag = f"seed={seed} t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.scales), w["s"], f"{tag} worker scales")
        same_f32(host(grp.ef), w["gc"], f"{tag} worker state")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        same_f32(host(grp.sv_ef), sv["g2"], f"{tag} server state")
        same_f32(host(x), x_h, f"{tag} parameters")
        if off is None:
            same_f32(host(grp.mbar), mbar, f"{tag} decompressed")
        e, E = w["e"], sv["E"]
