"""GPU parity over seeded random configurations at medium sizes, whole
buffers against the C++ oracle: chunks from 4K to 2M elements (several
compress iterations per workgroup, finalizes over thousands of partials, both
server plans), worker counts 1..64, random layer tables with coefficients,
the step-ratio error at both levels, clamp, periodic reset and the unscaled
sign, with the decompression inside the Adam pass. Three free-running steps
each; every worker and server output and every parameter bit-identical."""

import os

import numpy as np
import pytest
import torch

from momentum_compression_amd.state import OneBitGroup
from oracle import cref as R
from tests._gpu import device, gen, host, same_whole

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]
F32 = np.float32


def _seeds(default: int) -> range:
    """The seeds of this family: `default` of them, or more when
    ONEBIT_RANDOM_SEEDS asks for a wider campaign."""
    return range(max(default, int(os.environ.get("ONEBIT_RANDOM_SEEDS", "0"))))


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    n = [1, 2, 3, 4, 5, 8, 12, 16, 17, 32, 48, 64][seed % 12]
    L = 64 * int(np.exp(rng.uniform(np.log(64), np.log(1 << 15))))  # 4K .. 2M
    if seed in (0, 4):  # the largest chunks: a whole and a ragged 2M
        L = (1 << 21) - 64 * seed
    while n * n * L > (1 << 28):  # at most 2^28 worker elements (n * N)
        L //= 2
    L -= L % 64
    N = n * L
    off = None
    if rng.integers(0, 3):
        cuts = np.sort(rng.integers(0, N + 1, size=int(rng.integers(1, 40))))
        off = np.concatenate([[0], cuts, [N]]).astype(np.int64)
    return dict(n=n, L=L, N=N, off=off,
                clip=float(rng.choice([0.0, 0.0, 2e-3])),
                R=int(rng.choice([0, 2, 3])),
                unit=seed % 7 == 5,
                ers=off is not None and bool(rng.integers(0, 2)),
                scale=float(10.0 ** rng.uniform(-5, -1)))


@pytest.mark.parametrize("seed", _seeds(24))
def test_random_medium(seed):
    cfg = _config(seed)
    n, N, off = cfg["n"], cfg["N"], cfg["off"]
    dev = device()
    print(f"[random medium] seed={seed} n={n} L={cfg['L']} layers="
          f"{None if off is None else len(off) - 1} clip={cfg['clip']} R={cfg['R']} "
          f"unit={cfg['unit']} ers={cfg['ers']}", flush=True)
    rng = np.random.default_rng(seed + 7)
    k = k_el = ratio = ratio_el = None
    if off is not None:
        k = np.exp(rng.uniform(-2, 2, len(off) - 1)).astype(F32)
        k_el = np.repeat(k, np.diff(off)).astype(F32)
    grp = OneBitGroup(N, n, dev, clip=cfg["clip"], reset_interval=cfg["R"],
                      seg_off=None if off is None else torch.from_numpy(off).to(dev),
                      seg_k=None if k is None else torch.from_numpy(k).to(dev),
                      unit_scale=cfg["unit"])
    gx = gen(seed + 900, dev)
    x = torch.randn(N, generator=gx, device=dev) * 0.02
    v = torch.rand(N, generator=gx, device=dev) * 1e-6 + 1e-8
    x_h, v_h = host(x).copy(), host(v)
    e = E = None
    for t in range(1, 4):
        if cfg["ers"]:  # a new factor per layer every step, as the LAMB step writes it
            ratio = (1 + 0.2 * rng.standard_normal(len(k))).astype(F32)
            ratio_el = np.repeat(ratio, np.diff(off)).astype(F32)
            grp.seg_err_ratio = torch.from_numpy(ratio).to(dev)
        m = torch.randn((n, N), generator=gen(seed * 100 + t, dev), device=dev) * cfg["scale"]
        grp.compress(m, t, first=t == 1)
        grp.server(t, first=t == 1, decompress=False)
        grp.adam_step_packed(x, v, 6e-5, 1e-6, decompress=True)
        torch.cuda.synchronize()
        reset = t == 1 or (cfg["R"] > 0 and t % cfg["R"] == 0)
        w = R.worker_compress(host(m), e, clip=cfg["clip"], reset=reset, k=k_el,
                              unit_scale=cfg["unit"], err_ratio=ratio_el, threads=16)
        sv = R.server_reduce(w["bits"], w["s"], E, reset=reset, unit_scale=cfg["unit"],
                             err_ratio=ratio_el, threads=16)
        # the Adam pass decodes the server words without / k (the LAMB path divides)
        mbar = R.decompress(sv["bits"], sv["S"])
        x_h = R.adam_frozen_step(x_h, mbar, v_h, 6e-5, 1e-6)
        tag = f"seed={seed} t={t}"
        same_whole(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_whole(host(grp.scales), w["s"], f"{tag} worker scales")
        same_whole(host(grp.ef), w["gc"], f"{tag} worker state")
        same_whole(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_whole(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        same_whole(host(grp.sv_ef), sv["g2"], f"{tag} server state")
        same_whole(host(grp.mbar), mbar, f"{tag} decompressed")
        same_whole(host(x), x_h, f"{tag} parameters")
        e, E = w["e"], sv["E"]
