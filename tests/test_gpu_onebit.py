"""GPU parity of the 1-bit worker/server path and the Adam step against the
CPU oracle, called through the C ABI.  Multi-step runs are free-running: the
GPU's error state evolves on its own and must stay bit-identical to the
oracle's, which requires exact chunk scales (a one-ulp scale difference
flips later signs)."""

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import OneBitGroup
from oracle import onebit as O
from oracle import optim as P
from tests._gpu import device, gen, host, same_bits, same_f32

pytestmark = pytest.mark.gpu
F32 = np.float32


def _momentum(shape, t, seed, dev, scale=1e-3, mode="normal"):
    g = gen(seed * 1000 + t, dev)
    if mode == "normal":
        return torch.randn(shape, generator=g, device=dev) * scale
    if mode == "mixed":  # per-row log-uniform spread plus exact zeros
        x = torch.randn(shape, generator=g, device=dev)
        sig = torch.exp(torch.rand((shape[0], 1), generator=g, device=dev) * 7 - 12)
        x = x * sig
        x[:, ::97] = 0.0
        return x
    raise ValueError(mode)


def run_adam(N, n, steps, clip=0.0, R=0, t0=1, seed=1, mode="normal", scale=1e-3, lr=6e-5,
             eps=1e-6, inject=None):
    dev = device()
    print(f"[adam parity] N={N} n={n} steps={steps} clip={clip} R={R} t0={t0} seed={seed} mode={mode}",
          flush=True)
    grp = OneBitGroup(N, n, dev, clip=clip, reset_interval=R)
    gx = gen(seed + 77, dev)
    x = torch.randn(N, generator=gx, device=dev) * 0.02
    v = torch.randn(N, generator=gx, device=dev).abs() * 1e-6 + 1e-8
    x_h, v_h = host(x).copy(), host(v)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    for t in range(t0, t0 + steps):
        m = _momentum((n, N), t, seed, dev, scale, mode)
        if inject is not None:
            inject(m, t)
        m_h = host(m)
        first = t == t0
        grp.compress(m, t, first=first)
        grp.server(t, first=first)
        grp.adam_step(x, v, lr, eps)
        torch.cuda.synchronize()
        reset = first or (R > 0 and t % R == 0)
        w = O.worker_compress(m_h, e, clip=clip, reset=reset)
        sv = O.server_reduce(w["bits"], w["s"], E, reset=reset)
        mbar = O.decompress(sv["bits"], sv["S"])
        x_h = P.adam_frozen_step(x_h, mbar, v_h, lr, eps)
        tag = f"t={t}"
        same_bits(host(grp.bits), w["bits"], f"{tag} worker bits")
        same_f32(host(grp.scales), w["s"], f"{tag} worker scales")
        same_f32(host(grp.ef), w["gc"], f"{tag} worker compensated")
        same_f32(host(grp.worker_error()), w["e"], f"{tag} worker error")
        same_bits(host(grp.sv_bits), sv["bits"], f"{tag} server bits")
        same_f32(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        same_f32(host(grp.sv_ef), sv["g2"], f"{tag} server compensated")
        same_f32(host(grp.server_error()), sv["E"], f"{tag} server error")
        same_f32(host(grp.mbar), mbar, f"{tag} decompressed momentum")
        same_f32(host(x), x_h, f"{tag} parameters")
        e, E = w["e"], sv["E"]


def test_adam_small_free_running():
    # L = 5 tiles of 1024 + a ragged 320, 4 workers, 6 steps
    run_adam(N=4 * (5 * 1024 + 320), n=4, steps=6)


def test_adam_eight_workers_mixed_scales():
    run_adam(N=8 * (3 * 1024 + 64), n=8, steps=4, mode="mixed", seed=5)


def test_adam_clamp_binding():
    # momentum well beyond the clip value on every step
    run_adam(N=4 * 2048, n=4, steps=4, clip=2e-3, scale=3e-3, seed=2)


def test_adam_reset_crossing():
    # starts at t = 1998 with reset every 2000 steps: the reset fires at t = 2000
    run_adam(N=4 * 1088, n=4, steps=4, R=2000, t0=1998, seed=3)


@pytest.mark.parametrize("n,L", [(1, 1024 * 3), (3, 2368), (5, 64), (64, 192), (16, 1024)])
def test_adam_worker_counts(n, L):
    run_adam(N=n * L, n=n, steps=3, seed=10 + n)


def test_specials_nan_inf_zero_denormal():
    def inject(m, t):
        m[0, 0] = float("nan")
        m[1, 5] = float("inf")
        m[2, 7] = float("-inf")
        m[3, :64] = 0.0          # whole first word zero
        m[3, 64:128] = -0.0
        m[2, 200:300] = 3e-42     # subnormals
    run_adam(N=4 * 1024, n=4, steps=3, inject=inject, seed=4)


def test_all_zero_chunks():
    dev = device()
    N, n = 4 * 1024, 4
    grp = OneBitGroup(N, n, dev)
    m = torch.zeros((n, N), device=dev)
    grp.compress(m, 1, first=True)
    grp.server(1, first=True)
    torch.cuda.synchronize()
    assert np.all(host(grp.scales) == 0) and np.all(host(grp.sv_scales) == 0)
    assert np.all(host(grp.bits) == 0xFFFFFFFF) and np.all(host(grp.mbar) == 0)


def test_exact_tie_takes_exact_path():
    """Chunk means that are exact binary32 midpoints (ties to even), among
    normal values, subnormals and values near the top of the range, and
    means within one unit of the last place of a midpoint."""
    dev = device()
    n, L = 4, 2048
    N = n * L
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2), dtype=F32)
    m_h = np.empty((n, N), dtype=F32)
    m_h[:, 0::2] = one
    m_h[:, 1::2] = -up            # mean |.| = 1 + 2^-24: a tie, rounds to 1
    m_h[1, :L] *= np.float32(2.0 ** -130)  # the same tie among subnormals
    m_h[0, L:2 * L] *= np.float32(2.0 ** 126)  # and among values near 2^126
    m_h[2, 3] = -np.nextafter(up, np.float32(2), dtype=F32)  # mean just above the tie
    m_h[3, L:2 * L] = np.float32(3.0)
    m_h[3, L] = np.float32(3.0 + 2 ** -22)  # mean 3 + 2^-33: not a tie, close to 3
    grp = OneBitGroup(N, n, dev)
    m = torch.from_numpy(m_h).to(dev)
    grp.compress(m, 1, first=True)
    grp.server(1, first=True)
    torch.cuda.synchronize()
    w = O.worker_compress(m_h, np.zeros_like(m_h), reset=True)
    same_f32(host(grp.scales), w["s"], "tie scales")
    assert host(grp.scales)[0, 0] == one
    assert host(grp.scales)[0, 1] == np.float32(2.0 ** 126)
    sv = O.server_reduce(w["bits"], w["s"], np.zeros(N, dtype=F32), reset=True)
    same_f32(host(grp.sv_scales), sv["S"], "tie server scales")
    same_bits(host(grp.sv_bits), sv["bits"], "tie server bits")



def test_mean_within_binary64_error_of_a_midpoint():
    """Chunk means a hair above and a hair below a binary32 midpoint, closer
    than binary64 can tell: the fp64 partial sums land on the midpoint
    itself, the certified rounding must find the decision ambiguous and the
    exact path must round the true value (up, and down)."""
    dev = device()
    n, L = 2, 2048
    N = n * L
    F = np.float32
    m_h = np.zeros((n, N), dtype=F)
    m_h[:, L:] = F(0.5)
    # worker 0, chunk 0: (2^11 + 2^-13 + 2^-100) / 2^11 = 1 + 2^-24 + 2^-111 -> up
    m_h[0, :3] = [2.0 ** 11, 2.0 ** -13, -(2.0 ** -100)]
    # worker 1, chunk 0: (2^11 + 3 2^-13 - 2^-59) / 2^11 = 1 + 3 2^-24 - 2^-70 -> down
    m_h[1, :3] = [-(2.0 ** 11), np.nextafter(F(3 * 2.0 ** -13), F(0)),
                  np.nextafter(F(2.0 ** -35), F(0))]
    print("[mean near midpoint] n=2 L=2048", flush=True)
    grp = OneBitGroup(N, n, dev)
    m = torch.from_numpy(m_h).to(dev)
    grp.compress(m, 1, first=True)
    torch.cuda.synchronize()
    s = host(grp.scales)
    assert s[0, 0] == F(1 + 2.0 ** -23) and s[1, 0] == F(1 + 2.0 ** -23)
    w = O.worker_compress(m_h, np.zeros_like(m_h), reset=True)
    same_f32(s, w["s"], "scales")


def test_zero_size_is_a_noop():
    dev = device()
    t = torch.zeros(16, device=dev)
    w = torch.zeros(16, dtype=torch.int32, device=dev)
    q = torch.zeros(16, dtype=torch.int8, device=dev)
    ob.onebit_compress(t, t, t, w, 0, 4, ws=None)
    ob.int8_sr_quantize(t, None, q, t, None, 0, 256, 1, 1)
    ob.frozen_v_step(mode=0, N=0, x=t, m=t, v=t, lr=1.0, eps=0.0)
    torch.cuda.synchronize()
    assert torch.all(t == 0) and torch.all(w == 0) and torch.all(q == 0)


def test_invalid_arguments_rejected_before_launch():
    dev = device()
    grp = OneBitGroup(4 * 1024, 4, dev)
    m = torch.zeros((4, 4 * 1024), device=dev)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress(m, grp.ef, grp.scales, grp.bits, 4 * 1000, 4, ws=grp.ws)
    assert ei.value.status == ob.ONEBIT_E_SIZE
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress(m, grp.ef, grp.scales, grp.bits, 4 * 1024, 4, ws=grp.ws[:8])
    assert ei.value.status == ob.ONEBIT_E_WORKSPACE
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress(m.view(-1)[1:].data_ptr(), grp.ef, grp.scales, grp.bits, 4 * 1024, 4,
                           ws=grp.ws)
    assert ei.value.status == ob.ONEBIT_E_ALIGN


def test_deterministic_across_runs():
    dev = device()
    N, n = 8 * 4096, 8
    outs = []
    for _ in range(2):
        grp = OneBitGroup(N, n, dev)
        for t in (1, 2, 3):
            m = _momentum((n, N), t, 9, dev)
            grp.compress(m, t, first=t == 1)
            grp.server(t, first=t == 1)
        torch.cuda.synchronize()
        outs.append([host(a).copy() for a in (grp.bits, grp.scales, grp.ef, grp.sv_bits,
                                              grp.sv_scales, grp.sv_ef, grp.mbar)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_decompress_entry_matches_server_output():
    dev = device()
    N, n = 4 * 2048, 4
    grp = OneBitGroup(N, n, dev)
    grp.compress(_momentum((n, N), 1, 3, dev), 1, first=True)
    grp.server(1, first=True)
    out = torch.empty(N, device=dev)
    ob.onebit_decompress(grp.sv_bits, grp.sv_scales, out, N, n)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), host(grp.mbar).view(np.uint32))
