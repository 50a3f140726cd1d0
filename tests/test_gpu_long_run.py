"""A long free-running 1-bit Adam run against the C++ oracle: 3000 steps
with the clamp on and the periodic error reset every 1000 steps (1-bit Adam
article, sections 2.1 and 4.1), so that the carried worker and server
errors accumulate over a thousand compressions between resets. Every
step's sign words, scales, compensated values and parameters are compared
bit for bit, so a drift at any step is caught where it starts."""

import numpy as np
import pytest
import torch

from momentum_compression_amd.state import OneBitGroup
from oracle import cref as R
from tests._gpu import device, gen, host

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]
F32 = np.float32


def _eq(got, want, what):
    g, w = np.ascontiguousarray(got), np.ascontiguousarray(want)
    assert g.shape == w.shape and np.array_equal(g.view(np.uint32), w.view(np.uint32)), what


def test_three_thousand_steps_with_resets():
    dev = device()
    n, L = 8, 3 * 1024 + 64
    N, steps, R_int, clip, lr, eps = n * L, 3000, 1000, 2e-3, 6e-5, 1e-6
    print(f"[long run] n={n} N={N} steps={steps} reset every {R_int}", flush=True)
    grp = OneBitGroup(N, n, dev, clip=clip, reset_interval=R_int)
    g0 = gen(4242, dev)
    x = torch.randn(N, generator=g0, device=dev) * 0.02
    v = torch.rand(N, generator=g0, device=dev) * 1e-6 + 1e-8
    x_h, v_h = host(x).copy(), host(v)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    m = torch.empty((n, N), device=dev)
    for t in range(1, steps + 1):
        # momenta of a slowly moving scale, so the errors carry real content
        m.normal_(0.0, 1e-3 * (1.0 + 0.5 * np.sin(t / 97.0)), generator=g0)
        first = t == 1
        reset = first or grp.is_reset(t)
        grp.compress(m, t, first=first)
        grp.server(t, first=first, decompress=False)
        grp.adam_step_packed(x, v, lr, eps, decompress=True)
        torch.cuda.synchronize()
        w = R.worker_compress(host(m), e, clip=clip, reset=reset)
        sv = R.server_reduce(w["bits"], w["s"], E, reset=reset)
        mbar = R.decompress(sv["bits"], sv["S"])
        x_h = R.adam_frozen_step(x_h, mbar, v_h, lr, eps)
        tag = f"t={t}{' (reset)' if reset else ''}"
        _eq(host(grp.bits), w["bits"], f"{tag} worker sign words")
        _eq(host(grp.scales), w["s"], f"{tag} worker scales")
        _eq(host(grp.ef), w["gc"], f"{tag} worker compensated values")
        _eq(host(grp.sv_bits), sv["bits"], f"{tag} server sign words")
        _eq(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        _eq(host(grp.sv_ef), sv["g2"], f"{tag} server compensated values")
        _eq(host(grp.mbar), mbar, f"{tag} decompressed momentum")
        _eq(host(x), x_h, f"{tag} parameters")
        e, E = w["e"], sv["E"]
        if t % 500 == 0:
            print(f"[long run] t={t} ok", flush=True)
    # the errors stayed bounded by the clamp's range between resets
    assert np.all(np.abs(e) <= 2 * clip) and np.all(np.isfinite(E))


def test_lamb_thousand_steps_step_ratio_chained():
    """1-bit LAMB on the BERT-Large layer structure scaled down (every
    tensor kept, 303 layers), 8 workers, 1000 steps: the step ratio
    c_{t-1}/c_t written by each step's LAMB pass scales the next step's
    carried errors at both levels (1-bit LAMB page, analysis paragraph), the
    clipped ratio r_t moves every step, and m_{t-1} is the previous step's
    decompressed momentum. Every step bit for bit against the C++ oracle."""
    from momentum_compression_amd.state import LambState, momentum_scale
    from workloads import configs as C
    from workloads import synth as S

    dev = device()
    wl = C.scaled_lamb(n=8, target_elems=1 << 16, seed=11)
    N, n = wl.N, wl.n
    steps = 1000
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    print(f"[long lamb] N={N} n={n} layers={len(off) - 1} steps={steps}", flush=True)
    off_d = torch.from_numpy(off).to(dev)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    m_tw = S.lamb_prev_momentum(wl, dev, sig)
    k_d = momentum_scale(m_tw, off_d)
    k_el = np.repeat(host(k_d), np.diff(off)).astype(F32)
    c_avg = S.lamb_c_avg(wl)
    st = LambState.create(S.params(wl, dev), S.frozen_variance(wl, dev), m_tw, off_d,
                          torch.from_numpy(c_avg).to(dev))
    grp = OneBitGroup(N, n, dev, seg_off=off_d, seg_k=k_d, seg_err_ratio=st.err_ratio)
    hp = (wl.lr, wl.eps, wl.beta1, wl.beta2, 0.5, 0.1, 10.0)  # a wide clip: c moves
    x_h, vf_h, mp_h = host(st.x).copy(), host(st.v_fresh).copy(), host(st.m_prev).copy()
    r_h, c_h, v_tw = host(st.r).copy(), host(st.c).copy(), host(st.v_frozen)
    rho = np.ones(len(off) - 1, dtype=F32)
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    m = torch.empty((n, N), device=dev)
    g0 = gen(77, dev)
    for t in range(1, steps + 1):
        m.normal_(0.0, 1.0, generator=g0)
        m.mul_(sig)
        first = t == 1
        grp.compress(m, t, first=first)
        grp.server(t, first=first, decompress=False)
        st.step_packed(grp.sv_bits, grp.sv_scales, k_d, n, *hp)
        torch.cuda.synchronize()
        rho_el = np.repeat(rho, np.diff(off)).astype(F32)
        w = R.worker_compress(host(m), e, reset=first, k=k_el, err_ratio=None if first else rho_el)
        sv = R.server_reduce(w["bits"], w["s"], E, reset=first,
                             err_ratio=None if first else rho_el)
        mbar = R.decompress(sv["bits"], sv["S"], k_el)
        out = R.lamb_frozen_step(x_h, mbar, mp_h, vf_h, v_tw, off, c_avg, r_h, c_h, *hp)
        tag = f"t={t}"
        _eq(host(grp.bits), w["bits"], f"{tag} worker sign words")
        _eq(host(grp.scales), w["s"], f"{tag} worker scales")
        _eq(host(grp.sv_bits), sv["bits"], f"{tag} server sign words")
        _eq(host(grp.sv_scales), sv["S"], f"{tag} server scales")
        _eq(host(st.m_prev), mbar, f"{tag} decompressed momentum / k")
        _eq(host(st.x), out["x"], f"{tag} parameters")
        _eq(host(st.v_fresh), out["v"], f"{tag} fresh variance")
        _eq(host(st.r), out["r"], f"{tag} r_t")
        _eq(host(st.c), out["c"], f"{tag} c_t")
        _eq(host(st.err_ratio), out["err_ratio"], f"{tag} step ratio")
        x_h, vf_h, r_h, c_h, mp_h = out["x"], out["v"], out["r"], out["c"], mbar
        e, E, rho = w["e"], sv["E"], out["err_ratio"]
        if t % 250 == 0:
            print(f"[long lamb] t={t} ok", flush=True)


def test_int8_two_thousand_steps_error_feedback():
    """Block-wise INT8 stochastic rounding with error feedback over 2000
    steps (gradient-quantisation tutorial, "FP32 -> INT8" and the error
    feedback of its 1-bit section): the residual of every step is added to
    the next gradient, and each step draws fresh Philox uniforms keyed by
    the step. Codes, scales, dequantised values and residuals bit for bit
    against the C++ oracle at every step."""
    from momentum_compression_amd import onebit as ob

    dev = device()
    N, block, steps, seed = 256 * 997, 256, 2000, 0x5EED_0F_1B17
    print(f"[long int8] N={N} block={block} steps={steps}", flush=True)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    g = torch.empty(N, device=dev)
    g0 = gen(91, dev)
    e_h = np.zeros(N, dtype=F32)
    for t in range(1, steps + 1):
        g.normal_(0.0, 1e-3, generator=g0)
        ob.int8_sr_quantize(g, err, codes, scales, deq, N, block, seed, t)
        torch.cuda.synchronize()
        o = R.int8_sr(host(g), e_h, seed, t, block=block)
        tag = f"t={t}"
        assert np.array_equal(host(codes), o["codes"]), f"{tag} codes"
        _eq(host(scales), o["scales"], f"{tag} scales")
        _eq(host(deq), o["deq"], f"{tag} dequantised")
        _eq(host(err), o["e"], f"{tag} residual")
        e_h = o["e"]
        if t % 500 == 0:
            print(f"[long int8] t={t} ok", flush=True)
    # the residual stays below one quantisation step of its block
    assert np.all(np.abs(e_h) <= np.repeat(host(scales), block) * (1 + 2.0 ** -20))


def test_lamb_warmup_five_hundred_steps():
    """500 uncompressed LAMB warmup steps on the scaled 303-layer BERT
    structure (1-bit LAMB page, algorithm paragraph: warmup before the
    compressed phase), the coefficient average carried from step to step,
    then the per-layer momentum scale k_l at the end (layer-scaling
    paragraph). Every step's x, m, v, c and c_avg, and k_l, bit for bit
    against the C++ oracle."""
    from momentum_compression_amd import onebit as ob
    from momentum_compression_amd.state import LambWarmup
    from workloads import configs as C
    from workloads import synth as S

    dev = device()
    wl = C.scaled_lamb(n=8, target_elems=1 << 16, seed=12)
    N = wl.N
    steps = 500
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    print(f"[long warmup] N={N} layers={len(off) - 1} steps={steps}", flush=True)
    off_d = torch.from_numpy(off).to(dev)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    hp = dict(lr=1e-3, eps=1e-6, beta1=0.9, beta2=0.999)
    x0 = S.params(wl, dev)
    st = LambWarmup.create(x0.clone(), off_d)
    xh, mh, vh, cav = host(x0).copy(), np.zeros(N, F32), np.zeros(N, F32), None
    g = torch.empty(N, device=dev)
    g0 = gen(13, dev)
    for t in range(1, steps + 1):
        g.normal_(0.0, 1.0, generator=g0)
        g.mul_(sig)
        st.step(g, beta_c=0.9, **hp)
        torch.cuda.synchronize()
        o = R.lamb_warmup_step(xh, mh, vh, host(g), off, c_avg=cav, beta_c=0.9, **hp)
        for name in ("x", "m", "v", "c", "c_avg"):
            _eq(host(getattr(st, name)), o[name], f"t={t} {name}")
        xh, mh, vh, cav = o["x"], o["m"], o["v"], o["c_avg"]
        if t % 100 == 0:
            print(f"[long warmup] t={t} ok", flush=True)
    k = torch.empty(len(off) - 1, device=dev)
    ws = torch.empty(ob.warmup_workspace_bytes(N, len(off) - 1), dtype=torch.uint8, device=dev)
    ob.lamb_momentum_scale(st.m, N, off_d, len(off) - 1, k, ws)
    torch.cuda.synchronize()
    _eq(host(k), R.momentum_scale(mh, off), "k_l")
