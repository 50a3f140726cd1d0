"""Parity at the workloads' full sizes, in the launch configuration the bench
times (the library derives its launch plan from N and n alone).  The oracle
checks sampled worker chunks end to end (free-running over the steps run),
server chunks in lock-step (the GPU's worker words and scales as inputs),
and the parameter step on samples or on the whole buffer."""

import gc

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import LambState, OneBitGroup
from oracle import onebit as O
from oracle import optim as P
from oracle.int8 import int8_sr
from tests._gpu import device, host, same_bits, same_f32
from workloads import configs as C
from workloads import synth as S

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
F32 = np.float32


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _need(dev, nbytes):
    free = torch.cuda.mem_get_info(dev)[0]
    if free < nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} free")


def _chunk_words(c, L):
    return slice(c * L // 32, (c + 1) * L // 32)


def _run_adam_fullsize(wl, steps, pairs, server_chunks, t0=1, sample=1 << 20):
    dev = device()
    N, n, L = wl.N, wl.n, wl.L
    _need(dev, int(n * N * 4 * 2.2 + N * 4 * 6))
    print(f"[fullsize] {wl.name} N={N} n={n} steps={steps} t0={t0}", flush=True)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    grp = OneBitGroup(N, n, dev, clip=wl.clip, reset_interval=wl.reset_interval)
    x = S.params(wl, dev)
    v = S.frozen_variance(wl, dev)
    m = torch.empty((n, N), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(0)
    idx = np.sort(rng.choice(N, size=sample, replace=False))
    idx_d = torch.from_numpy(idx).to(dev)
    e_w = {p: np.zeros(L, dtype=F32) for p in pairs}
    E_s = {c: np.zeros(L, dtype=F32) for c in server_chunks}
    for t in range(t0, t0 + steps):
        S.momentum(wl, t, dev, sigma_elem=sig, out=m)
        first = t == t0
        reset = first or grp.is_reset(t)
        x_before = host(x[idx_d])
        grp.compress(m, t, first=first)
        grp.server(t, first=first)
        grp.adam_step(x, v, wl.lr, wl.eps)
        torch.cuda.synchronize()
        tag = f"{wl.name} t={t}"
        scales = host(grp.scales)
        for (i, c) in pairs:
            sl = slice(c * L, (c + 1) * L)
            w = O.worker_compress(host(m[i, sl])[None, :], e_w[(i, c)][None, :], clip=wl.clip,
                                  reset=reset)
            same_f32(np.array([scales[i, c]]), w["s"][0, :1], f"{tag} scale[{i},{c}]")
            same_bits(host(grp.bits[i, _chunk_words(c, L)]), w["bits"][0], f"{tag} bits[{i},{c}]")
            same_f32(host(grp.ef[i, sl]), w["gc"][0], f"{tag} state[{i},{c}]")
            e_w[(i, c)] = w["e"][0]
        sv_scales = host(grp.sv_scales)
        for c in server_chunks:
            sl = slice(c * L, (c + 1) * L)
            r = O.server_chunk(host(grp.bits[:, _chunk_words(c, L)]), scales[:, c], E_s[c],
                               reset=reset)
            same_f32(np.array([sv_scales[c]]), np.array([r["S"]]), f"{tag} server scale[{c}]")
            same_bits(host(grp.sv_bits[_chunk_words(c, L)]), r["bits"], f"{tag} server bits[{c}]")
            same_f32(host(grp.sv_ef[sl]), r["g2"], f"{tag} server state[{c}]")
            same_f32(host(grp.mbar[sl]), O.decompress(r["bits"], np.array([r["S"]], dtype=F32)),
                     f"{tag} decompressed[{c}]")
            E_s[c] = r["E"]
        x_want = P.adam_frozen_step(x_before, host(grp.mbar[idx_d]), host(v[idx_d]), wl.lr, wl.eps)
        same_f32(host(x[idx_d]), x_want, f"{tag} parameters (sampled)")
    del grp, x, v, m, sig
    _free()


def test_bert_large_335M_x8_bench_configuration():
    wl = C.get("bert_large_335M_x8")
    _run_adam_fullsize(wl, steps=3, pairs=[(0, 0), (3, 5), (7, 7)], server_chunks=[0, 5])


def test_gpt_1_3B_x16_clamp_and_reset():
    """The reset interval (2000) is crossed: t = 1999 (first step), 2000
    (periodic reset), 2001; the 2.0 clamp is on."""
    wl = C.get("gpt_1.3B_x16")
    _run_adam_fullsize(wl, steps=3, pairs=[(0, 0), (15, 9)], server_chunks=[9], t0=1999,
                       sample=1 << 18)


def test_bert_large_lamb_302t_x16():
    """Two 1-bit LAMB steps on the 302-tensor buffer; the LAMB step is
    checked on the whole buffer (every layer's ratio, r_t, c_t, x, v).  A
    second state stepping from the server's sign words (decompression inside
    the LAMB pass) must match it bit for bit on the whole buffer."""
    dev = device()
    wl = C.get("bert_large_lamb_302t_x16")
    N, n, L = wl.N, wl.n, wl.L
    _need(dev, int(n * N * 4 * 2.2 + N * 4 * 12))
    print(f"[fullsize] {wl.name} N={N} n={n} segments={len(wl.segments)}", flush=True)
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    k, c_avg = S.lamb_tables(wl)
    k_el = O.per_element_k(off, k)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    off_d, k_d = torch.from_numpy(off).to(dev), torch.from_numpy(k).to(dev)
    grp = OneBitGroup(N, n, dev, seg_off=off_d, seg_k=k_d)
    st = LambState.create(S.params(wl, dev), S.frozen_variance(wl, dev),
                          S.lamb_prev_momentum(wl, dev, sig), off_d, torch.from_numpy(c_avg).to(dev))
    st2 = LambState.create(st.x.clone(), st.v_frozen, st.m_prev.clone(), off_d,
                           torch.from_numpy(c_avg).to(dev))
    m = torch.empty((n, N), dtype=torch.float32, device=dev)
    pairs = [(0, 0), (9, 15)]
    e_w = {p: np.zeros(L, dtype=F32) for p in pairs}
    E_c = np.zeros(L, dtype=F32)
    csrv = 15
    v_h = host(st.v_frozen)
    for t in (1, 2):
        S.momentum(wl, t, dev, sigma_elem=sig, out=m)
        first = t == 1
        x_h, vf_h, mp_h = host(st.x).copy(), host(st.v_fresh).copy(), host(st.m_prev).copy()
        r_h, c_h = host(st.r).copy(), host(st.c).copy()
        grp.compress(m, t, first=first)
        grp.server(t, first=first)
        st.step(grp.mbar, wl.lr, wl.eps, wl.beta1, wl.beta2, wl.r_threshold, wl.r_min, wl.r_max)
        st2.step_packed(grp.sv_bits, grp.sv_scales, k_d, n, wl.lr, wl.eps, wl.beta1, wl.beta2,
                        wl.r_threshold, wl.r_min, wl.r_max)
        torch.cuda.synchronize()
        tag = f"lamb t={t}"
        scales = host(grp.scales)
        for (i, c) in pairs:
            sl = slice(c * L, (c + 1) * L)
            w = O.worker_compress(host(m[i, sl])[None, :], e_w[(i, c)][None, :], reset=first,
                                  k=k_el[sl])
            same_f32(np.array([scales[i, c]]), w["s"][0, :1], f"{tag} scale[{i},{c}]")
            same_bits(host(grp.bits[i, _chunk_words(c, L)]), w["bits"][0], f"{tag} bits[{i},{c}]")
            e_w[(i, c)] = w["e"][0]
        sl = slice(csrv * L, (csrv + 1) * L)
        r = O.server_chunk(host(grp.bits[:, _chunk_words(csrv, L)]), scales[:, csrv], E_c, reset=first)
        same_f32(np.array([host(grp.sv_scales)[csrv]]), np.array([r["S"]]), f"{tag} server scale")
        same_bits(host(grp.sv_bits[_chunk_words(csrv, L)]), r["bits"], f"{tag} server bits")
        same_f32(host(grp.mbar[sl]),
                 O.decompress(r["bits"], np.array([r["S"]], dtype=F32), k=k_el[sl]), f"{tag} m / k")
        E_c = r["E"]
        out = P.lamb_frozen_step(x_h, host(grp.mbar), mp_h, vf_h, v_h, off, c_avg, r_h, c_h,
                                 wl.lr, wl.eps, wl.beta1, wl.beta2, wl.r_threshold, wl.r_min,
                                 wl.r_max)
        same_f32(host(st.ratio_max), out["R"], f"{tag} layer max ratio")
        same_f32(host(st.r), out["r"], f"{tag} r_t")
        same_f32(host(st.c), out["c"], f"{tag} c_t")
        same_f32(host(st.v_fresh), out["v"], f"{tag} fresh variance")
        same_f32(host(st.x), out["x"], f"{tag} parameters")
        st.m_prev.copy_(grp.mbar)
        for name in ("x", "v_fresh", "ratio_max", "r", "c", "err_ratio", "m_prev"):
            assert torch.equal(getattr(st, name).view(torch.int32),
                               getattr(st2, name).view(torch.int32)), f"{tag} packed {name}"
        del out, x_h, vf_h, mp_h
    del grp, st, st2, m, sig
    _free()


def test_int8_2_30_with_error_feedback():
    dev = device()
    N, block, seed = 1 << 30, 256, 4
    _need(dev, N * 18)
    print(f"[fullsize] int8 N={N}", flush=True)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    g = torch.empty(N, device=dev)
    ranges = [0, (N // 2) - 4096, N - (1 << 20)]
    e_prev = {a: np.zeros(1 << 20, dtype=F32) for a in ranges}
    for step in (1, 2):
        S.laplace_gradient(N, step, seed, dev, out=g)
        ob.int8_sr_quantize(g, err, codes, scales, deq, N, block, seed, step)
        torch.cuda.synchronize()
        for a in ranges:
            sl = slice(a, a + (1 << 20))
            o = int8_sr(host(g[sl]), e_prev[a], seed, step, block, J0=a)
            assert np.array_equal(host(codes[sl]), o["codes"]), f"step {step} codes at {a}"
            same_f32(host(scales[a // block:(a + (1 << 20)) // block]), o["scales"], f"scales {a}")
            same_f32(host(deq[sl]), o["deq"], f"deq {a}")
            same_f32(host(err[sl]), o["e"], f"residual {a}")
            e_prev[a] = o["e"]
        q = host(codes)
        assert q.min() >= -127 and q.max() <= 127
        del q
    del err, codes, scales, deq, g
    _free()


def test_bert_large_335M_x8_from_gradients():
    """The fused path at full size: two steps of compress_grad + server +
    packed Adam; sampled worker chunks free-running, server in lock-step."""
    dev = device()
    wl = C.get("bert_large_335M_x8")
    N, n, L = wl.N, wl.n, wl.L
    _need(dev, int(n * N * 4 * 2.2 + N * 4 * 6))
    print(f"[fullsize] fused {wl.name}", flush=True)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    grp = OneBitGroup(N, n, dev)
    x = S.params(wl, dev)
    v = S.frozen_variance(wl, dev)
    g = torch.empty((n, N), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(1)
    idx = torch.from_numpy(np.sort(rng.choice(N, size=1 << 20, replace=False))).to(dev)
    pairs, csrv = [(2, 6), (7, 1)], 6
    e_w = {p: np.zeros(L, dtype=F32) for p in pairs}
    E_c = np.zeros(L, dtype=F32)
    mbar_prev = np.zeros(N, dtype=F32)
    for t in (1, 2):
        S.momentum(wl, 100 + t, dev, sigma_elem=sig, out=g)
        first = t == 1
        x_before = host(x[idx])
        grp.compress_grad(g, t, wl.beta1, first=first)
        grp.server(t, first=first, decompress=True)
        grp.adam_step_packed(x, v, wl.lr, wl.eps)
        torch.cuda.synchronize()
        scales = host(grp.scales)
        for (i, c) in pairs:
            sl = slice(c * L, (c + 1) * L)
            m = O.local_momentum(host(g[i, sl])[None, :], mbar_prev[sl], wl.beta1)
            w = O.worker_compress(m, e_w[(i, c)][None, :], reset=first)
            same_f32(np.array([scales[i, c]]), w["s"][0, :1], f"t={t} scale[{i},{c}]")
            same_bits(host(grp.bits[i, _chunk_words(c, L)]), w["bits"][0], f"t={t} bits[{i},{c}]")
            e_w[(i, c)] = w["e"][0]
        sl = slice(csrv * L, (csrv + 1) * L)
        r = O.server_chunk(host(grp.bits[:, _chunk_words(csrv, L)]), scales[:, csrv], E_c, reset=first)
        same_f32(np.array([host(grp.sv_scales)[csrv]]), np.array([r["S"]]), f"t={t} server scale")
        same_bits(host(grp.sv_bits[_chunk_words(csrv, L)]), r["bits"], f"t={t} server bits")
        E_c = r["E"]
        mbar_now = host(grp.mbar)
        x_want = P.adam_frozen_step(x_before, mbar_now[host(idx)], host(v[idx]), wl.lr, wl.eps)
        same_f32(host(x[idx]), x_want, f"t={t} parameters (sampled)")
        mbar_prev = mbar_now.copy()
    del grp, x, v, g, sig
    _free()


def test_warmup_fullsize():
    """The warmup rows the bench times, at full size: Adam on the 335M
    buffer (sampled elements against the oracle), LAMB on the 302-tensor
    buffer (whole sampled layers through the oracle: m, v, x, c, c_avg;
    among them the 31M-element word embedding, small LayerNorm vectors and
    the pad), and k_l for every layer against a binary64 reference."""
    from momentum_compression_amd.state import AdamWarmup, LambWarmup
    from oracle import warmup as W

    dev = device()
    wa = C.get("bert_large_335M_x8")
    N = wa.N
    _need(dev, N * 4 * 8)
    print(f"[fullsize warmup] adam N={N}", flush=True)
    hp = dict(lr=wa.lr, eps=wa.eps, beta1=wa.beta1, beta2=wa.beta2)
    ad = AdamWarmup.create(S.params(wa, dev))
    rng = np.random.default_rng(4)
    idx_d = torch.from_numpy(np.sort(rng.choice(N, size=1 << 20, replace=False))).to(dev)
    for t in range(1, 3):
        g = S.laplace_gradient(N, t, 21, dev)
        xb, mb, vb = host(ad.x[idx_d]), host(ad.m[idx_d]), host(ad.v[idx_d])
        ad.step(g, **hp)
        torch.cuda.synchronize()
        o = W.adam_warmup_step(xb, mb, vb, host(g[idx_d]), **hp)
        for key in ("x", "m", "v"):
            same_f32(host(getattr(ad, key)[idx_d]), o[key], f"adam warmup t={t} {key} (sampled)")
    del ad, g
    _free()

    wl = C.get("bert_large_lamb_302t_x16")
    N = wl.N
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    Sg = len(off) - 1
    print(f"[fullsize warmup] lamb N={N} layers={Sg}", flush=True)
    lw = LambWarmup.create(S.params(wl, dev), torch.from_numpy(off).to(dev))
    layers = [0, 1, 3, 4, 5, 6, 150, Sg - 3, Sg - 2, Sg - 1]
    cav = {l: None for l in layers}
    for t in range(1, 3):
        g = S.laplace_gradient(N, t, 22, dev)
        before = {}
        for l in layers:
            sl = slice(int(off[l]), int(off[l + 1]))
            before[l] = (host(lw.x[sl]), host(lw.m[sl]), host(lw.v[sl]), host(g[sl]))
        lw.step(g, wl.lr, wl.eps, wl.beta1, wl.beta2, 0.9)
        torch.cuda.synchronize()
        c = host(lw.c)
        c_avg = host(lw.c_avg)
        for l in layers:
            sl = slice(int(off[l]), int(off[l + 1]))
            xb, mb, vb, gb = before[l]
            o = W.lamb_warmup_step(xb, mb, vb, gb, [0, xb.size], wl.lr, wl.eps, wl.beta1,
                                   wl.beta2, c_avg=cav[l], beta_c=0.9)
            tag = f"lamb warmup t={t} layer {l} ({xb.size})"
            same_f32(c[l:l + 1], o["c"], f"{tag} c")
            same_f32(c_avg[l:l + 1], o["c_avg"], f"{tag} c_avg")
            same_f32(host(lw.m[sl]), o["m"], f"{tag} m")
            same_f32(host(lw.v[sl]), o["v"], f"{tag} v")
            same_f32(host(lw.x[sl]), o["x"], f"{tag} x")
            cav[l] = o["c_avg"]
    k = host(lw.momentum_scale())
    torch.cuda.synchronize()
    mh = host(lw.m).astype(np.float64)
    rms = np.array([np.sqrt(np.dot(mh[int(off[l]):int(off[l + 1])], mh[int(off[l]):int(off[l + 1])])
                            / max(1, int(off[l + 1] - off[l]))) for l in range(Sg)])
    ok = rms > 0
    want = np.where(ok, rms[ok].mean() / np.where(ok, rms, 1.0), 1.0)
    assert np.all(np.abs(k.astype(np.float64) - want) <= 1e-6 * np.abs(want)), "k_l"
    del lw, g, mh
    _free()


def test_64_workers_largest_worker_count():
    """The largest worker count (64, the general-n server) on a 2^27-element
    buffer: 4096 (worker, chunk) pairs of 2^21 elements, about 69 GB of
    momenta and error states."""
    wl = C.Workload(name="adam_2^27_x64", kind="adam", N=1 << 27, n=64, steps=2,
                    segments=[1 << 20] * 128, seg_names=[f"seg{i}" for i in range(128)],
                    sigma_mode="loguniform_1e-5_1e-2", seed=6)
    _run_adam_fullsize(wl, steps=2, pairs=[(0, 0), (17, 40), (63, 63)], server_chunks=[0, 63],
                       sample=1 << 18)
