"""Benchmark of the error-compensated 1-bit compression stage on one MI355X.

One step = the whole compressed 1-bit Adam hot path over one batch of
synthetic momenta resident in HBM: worker compress of all n workers (reset,
compensate, chunk scale, sign pack, error), server reduce (unpack, average,
compensate, scale, pack, error), decompression of the global momentum, and
the frozen-variance Adam update.  The decompression runs inside the Adam
pass, which reads the packed server words once and writes both the
decompressed momentum and the parameters; the separate decompression and
Adam kernels are timed after the step as a row of their own.  Default
workload: the GPT-style 1.3B-parameter buffer (1,311,528,960 fp32 elements,
291 tensors) with 16 simulated workers, clamp 2.0 and the error reset every
2000 steps (the 1-bit Adam article's GPT-3 1.3B workload); the BERT-Large
335M x 8 buffer, the LAMB, INT8, fused and warmup paths are rows.

Prints ONE JSON line.  `value` = compressed worker elements per second
(n * N per step).  `roofline` reports the dominant kernel (worker compress)
against 8 TB/s of HBM using its algorithmic bytes (12.125 B per element:
read m and the error state, write the state and 1 bit), with the duration
measured by HIP events on the launch stream.  `cpu_baseline` times the C++
CPU oracle on a bounded sample of the same step (chunk 0 of every worker:
1/n of the step's work), on the bench's own inputs.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
    python bench.py --only compress|server|decompress_adam|decompress|adam|copy  # profiling aid
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "compressed elements/s and HBM GB/s (% of peak), 1-bit EF compress+decompress"

# algorithmic bytes per element (single pass, what the method must move)
B_COMPRESS = 12.125            # m 4 + error state 4 in + 4 out + 1/8 bit
B_DECOMPRESS = 4.125           # 1/8 bit in + 4 out
B_ADAM = 16.0                  # x 4 in/out, m 4, v 4
B_DECOMPRESS_ADAM = 16.125     # 1/8 bit, x 4, v 4 in; x 4, decompressed momentum 4 out


def b_server(n: int) -> float:  # n/8 bits in, state 4 in + 4 out, 1/8 bit out
    return 8.125 + n / 8.0


def counter_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"compress_{workload}_counters.txt")


KERNEL_SOURCES = [os.path.join(ROOT, "momentum_compression_amd", "csrc", f)
                  for f in ("compress.hip", "common.h")]


def kernel_source_hash() -> str:
    """Hash of the compress kernel's code: comments and whitespace removed, so
    that only a change of the code makes the stored counters stale."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, launch_elems: int):
    """HBM bytes per compress launch from the committed rocprofv3 counter
    summary of the workload, if it was taken on the current kernel source
    (else None)."""
    path = counter_file(workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        fetch = float(vals["FETCH_SIZE_KiB_per_dispatch"]) * float(vals["fetch_scale_factor"])
        write = float(vals["WRITE_SIZE_KiB_per_dispatch"]) * float(vals["write_scale_factor"])
        elems = int(vals["elements_per_dispatch"])
    except (KeyError, ValueError):
        return None
    if elems != launch_elems:
        return None
    return (fetch + write) * 1024.0


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_STEPS = 2  # compressed steps in the oracle's timed sample


def cpu_baseline(wl, m, x, v):
    """Time the C++ oracle on a bounded sample of the workload: chunk 0 of
    every worker (compress of the n worker-chunk pairs, the server of chunk
    0, its decompression and Adam step), which is 1/n of a step's work, over
    CPU_STEPS consecutive steps, so the rate is CPU_STEPS n L worker elements
    over the sample's time. A reset step on the same momenta runs first,
    untimed, so the timed compression carries the error like the steps on
    the GPU. The sample runs on one thread (the reported value), then once
    more with the worker chunks and the tail's slices over the host's threads
    (the server chunk stays on one thread). m [n, N], x, v [N]: device
    float32; only chunk 0 is copied to the host."""
    import numpy as np

    from oracle import cref as R

    n, N, L = wl.n, wl.N, wl.L
    R.load()
    threads = max(1, min(16, os.cpu_count() or 1))
    mh = m[:, :L].cpu().numpy()
    xh, vh = x[:L].cpu().numpy(), v[:L].cpu().numpy()
    W = L // 32

    def sample(reset, e, E, th):
        """Worker rows of one chunk (n = 1 per call), the server of chunk 0
        over those words, then the tail; returns (seconds, e, E)."""
        t0 = time.perf_counter()
        bits = np.zeros((n, N // 32), dtype=np.uint32)  # chunk 0's words at the row starts
        s = np.zeros((n, n), dtype=np.float32)
        e_new = np.empty((n, L), dtype=np.float32)

        def pair(i):
            w = R.worker_compress_row(mh[i], None if reset else e[i], 1, wl.clip, reset,
                                      e_out=e_new[i])
            bits[i, :W], s[i, 0] = w["bits"], w["s"][0]

        R._run(pair, range(n), th)
        t1 = time.perf_counter()
        # the server of chunk 0 sees exactly these words and scales (the
        # other chunks' words are zero and never read)
        sv = R.server_reduce_chunk(bits, s, E, 0, reset=reset)
        t2 = time.perf_counter()
        mbar = R.decompress(sv["bits"][:W], sv["S"][:1], threads=th)
        R.adam_frozen_step(xh, mbar, vh, wl.lr, wl.eps, threads=th)
        t3 = time.perf_counter()
        return (t3 - t0, (t1 - t0, t2 - t1, t3 - t2)), e_new, sv["E"]

    _, e0, E0 = sample(True, None, None, threads)

    def steps(th):
        e, E, sec, parts = e0, E0, 0.0, [0.0, 0.0, 0.0]
        for _ in range(CPU_STEPS):
            (s1, p1), e, E = sample(False, e, E, th)
            sec, parts = sec + s1, [a + b for a, b in zip(parts, p1)]
        return sec, parts

    sec1, parts1 = steps(1)
    secm, partsm = steps(threads)
    fmt = "compress {:.1f} s, server {:.1f} s, decompression and Adam {:.1f} s"
    return {
        "value": CPU_STEPS * n * L / sec1,
        "unit": "elements/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"chunk 0 ({L} elements) of all {n} workers over {CPU_STEPS} consecutive "
                   f"steps, {CPU_STEPS}/{n} of a step of {wl.name}: compress of the {n} worker "
                   f"chunks, the server of chunk 0, its decompression and Adam step, by the "
                   f"C++ oracle on one thread, on the bench's own inputs copied from the GPU, "
                   f"after an untimed reset step on the same momenta; {sec1:.1f} s "
                   f"({fmt.format(*parts1)}), scaled to the step as {n} L worker elements "
                   f"per step of the sample"),
        "cpu_model": _cpu_model(),
        "threads_available": os.cpu_count(),
        "multithreaded": {"value": CPU_STEPS * n * L / secm, "unit": "elements/s",
                          "cores": threads,
                          "sample": (f"the same sample with the {n} worker chunks and the "
                                     f"tail's slices over {threads} threads (the server "
                                     f"chunk on one): {secm:.1f} s ({fmt.format(*partsm)})")},
    }


B_COMPRESS_GRAD = 12.25        # g 4 + state 4 in + 4 out + 1/8 bit + 1/8 packed previous momentum
B_ADAM_PACKED = 12.125         # x 4 in/out, v 4, 1/8 packed momentum
B_LAMB_STEP = 28.0             # read x, m, m_prev, v_fresh, v_Tw; write x, v_fresh
B_LAMB_PACKED = 28.125         # read 1/8 bit, x, m_prev, v_fresh, v_Tw; write x, v_fresh, m
B_LAMB_PACKED_PREV = 20.25     # read 1/8 bit twice (m_t, m_{t-1}), x, v_fresh, v_Tw; write x, v_fresh
B_INT8 = 17.015625             # read g, err; write code, err, deq; scale per 256
B_WARMUP_ADAM = 28.0           # read x, m, v, g; write x, m, v
B_WARMUP_LAMB = 40.0           # pass 1: read x, m, v, g, write m, v; pass 2: read x, m, v, write x
B_MOMENTUM_SCALE = 4.0         # read m


def _time_calls(fns, warmup: int, steps: int, stream):
    """Run the callables in order `warmup` + `steps` times; return the mean
    event time (ms) of each callable over the timed repetitions."""
    import torch

    for _ in range(warmup):
        for f in fns:
            f()
    acc = [0.0] * len(fns)
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        ev[0].record(stream)
        for k, f in enumerate(fns):
            f()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        for k in range(len(fns)):
            acc[k] += ev[k].elapsed_time(ev[k + 1])
    return [a / steps for a in acc]


def _rel(a, b) -> float:
    """||a|| / ||b|| (binary64 norms): a report-only diagnostic of the
    compression error against what was compressed."""
    import torch

    na = torch.linalg.vector_norm(a.double()).item()
    nb = torch.linalg.vector_norm(b.double()).item()
    return na / nb if nb > 0 else float("nan")


def _inputs(wl) -> str:
    if wl.sigma_mode == "const1e-3":
        return "momentum N(0, 1e-3), fresh per worker"
    per = "per 2^20-element block" if wl.name == "bert_large_335M_x8" else "per tensor"
    lo, hi = {"loguniform_1e-5_1e-2": ("1e-5", "1e-2"),
              "loguniform_1e-6_1e-1": ("1e-6", "1e-1")}[wl.sigma_mode]
    return f"momentum N(0, sigma), sigma log-uniform [{lo}, {hi}] {per}"


def _row(ms: float, nbytes: float, elems: int) -> dict:
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "elements_per_s": elems / (ms * 1e-3),
            "algorithmic_GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4)}


def measure_lamb(steps: int, warmup: int) -> dict:
    """1-bit LAMB path on the 302-tensor BERT-Large buffer, 16 workers:
    compress with x k_l fused, server reduce, the decompression with / k_l,
    and the LAMB frozen-variance step with the per-layer ratio and r/c
    update -- as two kernels, as one pass that reads the server's sign
    words and writes the decompressed momentum, and as one pass that reads
    the previous step's sign words for m_{t-1} and writes no momentum (the
    steady state from the second compressed step on, which the step's total
    uses)."""
    import numpy as np
    import torch

    from momentum_compression_amd import onebit as ob
    from momentum_compression_amd.state import LambState, OneBitGroup, momentum_scale
    from workloads import configs as C
    from workloads import synth as S

    dev = torch.device("cuda:0")
    wl = C.get("bert_large_lamb_302t_x16")
    N, n = wl.N, wl.n
    print(f"[bench] rows: {wl.name} N={N} n={n}", file=sys.stderr, flush=True)
    off = np.array(C.segment_offsets(wl.segments), dtype=np.int64)
    c_avg = S.lamb_c_avg(wl)
    off_d = torch.from_numpy(off).to(dev)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    # the fixed layer coefficients k_l from the momentum at the end of warmup
    k_d = momentum_scale(S.lamb_prev_momentum(wl, dev, sig), off_d)
    n_seg = k_d.numel()
    m = S.momentum(wl, 1, dev, sigma_elem=sig)
    grp = OneBitGroup(N, n, dev, seg_off=off_d, seg_k=k_d, keep_prev=True)
    st = LambState.create(S.params(wl, dev), S.frozen_variance(wl, dev),
                          S.lamb_prev_momentum(wl, dev, sig), off_d, torch.from_numpy(c_avg).to(dev))
    st2 = LambState.create(S.params(wl, dev), st.v_frozen, S.lamb_prev_momentum(wl, dev, sig),
                           off_d, torch.from_numpy(c_avg).to(dev))
    st3 = LambState.create(S.params(wl, dev), st.v_frozen, S.lamb_prev_momentum(wl, dev, sig),
                           off_d, torch.from_numpy(c_avg).to(dev))
    del sig
    stream = torch.cuda.current_stream()
    grp.compress(m, 1, first=True)
    grp.server(1, first=True)
    t = [2]

    def comp():
        grp.compress(m, t[0])

    def serv():
        grp.server(t[0], decompress=False)

    def dec():
        ob.onebit_decompress(grp.sv_bits, grp.sv_scales, grp.mbar, N, n, seg_off=off_d,
                             seg_k=k_d, n_seg=n_seg)

    def lamb():
        st.step(grp.mbar, wl.lr, wl.eps, wl.beta1, wl.beta2, wl.r_threshold, wl.r_min, wl.r_max)
        t[0] += 1

    def lamb_packed():
        st2.step_packed(grp.sv_bits, grp.sv_scales, k_d, n, wl.lr, wl.eps, wl.beta1, wl.beta2,
                        wl.r_threshold, wl.r_min, wl.r_max)

    def lamb_packed_prev():
        st3.step_packed(grp.sv_bits, grp.sv_scales, k_d, n, wl.lr, wl.eps, wl.beta1, wl.beta2,
                        wl.r_threshold, wl.r_min, wl.r_max, prev_bits=grp.sv_bits_prev,
                        prev_scales=grp.sv_scales_prev)

    # step-ratio-scaled error feedback: the carried errors times c_{t-1}/c_t
    # per layer, at both levels (the same bytes as the plain kernels)
    def comp_ers():
        grp.seg_err_ratio = st.err_ratio
        grp.compress(m, t[0])
        grp.seg_err_ratio = None

    def serv_ers():
        grp.seg_err_ratio = st.err_ratio
        grp.server(t[0], decompress=False)
        grp.seg_err_ratio = None

    ms = _time_calls([comp, serv, dec, lamb, comp_ers, serv_ers, lamb_packed, lamb_packed_prev],
                     warmup, steps, stream)
    step_ms = ms[0] + ms[1] + ms[7]
    out = {"workload": wl.name, "N": N, "workers": n, "layers": len(wl.segments),
           "step_ms": round(step_ms, 4), "worker_elements_per_s": n * N / (step_ms * 1e-3),
           "compress_x_k": _row(ms[0], B_COMPRESS * n * N, n * N),
           "server": _row(ms[1], b_server(n) * N, N),
           "decompress_div_k_lamb_step": _row(ms[6], B_LAMB_PACKED * N, N),
           "lamb_step_both_momenta_packed": _row(ms[7], B_LAMB_PACKED_PREV * N, N),
           "decompress_div_k": _row(ms[2], B_DECOMPRESS * N, N),
           "lamb_step": _row(ms[3], B_LAMB_STEP * N, N),
           "compress_x_k_step_ratio_ef": _row(ms[4], B_COMPRESS * n * N, n * N),
           "server_step_ratio_ef": _row(ms[5], b_server(n) * N, N)}
    r = st2.r.double()
    out["r_t"] = {"min": r.min().item(), "median": r.median().item(), "max": r.max().item()}
    kk = k_d.double()
    out["k_l"] = {"from": "momentum scale of the warmup momentum", "min": kk.min().item(),
                  "median": kk.median().item(), "max": kk.max().item()}
    del grp, st, st2, st3, m
    torch.cuda.empty_cache()
    return out


def measure_fused(steps: int, warmup: int) -> dict:
    """The 1-bit Adam step fed with gradients on the 335M x 8 workload, with
    the local momentum update fused into compression and the decompression
    fused into the Adam step: compress_grad, server (no decompressed
    buffer), Adam from the packed global momentum."""
    import torch

    from momentum_compression_amd.state import OneBitGroup
    from workloads import configs as C
    from workloads import synth as S

    dev = torch.device("cuda:0")
    wl = C.get("bert_large_335M_x8")
    N, n = wl.N, wl.n
    print(f"[bench] rows: fused {wl.name} N={N} n={n}", file=sys.stderr, flush=True)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    g = S.momentum(wl, 7, dev, sigma_elem=sig)  # gradient stand-in drawn with the same recipe
    del sig
    x = S.params(wl, dev)
    v = S.frozen_variance(wl, dev)
    grp = OneBitGroup(N, n, dev)
    stream = torch.cuda.current_stream()
    grp.compress_grad(g, 1, wl.beta1, first=True)
    grp.server(1, first=True, decompress=False)
    t = [2]

    def comp():
        grp.compress_grad(g, t[0], wl.beta1)

    def serv():
        grp.server(t[0], decompress=False)

    def adam():
        grp.adam_step_packed(x, v, wl.lr, wl.eps)
        t[0] += 1

    # the unscaled +-1 variant of the worker compression
    def comp_unit():
        grp.unit_scale = True
        grp.compress_grad(g, t[0], wl.beta1)
        grp.unit_scale = False

    ms = _time_calls([comp, serv, adam, comp_unit], warmup, steps, stream)
    step_ms = sum(ms[:3])
    out = {"workload": wl.name, "N": N, "workers": n, "step_ms": round(step_ms, 4),
           "worker_elements_per_s": n * N / (step_ms * 1e-3),
           "compress_grad": _row(ms[0], B_COMPRESS_GRAD * n * N, n * N),
           "server": _row(ms[1], b_server(n) * N, N),
           "adam_packed": _row(ms[2], B_ADAM_PACKED * N, N),
           "compress_grad_unit_scale": _row(ms[3], B_COMPRESS_GRAD * n * N, n * N)}
    del grp, g, x, v
    torch.cuda.empty_cache()
    return out


def measure_warmup(steps: int, warmup: int) -> dict:
    """Uncompressed warmup steps before the compressed phase: Adam on the
    335M buffer, LAMB (per-layer trust ratio and coefficient average) on the
    302-tensor BERT-Large buffer, and the per-layer momentum scale taken at
    the end of warmup."""
    import numpy as np
    import torch

    from momentum_compression_amd import onebit as ob
    from momentum_compression_amd.state import AdamWarmup, LambWarmup
    from workloads import configs as C
    from workloads import synth as S

    dev = torch.device("cuda:0")
    wa = C.get("bert_large_335M_x8")
    wlb = C.get("bert_large_lamb_302t_x16")
    print(f"[bench] rows: warmup {wa.name} N={wa.N}, {wlb.name} N={wlb.N}", file=sys.stderr,
          flush=True)
    stream = torch.cuda.current_stream()
    ad = AdamWarmup.create(S.params(wa, dev))
    g = S.laplace_gradient(wa.N, 1, 21, dev)

    def adam():
        ad.step(g, wa.lr, wa.eps, wa.beta1, wa.beta2)

    ms_a = _time_calls([adam], warmup, steps, stream)[0]
    del ad, g
    torch.cuda.empty_cache()
    off = torch.from_numpy(np.array(C.segment_offsets(wlb.segments), dtype=np.int64)).to(dev)
    lw = LambWarmup.create(S.params(wlb, dev), off)
    g = S.laplace_gradient(wlb.N, 1, 22, dev)
    k = torch.empty(off.numel() - 1, device=dev)

    def lamb():
        lw.step(g, wlb.lr, wlb.eps, wlb.beta1, wlb.beta2, 0.9)

    def scale():
        ob.lamb_momentum_scale(lw.m, wlb.N, off, off.numel() - 1, k, lw.ws)

    ms = _time_calls([lamb, scale], warmup, steps, stream)
    out = {"adam_workload": wa.name, "lamb_workload": wlb.name, "layers": len(wlb.segments),
           "adam_warmup_step": _row(ms_a, B_WARMUP_ADAM * wa.N, wa.N),
           "lamb_warmup_step": _row(ms[0], B_WARMUP_LAMB * wlb.N, wlb.N),
           "momentum_scale": _row(ms[1], B_MOMENTUM_SCALE * wlb.N, wlb.N)}
    del lw, g
    torch.cuda.empty_cache()
    return out


def measure_adam_row(name: str, steps: int, warmup: int) -> dict:
    """Another 1-bit Adam workload as a row (the BERT-Large 335M x 8 buffer,
    or the 1.3B GPT-style buffer x 16 with its clamp and reset): compress,
    server, and the decompression with the frozen-v Adam step in one pass;
    the decompression and Adam kernels are also timed on their own."""
    import torch

    from momentum_compression_amd import onebit as ob
    from momentum_compression_amd.state import OneBitGroup
    from workloads import configs as C
    from workloads import synth as S

    dev = torch.device("cuda:0")
    wl = C.get(name)
    N, n = wl.N, wl.n
    print(f"[bench] rows: {wl.name} N={N} n={n}", file=sys.stderr, flush=True)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    m = S.momentum(wl, 1, dev, sigma_elem=sig)
    del sig
    x = S.params(wl, dev)
    v = S.frozen_variance(wl, dev)
    grp = OneBitGroup(N, n, dev, clip=wl.clip, reset_interval=wl.reset_interval)
    stream = torch.cuda.current_stream()
    grp.compress(m, 1, first=True)
    grp.server(1, first=True, decompress=False)
    t = [2]

    def comp():
        grp.compress(m, t[0])

    def serv():
        grp.server(t[0], decompress=False)

    def dec():
        ob.onebit_decompress(grp.sv_bits, grp.sv_scales, grp.mbar, N, n)

    def adam():
        grp.adam_step(x, v, wl.lr, wl.eps)

    def dec_adam():
        grp.adam_step_packed(x, v, wl.lr, wl.eps, decompress=True)
        t[0] += 1

    ms = _time_calls([comp, serv, dec, adam, dec_adam], warmup, steps, stream)
    step_ms = ms[0] + ms[1] + ms[4]  # the step with the decompression inside the Adam pass
    out = {"workload": wl.name, "N": N, "workers": n, "step_ms": round(step_ms, 4),
           "worker_elements_per_s": n * N / (step_ms * 1e-3),
           "compress_clamp" if wl.clip > 0 else "compress": _row(ms[0], B_COMPRESS * n * N,
                                                                  n * N),
           "server": _row(ms[1], b_server(n) * N, N),
           "decompress_adam": _row(ms[4], B_DECOMPRESS_ADAM * N, N),
           "decompress": _row(ms[2], B_DECOMPRESS * N, N),
           "adam": _row(ms[3], B_ADAM * N, N)}
    del grp, m, x, v
    torch.cuda.empty_cache()
    return out


# plain stream probes (libonebit_probe.so): mode, name, bytes per float
BASIC_PROBES = ((0, "read", 4.0), (1, "write", 4.0), (2, "copy", 8.0),
                (3, "read_two_write_one_in_place", 12.0))
# the parameter passes' mixes: (reads, writes), name, bytes per float, and
# the element count of the row whose pass has that mix (the LAMB pass on the
# 302-tensor buffer, the Adam warm-up step on the 335M buffer)
MIX_PROBES = (((3, 2), "read_three_write_two_in_place", 20.0, 336226304),
              ((4, 3), "read_four_write_three_in_place", 28.0, 335141888))


def measure_copy(steps: int, warmup: int) -> dict:
    """Plain streams over 2^31 floats as context for the rows: torch's device
    copy, and the probe library's hand-written read, write, copy and
    read-two-write-one-in-place streams (one float4 per lane, 256-thread
    workgroups, nontemporal, the library kernels' access shape), and the
    read/write mixes of the LAMB pass (three reads, two writes) and the Adam
    warm-up step (four reads, three writes): the practical HBM ceilings of
    those mixes on this GPU."""
    import ctypes

    import torch

    dev = torch.device("cuda:0")
    src = torch.empty(1 << 31, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    dst.fill_(0.5)
    stream = torch.cuda.current_stream()
    N = src.numel()

    def rate(ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "GBps": round(gbs, 1),
                "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4)}

    ms = _time_calls([lambda: dst.copy_(src)], warmup, steps, stream)[0]
    out = {"floats": N, **rate(ms, 8.0 * N)}
    lib = _probe_lib()
    if lib is not None:
        lib.onebit_probe_basic.restype = ctypes.c_int32
        lib.onebit_probe_basic.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_void_p]

        def probe(mode):
            rc = lib.onebit_probe_basic(src.data_ptr(), dst.data_ptr(), N, mode,
                                        ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"stream probe mode {mode}: status {rc}")

        lib.onebit_probe_mix.restype = ctypes.c_int32
        lib.onebit_probe_mix.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int32,
                                                                 ctypes.c_int32, ctypes.c_void_p]
        c3 = torch.empty_like(src)
        c3.fill_(0.25)
        c4 = torch.empty_like(src)
        c4.fill_(0.125)

        def mix(reads, writes, n_el):
            rc = lib.onebit_probe_mix(src.data_ptr(), dst.data_ptr(), c3.data_ptr(), c4.data_ptr(),
                                      n_el, reads, writes, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"mix probe {reads}r{writes}w: status {rc}")

        fns = [lambda mode=mode: probe(mode) for mode, _, _ in BASIC_PROBES]
        fns += [lambda rw=rw: mix(*rw, N) for rw, _, _, _ in MIX_PROBES]
        fns += [lambda rw=rw, n_row=n_row: mix(*rw, n_row) for rw, _, _, n_row in MIX_PROBES]
        try:  # context only: a probe failure never fails the bench line
            ms_p = _time_calls(fns, warmup, steps, stream)
            nb = len(BASIC_PROBES)
            sp = {name: rate(t, per * N) for (_, name, per), t in zip(BASIC_PROBES, ms_p)}
            sp.update({name: rate(t, per * N)
                       for (_, name, per, _), t in zip(MIX_PROBES, ms_p[nb:])})
            out["stream_probes"] = sp
            out["mix_probes_at_row_size"] = {
                name: {"floats": n_row, **rate(t, per * n_row)}
                for (_, name, per, n_row), t in zip(MIX_PROBES, ms_p[nb + len(MIX_PROBES):])}
        except RuntimeError as exc:
            out["stream_probes"] = {"error": str(exc)}
        del c3, c4
    del src, dst
    torch.cuda.empty_cache()
    return out


def measure_int8(steps: int, warmup: int) -> dict:
    """Block INT8 stochastic rounding with error feedback and dequantised
    output on 2^30 Laplace gradients (block 256)."""
    import torch

    from momentum_compression_amd import onebit as ob
    from workloads import synth as S

    dev = torch.device("cuda:0")
    N, block = 1 << 30, 256
    print(f"[bench] rows: int8 N={N}", file=sys.stderr, flush=True)
    g = S.laplace_gradient(N, 1, 4, dev)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    stream = torch.cuda.current_stream()
    step = [1]

    def q():
        ob.int8_sr_quantize(g, err, codes, scales, deq, N, block, 4, step[0])
        step[0] += 1

    ws = torch.empty(256, dtype=torch.uint8, device=dev)

    def rtn():
        ob.int8_quantize(g, err, codes, scales, deq, N, block, 1, 4, 1, ws=ws)

    def tensor_scale():
        ob.int8_quantize(g, err, codes, scales, deq, N, 0, 0, 4, 1, ws=ws)

    ms = _time_calls([q, rtn, tensor_scale], warmup, steps, stream)
    # report-only: ||deq - g|| / ||g|| of one call from zero error
    err.zero_()
    q()
    rel = _rel(deq - g, g)
    out = {"workload": "int8_sr_2^30", "N": N, "block": block, "dequantised_error_rel": rel,
           "int8_sr_ef_deq": _row(ms[0], B_INT8 * N, N),
           "int8_nearest_ef_deq": _row(ms[1], B_INT8 * N, N),
           # one extra read pass of g and the error for the tensor maximum
           "int8_sr_tensor_scale_ef_deq": _row(ms[2], (B_INT8 + 8.0) * N, N)}
    del g, err, codes, scales, deq
    torch.cuda.empty_cache()
    return out


def measure_sweep(wl, steps: int, warmup: int) -> list:
    """The step (compress, server, decompression inside the Adam pass) of the
    workload's worker count over buffer sizes from 2^20 elements to N: where
    launches and the finalize stop mattering next to the streams."""
    import torch

    from momentum_compression_amd.state import OneBitGroup

    dev = torch.device("cuda:0")
    n = wl.n
    sizes = [1 << k for k in range(20, 30, 2) if (1 << k) < wl.N] + [wl.N]
    out = []
    for N in sizes:
        N -= N % (64 * n)
        print(f"[bench] sweep N={N} n={n}", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev)
        g.manual_seed(N)
        m = torch.randn((n, N), generator=g, device=dev) * 1e-3
        x = torch.randn(N, generator=g, device=dev) * 0.02
        v = torch.rand(N, generator=g, device=dev) * 1e-6 + 1e-8
        grp = OneBitGroup(N, n, dev)
        stream = torch.cuda.current_stream()

        def step(t):
            grp.compress(m, t, first=t == 1)
            grp.server(t, first=t == 1, decompress=False)
            grp.adam_step_packed(x, v, wl.lr, wl.eps, decompress=True)

        for t in range(1, warmup + 1):
            step(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(warmup + 1, warmup + steps + 1):
            step(t)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        # the same non-reset step as one HIP graph per replay
        graph = grp.capture_step(m, x, v, wl.lr, wl.eps)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_g = e0.elapsed_time(e1) / steps
        nbytes = B_COMPRESS * n * N + b_server(n) * N + B_DECOMPRESS_ADAM * N
        out.append({"N": N, "workers": n, "ms_per_step": round(ms, 4),
                    "elements_per_s": n * N / (ms * 1e-3),
                    "algorithmic_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "graph_ms_per_step": round(ms_g, 4)})
        del m, x, v, grp, graph
        torch.cuda.empty_cache()
    return out


PROBE_MODES = [(0, "stream: read m and state, write state"),
               (1, "stream + sign words"),
               (2, "stream + binary64 block sum"),
               (3, "stream + sign words + block sum (the compression's memory operations)")]


def _probe_lib():
    """The probe library (built by build() next to libonebit.so), or None.
    torch is imported first, so that the library binds to torch's HIP
    runtime (see ``onebit.load``)."""
    import ctypes

    import torch  # noqa: F401

    from momentum_compression_amd.build import PROBE_LIB

    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.onebit_probe_stream.restype = I32
    lib.onebit_probe_stream.argtypes = [P, P, P, P, I64, I32, I32, P]
    lib.onebit_probe_server.restype = I32
    lib.onebit_probe_server.argtypes = [P, P, P, P, I64, I32, I64, P]
    lib.onebit_probe_int8.restype = I32
    lib.onebit_probe_int8.argtypes = [P, P, P, P, P, I64, P]
    return lib


def measure_probe(wl, steps: int, warmup: int, bufs=None, modes=None) -> dict:
    """The ceiling of the worker compression's memory pattern: probe kernels
    (libonebit_probe.so) with the compression's geometry and launch shape that
    only move its bytes, each extra output switched on in turn, timed with
    HIP events interleaved with the real compression (clamp on, non-reset) on
    the same two [n][N] buffers, so that placement is shared.  bufs: the
    momentum, state, sign words and workspace to use (overwritten), else
    allocated here; modes: the probe modes to time (all by default)."""
    import ctypes

    import torch

    from momentum_compression_amd import onebit as ob

    lib = _probe_lib()
    if lib is None:
        raise RuntimeError("libonebit_probe.so is not built (python __graft_entry__.py build)")
    P = ctypes.c_void_p
    dev = torch.device("cuda:0")
    N, n = wl.N, wl.n
    if bufs is None:
        g = torch.Generator(device=dev)
        g.manual_seed(N)
        a = torch.empty((n, N), device=dev).normal_(0.0, 1e-3, generator=g)  # the momentum
        b = torch.zeros((n, N), device=dev)                        # the state
        bits = torch.zeros((n, N // 32), dtype=torch.int32, device=dev)
        ws = torch.empty(ob.workspace_bytes(N, n, 0), dtype=torch.uint8, device=dev)
    else:
        a, b, bits, ws = bufs
    scales = torch.zeros((n, n), device=dev)
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)
    modes = [m for m in PROBE_MODES if modes is None or m[0] in modes]

    def probe(mode):
        rc = lib.onebit_probe_stream(a.data_ptr(), b.data_ptr(), bits.data_ptr(), ws.data_ptr(),
                                     N, n, mode, sp)
        if rc != 0:
            raise RuntimeError(f"probe mode {mode}: status {rc}")

    def compress():
        ob.onebit_compress(a, b, scales, bits, N, n, clip=wl.clip, reset=False, ws=ws)

    ob.onebit_compress(a, b, scales, bits, N, n, clip=wl.clip, reset=True, ws=ws)
    fns = [lambda mode=mode: probe(mode) for mode, _ in modes] + [compress]
    ms = _time_calls(fns, warmup, steps, stream)
    # sign words in modes 1 and 3 (and the compression): 1/8 byte per element
    nbytes = [B_COMPRESS * n * N - (0 if mode & 1 else n * N / 8) for mode, _ in modes]
    nbytes.append(B_COMPRESS * n * N)
    names = [name for _, name in modes] + ["the worker compression (clamp on, with finalize)"]
    rows = [{"kernel": nm, "ms": round(t, 4), "GBps": round(nb / (t * 1e-3) / 1e9, 1),
             "frac_of_8TBps": round(nb / (t * 1e-3) / 8e12, 4)}
            for nm, t, nb in zip(names, ms, nbytes)]
    del a, b, bits, scales, ws
    if bufs is None:
        torch.cuda.empty_cache()
    return {"workload": wl.name, "N": N, "workers": n, "elements_per_launch": n * N,
            "steps": steps, "warmup": warmup, "rows": rows}


def measure_probe_server(wl, steps: int, warmup: int, grp=None, m=None) -> dict:
    """The ceiling of the server's memory pattern: a probe kernel
    (libonebit_probe.so) with the server's grid and launch shape that does
    its global memory operations (every worker's sign words staged through
    LDS, the state in and out, the server's sign words, the block sum)
    without decoding and adding the workers, timed like the server in the
    step: each right after a worker compression of the same buffers.  grp,
    m: the group and momentum to use (their state is overwritten), else
    allocated here."""
    import ctypes

    import torch

    from momentum_compression_amd.state import OneBitGroup

    lib = _probe_lib()
    if lib is None:
        raise RuntimeError("libonebit_probe.so is not built (python __graft_entry__.py build)")
    P = ctypes.c_void_p
    dev = torch.device("cuda:0")
    N, n = wl.N, wl.n
    own = grp is None
    if own:
        g = torch.Generator(device=dev)
        g.manual_seed(N + 1)
        m = torch.empty((n, N), device=dev).normal_(0.0, 1e-3, generator=g)
        grp = OneBitGroup(N, n, dev)
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)

    def probe():
        rc = lib.onebit_probe_server(grp.bits.data_ptr(), grp.sv_ef.data_ptr(),
                                     grp.sv_bits.data_ptr(), grp.ws.data_ptr(), N, n, 0, sp)
        if rc != 0:
            raise RuntimeError(f"server probe: status {rc}")

    grp.compress(m, 1, first=True)
    grp.server(1, first=True, decompress=False)
    ms = _time_calls([lambda: grp.compress(m, 2), probe, lambda: grp.compress(m, 2),
                      lambda: grp.server(2, decompress=False)], warmup, steps, stream)
    nb = b_server(n) * N
    rows = [{"kernel": nm, "ms": round(t, 4), "GBps": round(nb / (t * 1e-3) / 1e9, 1),
             "frac_of_8TBps": round(nb / (t * 1e-3) / 8e12, 4)}
            for nm, t in (("probe: the server's memory operations, after a compression", ms[1]),
                          ("the server (with finalize), after a compression", ms[3]))]
    del m, grp
    if own:
        torch.cuda.empty_cache()
    return {"workload": wl.name, "N": N, "workers": n, "bytes_per_element": b_server(n),
            "steps": steps, "warmup": warmup, "rows": rows}


def measure_probe_int8(steps: int, warmup: int) -> dict:
    """The ceiling of the INT8 quantiser's memory pattern on 2^30 elements: a
    probe kernel with its grid and launch shape that reads g and the error
    and writes the codes, the error, the dequantised values and the block
    scales without quantising, timed interleaved with the quantiser (block
    256, stochastic rounding, error feedback, dequantised output) on the
    same buffers."""
    import ctypes

    import torch

    from momentum_compression_amd import onebit as ob
    from workloads import synth as S

    lib = _probe_lib()
    if lib is None:
        raise RuntimeError("libonebit_probe.so is not built (python __graft_entry__.py build)")
    P = ctypes.c_void_p
    dev = torch.device("cuda:0")
    N, block = 1 << 30, 256
    g = S.laplace_gradient(N, 1, 4, dev)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)

    def probe():
        rc = lib.onebit_probe_int8(g.data_ptr(), err.data_ptr(), codes.data_ptr(),
                                   scales.data_ptr(), deq.data_ptr(), N, sp)
        if rc != 0:
            raise RuntimeError(f"int8 probe: status {rc}")

    def quantise():  # the error carries whatever the probe left: finite values
        ob.int8_sr_quantize(g, err, codes, scales, deq, N, block, 4, 1)

    ms = _time_calls([probe, quantise], warmup, steps, stream)
    rows = [{"kernel": "probe: the quantiser's memory operations", **_row(ms[0], B_INT8 * N, N)},
            {"kernel": "the quantiser (block 256, stochastic rounding, error feedback, "
                       "dequantised output)", **_row(ms[1], B_INT8 * N, N)}]
    del g, err, codes, scales, deq
    torch.cuda.empty_cache()
    return {"N": N, "block": block, "bytes_per_element": B_INT8, "steps": steps,
            "warmup": warmup, "rows": rows}


def step_log_lines(step_ms: dict, t_first: int, elems: int, bytes_: dict) -> list:
    """One record per timed step from the per-call event times already taken
    (``step_ms[k][i]``: call k of the i-th timed step, in ms): each call's time
    and algorithmic rate, the step's sum of calls and its worker elements/s.
    Pure host arithmetic; nothing here touches the GPU."""
    keys = list(step_ms)
    count = min(len(v) for v in step_ms.values()) if keys else 0
    lines = []
    for i in range(count):
        rec = {"step": t_first + i}
        total = 0.0
        for k in keys:
            ms = step_ms[k][i]
            total += ms
            gbs = bytes_[k] / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
            rec[k] = {"ms": round(ms, 4), "algorithmic_GBps": round(gbs, 1),
                      "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4)}
        rec["calls_ms"] = round(total, 4)
        rec["worker_elements_per_s"] = elems / (total * 1e-3) if total > 0 else 0.0
        lines.append(rec)
    return lines


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt_1.3B_x16")
    ap.add_argument("--only", default="", choices=["", "compress", "server", "decompress_adam",
                                                   "decompress", "adam", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--log", default="",
                    help="also write one JSON line per timed step (each call's time and rate, "
                         "from the same events) and a closing line with the diagnostics")
    ap.add_argument("--sweep", action="store_true",
                    help="time the step over buffer sizes from 2^20 to the workload's N "
                         "(profiling aid; prints its own JSON line)")
    ap.add_argument("--probe", nargs="?", const="compress", default="",
                    choices=["", "compress", "server", "int8"],
                    help="time memory-pattern probes of the worker compression (or of the "
                         "server) beside it (profiling aid; prints its own JSON line)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the rows measured after the headline step (LAMB, INT8, fused, "
                         "warmup, the other Adam workload, copy reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the n workers are simulated as a batch on one device)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print(f"bench.py needs --steps >= 1 and --warmup >= 0 (got {args.steps}, {args.warmup})",
              file=sys.stderr)
        return 2

    import torch

    from momentum_compression_amd import onebit as ob
    from momentum_compression_amd.state import OneBitGroup
    from workloads import configs as C
    from workloads import synth as S

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    ob.load()
    wl = C.get(args.workload)
    if args.probe == "server":  # any 1-bit workload: the server's shape is (N, n)
        print(json.dumps({"probe": measure_probe_server(wl, args.steps, args.warmup)}))
        return 0
    if args.probe == "int8":
        print(json.dumps({"probe": measure_probe_int8(args.steps, args.warmup)}))
        return 0
    if wl.kind != "adam":
        print(f"workload {wl.name} is a parity case; the bench times the 1-bit Adam path",
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    N, n = wl.N, wl.n
    if args.sweep:
        print(json.dumps({"sweep": measure_sweep(wl, args.steps, args.warmup)}))
        return 0
    if args.probe:
        print(json.dumps({"probe": measure_probe(wl, args.steps, args.warmup)}))
        return 0
    print(f"[bench] workload={wl.name} N={N} n={n} steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)
    sig = S.per_element(S.segment_sigmas(wl), wl, dev)
    m = S.momentum(wl, 1, dev, sigma_elem=sig)
    del sig
    x = S.params(wl, dev)
    v = S.frozen_variance(wl, dev)
    grp = OneBitGroup(N, n, dev, clip=wl.clip, reset_interval=wl.reset_interval)
    stream = torch.cuda.current_stream()

    if args.only == "copy":
        # plain copy of n*N floats: the reference for counter scaling
        src = m.view(-1)
        dst = grp.ef.view(-1)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_per_launch": 2 * 4 * src.numel()}))
        return 0

    ev = {k: [] for k in ("compress", "server", "decompress_adam")}
    # with --only decompress or adam, that standalone kernel takes the third slot
    tail_only = args.only in ("decompress", "adam")

    def step(t: int, timed: bool) -> None:
        first = t == 1
        marks = []

        def mark():
            if timed:
                marks.append(torch.cuda.Event(enable_timing=True))
                marks[-1].record(stream)

        mark()
        if args.only in ("", "compress"):
            grp.compress(m, t, first=first)
        mark()
        if args.only in ("", "server"):
            grp.server(t, first=first, decompress=False)
        mark()
        if args.only in ("", "decompress_adam"):
            grp.adam_step_packed(x, v, wl.lr, wl.eps, decompress=True)
        elif args.only == "decompress":
            ob.onebit_decompress(grp.sv_bits, grp.sv_scales, grp.mbar, N, n)
        elif args.only == "adam":
            grp.adam_step(x, v, wl.lr, wl.eps)
        mark()
        if timed:
            for k, (a, b) in zip(ev, zip(marks[:-1], marks[1:])):
                ev[k].append((a, b))

    t = 1
    for _ in range(args.warmup):
        step(t, False)
        t += 1
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(t, True)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = {k: sum(a.elapsed_time(b) for a, b in v_) / max(1, len(v_)) for k, v_ in ev.items()}
    ms_per_step = wall * 1e3 / args.steps
    bytes_ = {"compress": B_COMPRESS * n * N, "server": b_server(n) * N,
              "decompress_adam": B_DECOMPRESS_ADAM * N, "decompress": B_DECOMPRESS * N,
              "adam": B_ADAM * N}
    if tail_only:
        ms[args.only] = ms.pop("decompress_adam")
    kernels = {}
    for k in ms:
        if args.only and args.only != k:
            continue
        gbs = bytes_[k] / (ms[k] * 1e-3) / 1e9 if ms[k] > 0 else 0.0
        kernels[k] = {"ms": round(ms[k], 4), "algorithmic_GBps": round(gbs, 1),
                      "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4)}
    if args.only:
        print(json.dumps({"only": args.only, "kernels": kernels}))
        return 0

    # the same tail as two kernels: decompression, then Adam reading it
    def dec():
        ob.onebit_decompress(grp.sv_bits, grp.sv_scales, grp.mbar, N, n)

    def adam():
        grp.adam_step(x, v, wl.lr, wl.eps)

    ms_u = _time_calls([dec, adam], 1, max(3, args.steps // 2), stream)
    separate = {"decompress": _row(ms_u[0], B_DECOMPRESS * N, N),
                "adam": _row(ms_u[1], B_ADAM * N, N),
                "sum_ms": round(ms_u[0] + ms_u[1], 4)}
    # compression error relative to the compensated values after the last
    # step (worker 0 and the server), outside every timed region
    diagnostics = {"worker0_error_rel": _rel(grp.worker_error()[0], grp.ef[0]),
                   "server_error_rel": _rel(grp.server_error(), grp.sv_ef)}
    if args.log:
        per_step = {k: [a.elapsed_time(b) for a, b in v_] for k, v_ in ev.items()}
        with open(args.log, "w") as f:
            for rec in step_log_lines(per_step, args.warmup + 1, n * N, bytes_):
                f.write(json.dumps({"workload": wl.name, **rec}) + "\n")
            f.write(json.dumps({"workload": wl.name, "after_step": args.warmup + args.steps,
                                "diagnostics": diagnostics}) + "\n")

    comp_gbs = bytes_["compress"] / (ms["compress"] * 1e-3) / 1e9
    traffic = read_traffic(wl.name, n * N)
    out = {
        "metric": METRIC,
        "value": n * N / (ms_per_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "workers": n, "chunk": wl.L,
                   "clip": wl.clip, "reset_interval": wl.reset_interval,
                   "path": "compress+server+(decompress+adam_frozen_v in one pass)",
                   "inputs": _inputs(wl)},
        "roofline": {"bound": "hbm", "kernel": "onebit_compress", "achieved": round(comp_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(comp_gbs / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 0),
                     "bytes_per_elem": B_COMPRESS, "elems_per_launch": n * N,
                     "launch_ms": round(ms["compress"], 4),
                     # the counters' bytes over the same event-measured duration
                     "counter_GBps": None if traffic is None else
                     round(traffic / (ms["compress"] * 1e-3) / 1e9, 1)},
        "kernels": kernels,
    }
    out["diagnostics"] = diagnostics
    out["rows"] = {"decompress_then_adam": separate}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one step of the workload", file=sys.stderr,
              flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, m, x, v)
    else:
        out["cpu_baseline"] = None
    # the hot kernels beside probes of their memory patterns, on the
    # headline's own buffers (after every use of their contents above)
    # (a diagnostic: a probe that cannot run is reported, never fatal)
    out["rows"]["pattern_ceiling"] = None
    if _probe_lib() is not None:
        print("[bench] pattern probes", file=sys.stderr, flush=True)
        k = max(3, args.steps // 2)
        try:
            pc = measure_probe(wl, k, 1, bufs=(m, grp.ef, grp.bits, grp.ws), modes=[3])
            ps = measure_probe_server(wl, k, 1, grp=grp, m=m)
            out["rows"]["pattern_ceiling"] = {"compress": pc["rows"], "server": ps["rows"]}
            # the same bytes over the probe's time: the access pattern's ceiling
            out["roofline"]["pattern_probe_GBps"] = pc["rows"][0]["GBps"]
        except RuntimeError as exc:
            out["rows"]["pattern_ceiling"] = {"error": str(exc)}
    if not args.no_rows:
        other = "bert_large_335M_x8" if wl.name == "gpt_1.3B_x16" else "gpt_1.3B_x16"
        del grp, m, x, v
        torch.cuda.empty_cache()
        out["rows"].update({"lamb": measure_lamb(max(3, args.steps // 2), 1),
                       "int8": measure_int8(max(3, args.steps // 2), 1),
                       "fused_adam_from_gradients": measure_fused(max(3, args.steps // 2), 1),
                       "warmup": measure_warmup(max(3, args.steps // 2), 1),
                       other: measure_adam_row(other, max(3, args.steps // 2), 1),
                       "copy_reference": measure_copy(max(3, args.steps // 2), 1)})
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
