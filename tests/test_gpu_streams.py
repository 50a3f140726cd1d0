"""Calls on different streams with disjoint buffers are independent: two
1-bit Adam groups and an INT8 quantiser, each driven from a host thread of
its own on a stream of its own (default priority), give results
bit-identical to the same calls made one after the other on one stream."""

import threading

import pytest
import torch

from momentum_compression_amd import onebit as ob
from momentum_compression_amd.state import OneBitGroup
from tests._gpu import device, gen

pytestmark = pytest.mark.gpu

STEPS = 4


def _inputs(dev, n, N, seed):
    g = gen(seed, dev)
    ms = [torch.empty((n, N), device=dev).normal_(0.0, 1e-3, generator=g) for _ in range(STEPS)]
    x = torch.empty(N, device=dev).normal_(0.0, 1.0, generator=g)
    v = torch.empty(N, device=dev).uniform_(1e-8, 1e-6, generator=g)
    return ms, x, v


def _adam_run(dev, n, N, ms, x0, v, stream):
    """STEPS compressed Adam steps of a fresh group on `stream` (None: the
    current stream); the group's buffers are made and filled first."""
    grp = OneBitGroup(N, n, dev)
    x = x0.clone()
    (stream or torch.cuda.current_stream()).synchronize()
    for t in range(1, STEPS + 1):
        grp.compress(ms[t - 1], t, first=t == 1, stream=stream)
        grp.server(t, first=t == 1, stream=stream)
        grp.adam_step(x, v, 6e-5, 1e-6, stream=stream)
    return grp, x


def _int8_run(dev, N, g_list, stream):
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // 256, device=dev)
    deq = torch.empty(N, device=dev)
    (stream or torch.cuda.current_stream()).synchronize()
    for t, g in enumerate(g_list, start=1):
        ob.int8_sr_quantize(g, err, codes, scales, deq, N, 256, 99, t, stream=stream)
    return err, codes, scales, deq


def _same(a, b, what):
    a, b = a.contiguous(), b.contiguous()
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what


def test_concurrent_streams_match_sequential():
    dev = device()
    n, N = 8, 8 * 131072
    NI = 1 << 22
    print(f"[streams] two groups n={n} N={N}, INT8 N={NI}, {STEPS} steps", flush=True)
    ins = [_inputs(dev, n, N, s) for s in (11, 12)]
    gi = gen(13, dev)
    g_list = [torch.empty(NI, device=dev).normal_(0.0, 1e-3, generator=gi) for _ in range(STEPS)]
    torch.cuda.synchronize()
    seq = [_adam_run(dev, n, N, ms, x0, v, None) for ms, x0, v in ins]
    seq_i8 = _int8_run(dev, NI, g_list, None)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(device=dev) for _ in range(3)]  # default priority
    out, errors = [None, None, None], []

    def work(k):
        try:
            with torch.cuda.stream(streams[k]):
                if k < 2:
                    ms, x0, v = ins[k]
                    out[k] = _adam_run(dev, n, N, ms, x0, v, streams[k])
                else:
                    out[k] = _int8_run(dev, NI, g_list, streams[k])
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(3)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        (g_s, x_s), (g_c, x_c) = seq[k], out[k]
        for name in ("ef", "scales", "bits", "sv_ef", "sv_scales", "sv_bits", "mbar"):
            _same(getattr(g_s, name), getattr(g_c, name), f"group {k} {name}")
        _same(x_s, x_c, f"group {k} x")
    for a, b, name in zip(seq_i8, out[2], ("err", "codes", "scales", "deq")):
        _same(a, b, f"int8 {name}")

