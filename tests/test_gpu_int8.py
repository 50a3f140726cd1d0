"""GPU parity of block-wise INT8 stochastic rounding with error feedback
(codes bit-exact, scales / dequantised values / residuals bit-identical) and
of the device Philox stream."""

import numpy as np
import pytest
import torch

from momentum_compression_amd import onebit as ob
from oracle.int8 import int8_sr
from tests._gpu import device, gen, host, same_f32
from workloads import synth as S

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.mark.parametrize("block", [64, 128, 256, 512, 1024])
def test_int8_free_running(block):
    dev = device()
    N = block * 997 if block <= 256 else block * 251  # not a multiple of the 1024-element tile
    print(f"[int8 parity] N={N} block={block}", flush=True)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    e_h = np.zeros(N, dtype=F32)
    seed = 0x1234_5678_9ABC
    for step in range(1, 4):
        g = S.laplace_gradient(N, step, 4, dev)
        g_h = host(g)
        ob.int8_sr_quantize(g, err, codes, scales, deq, N, block, seed, step)
        torch.cuda.synchronize()
        o = int8_sr(g_h, e_h, seed, step, block)
        tag = f"step={step}"
        assert np.array_equal(host(codes), o["codes"]), f"{tag} codes"
        same_f32(host(scales), o["scales"], f"{tag} scales")
        same_f32(host(deq), o["deq"], f"{tag} dequantised")
        same_f32(host(err), o["e"], f"{tag} residual")
        e_h = o["e"]


def test_int8_without_feedback_and_specials():
    dev = device()
    N, block = 256 * 64, 256
    g = S.laplace_gradient(N, 1, 9, dev)
    g[:256] = 0.0                       # all-zero block
    g[256:512] = torch.arange(256, device=dev, dtype=torch.float32) - 128  # integral, scale 1
    g[256 + 255] = 127.0
    g[600] = float("nan")
    g[900] = float("inf")
    g[1300] = -float("inf")
    g[2000:2100] = 1e-41                # subnormal block content
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    ob.int8_sr_quantize(g, None, codes, scales, deq, N, block, 77, 5)
    torch.cuda.synchronize()
    o = int8_sr(host(g), None, 77, 5, block)
    assert np.array_equal(host(codes), o["codes"])
    same_f32(host(scales), o["scales"], "scales")
    same_f32(host(deq), o["deq"], "deq")
    assert np.all(host(codes)[:256] == 0)


def test_int8_fraction_equal_to_its_uniform():
    """Elements whose fraction equals their own Philox uniform round down
    (u < p); one grid step of the uniforms above, they round up."""
    from tests.test_oracle_int8 import _tie_block

    dev = device()
    for above in (False, True):
        g_h, idx = _tie_block(5, 2, above)
        print(f"[int8 tie] above={above}", flush=True)
        g = torch.from_numpy(g_h).to(dev)
        codes = torch.empty(256, dtype=torch.int8, device=dev)
        scales = torch.empty(1, device=dev)
        deq = torch.empty(256, device=dev)
        ob.int8_sr_quantize(g, None, codes, scales, deq, 256, 256, 5, 2)
        torch.cuda.synchronize()
        o = int8_sr(g_h, None, 5, 2, 256)
        assert np.array_equal(host(codes), o["codes"])
        assert np.all(host(codes)[idx] == (1 if above else 0))
        same_f32(host(deq), o["deq"], "deq")


def test_int8_large_step_counter_and_index():
    """Element indices beyond 2^32 exercise the high counter word."""
    dev = device()
    N, block = (1 << 32) + (1 << 14), 256
    free = torch.cuda.mem_get_info()[0]
    if free < N * 7:
        pytest.skip("not enough device memory for a 2^32-element buffer")
    g = torch.empty(N, device=dev)
    g.normal_(0.0, 1e-3, generator=gen(1, dev))
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    ob.int8_sr_quantize(g, None, codes, scales, None, N, block, 2**40 + 3, 0xFFFF_FFF0)
    torch.cuda.synchronize()
    for J0 in (0, (1 << 32) - 512, 1 << 32):
        sl = slice(J0, J0 + 1024)
        o = int8_sr(host(g[sl]), None, 2**40 + 3, 0xFFFF_FFF0, block, J0=J0)
        assert np.array_equal(host(codes[sl]), o["codes"]), J0


def test_int8_clamp_reached_from_128():
    """The block maxima of the oracle pin's clamp case (x = -(127 + 2^-17)
    and +(127 + 2^-17) at elements whose uniforms send them to -128 and
    +128 before the clamp) code to -127 and +127 on the GPU too, bit-exact
    with the oracle over the whole buffer, residuals included."""
    from tests.test_oracle_int8 import clamp_case

    dev = device()
    seed, step, block = 3, 1, 256
    M, scale, j_neg, j_pos = clamp_case(seed, step)
    N = 1 << 19
    print(f"[int8 clamp] N={N} J-={j_neg} J+={j_pos}", flush=True)
    g_h = np.zeros(N, dtype=F32)
    g_h[j_neg], g_h[j_pos] = -M, M
    g = torch.from_numpy(g_h).to(dev)
    err = torch.zeros(N, device=dev)
    codes = torch.empty(N, dtype=torch.int8, device=dev)
    scales = torch.empty(N // block, device=dev)
    deq = torch.empty(N, device=dev)
    ob.int8_sr_quantize(g, err, codes, scales, deq, N, block, seed, step)
    torch.cuda.synchronize()
    o = int8_sr(g_h, np.zeros(N, dtype=F32), seed, step, block)
    c = host(codes)
    assert int(c[j_neg]) == -127 and int(c[j_pos]) == 127
    assert np.array_equal(c, o["codes"])
    same_f32(host(scales), o["scales"], "scales")
    same_f32(host(deq), o["deq"], "deq")
    same_f32(host(err), o["e"], "residual")
