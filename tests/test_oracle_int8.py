"""Pins of the oracle's block-wise INT8 stochastic rounding (oracle/int8.py).

Properties fixed by the gradient-quantisation tutorial's INT8 recipe: codes
stay in [-127, 127]; the dequantised value is within one scale step of the
input; an input that is an exact multiple of the scale is coded exactly;
zero blocks stay zero; the block maximum codes to 126 or 127; stochastic
rounding is unbiased and rounds up with probability equal to the fraction,
which fixes the comparison u < p (a fraction equal to its uniform rounds down).
"""

import numpy as np

from oracle.int8 import int8_sr
from oracle.philox import uniforms

F32 = np.float32


def _laplace(rng, n, b=1e-3):
    return rng.laplace(0.0, b, size=n).astype(F32)


def test_codes_range_and_error_bound():
    rng = np.random.default_rng(0)
    g = _laplace(rng, 256 * 64)
    g[::997] *= 100
    out = int8_sr(g, None, seed=4, step=1)
    q = out["codes"].astype(np.int32)
    assert q.min() >= -127 and q.max() <= 127
    sc = np.repeat(out["scales"], 256).astype(np.float64)
    err = np.abs(out["deq"].astype(np.float64) - g.astype(np.float64))
    assert np.all(err < sc * (1 + 2.0 ** -20))
    # scale = max|g| / 127 per block (one binary32 division)
    M = np.abs(g).reshape(-1, 256).max(axis=1)
    assert np.array_equal(out["scales"], (M / F32(127)).astype(F32))


def test_integral_inputs_are_exact():
    # block max 127 gives scale exactly 1, so integers code to themselves
    rng = np.random.default_rng(1)
    g = rng.integers(-127, 128, size=256).astype(F32)
    g[17] = 127
    out = int8_sr(g, None, seed=9, step=3)
    assert out["scales"][0] == 1
    assert np.array_equal(out["codes"].astype(F32), g)
    assert np.array_equal(out["deq"], g)
    assert np.all(out["e"] == 0)


def _tie_block(seed, step, above):
    """One block whose maximum 127 gives scale 1 and whose other elements
    carry x = u_J (above=False) or u_J + 2^-24 (above=True): fraction p = x."""
    u = uniforms(0, 256, seed, step)
    idx = np.array([j for j in range(1, 256) if u[j] > 0][:64])
    g = np.zeros(256, dtype=F32)
    g[0] = 127
    g[idx] = (u[idx] + (F32(2.0 ** -24) if above else F32(0))).astype(F32)
    return g, idx


def test_fraction_equal_to_its_uniform_rounds_down():
    """Rounding up with probability p, the fraction: of the 2^24 equally likely
    uniforms (multiples of 2^-24 in [0, 1)) exactly p * 2^24 lie below a p that
    is itself such a multiple, so the unbiased rule is u < p, and u == p rounds
    down (u <= p would round up with probability p + 2^-24)."""
    g, idx = _tie_block(5, 2, above=False)
    out = int8_sr(g, None, seed=5, step=2)
    assert out["scales"][0] == 1
    assert np.all(out["codes"][idx] == 0)
    g, idx = _tie_block(5, 2, above=True)
    out = int8_sr(g, None, seed=5, step=2)
    assert np.all(out["codes"][idx] == 1)


def test_zero_block_and_max_code():
    rng = np.random.default_rng(2)
    g = _laplace(rng, 512)
    g[:256] = 0.0
    out = int8_sr(g, None, seed=1, step=1)
    assert np.all(out["codes"][:256] == 0) and np.all(out["deq"][:256] == 0)
    assert out["scales"][0] == 0
    j = 256 + int(np.argmax(np.abs(g[256:])))
    assert abs(int(out["codes"][j])) in (126, 127)


def test_error_feedback_adds_residual():
    rng = np.random.default_rng(3)
    g = _laplace(rng, 1024)
    e = _laplace(rng, 1024, 1e-4)
    a = int8_sr(g, e, seed=2, step=5)
    b = int8_sr((g + e).astype(F32), None, seed=2, step=5)
    for key in ("codes", "scales", "deq", "e"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["e"], ((g + e).astype(F32) - a["deq"]).astype(F32))


def test_rounds_up_with_probability_of_fraction():
    # scale 1 (max 127): values k + 1/4 round up a quarter of the time
    n = 256 * 400
    g = np.full(n, F32(10.25))
    g[::256] = 127
    out = int8_sr(g, None, seed=11, step=2)
    mask = np.ones(n, dtype=bool)
    mask[::256] = False
    up = (out["codes"][mask] == 11).mean()
    assert abs(up - 0.25) < 4 * np.sqrt(0.25 * 0.75 / mask.sum())
    assert set(np.unique(out["codes"][mask])) <= {10, 11}


def test_unbiased_over_seeds():
    rng = np.random.default_rng(4)
    g = _laplace(rng, 256 * 4)
    acc = np.zeros(g.size)
    seeds = 256
    for s in range(seeds):
        acc += int8_sr(g, None, seed=1000 + s, step=1)["deq"].astype(np.float64) - g
    mean_err = acc / seeds
    sc = np.repeat(int8_sr(g, None, seed=0, step=1)["scales"], 256).astype(np.float64)
    # each draw has |err| < scale, so the std of the mean is below scale/2/16
    assert np.all(np.abs(mean_err) <= 4 * 0.5 * sc / np.sqrt(seeds))


def test_uniforms_grid_and_range():
    u = uniforms(12345, 10000, seed=7, step=3)
    assert u.min() >= 0 and u.max() < 1
    assert np.all((u * 2 ** 24) == np.floor(u * 2 ** 24))
    assert abs(u.mean() - 0.5) < 0.02


def test_nearest_rounding_hand_values():
    """Round to nearest, halves away from zero (tutorial, step 1)."""
    from oracle.int8 import round_half_away
    x = np.array([2.5, -2.5, 2.4999998, -0.5, 0.5, 126.5, -126.5, 3.0, -0.49999997, 0.0],
                 dtype=F32)
    assert round_half_away(x).tolist() == [3, -3, 2, -1, 1, 127, -127, 3, -0, 0]
    # block max 127 -> scale 1: codes are the rounded inputs, clamped to +-127
    g = np.zeros(256, dtype=F32)
    g[:6] = [127, -126.5, 2.5, -2.5, 0.4, 1.5]
    out = int8_sr(g, None, seed=1, step=1, rounding="nearest")
    assert out["codes"][:6].tolist() == [127, -127, 3, -3, 0, 2]


def test_per_tensor_scale():
    """block = 0: one scale from the max over the whole tensor (the PyTorch
    example)."""
    rng = np.random.default_rng(6)
    g = _laplace(rng, 4096)
    g[1234] = 0.5
    out = int8_sr(g, None, seed=3, step=2, block=0)
    assert out["scales"].shape == (1,)
    assert out["scales"][0] == F32(0.5) / F32(127)
    assert out["codes"][1234] in (126, 127)
    q = out["codes"].astype(np.int32)
    assert q.min() >= -127 and q.max() <= 127


def clamp_case(seed: int = 3, step: int = 1):
    """A block maximum M (the first binary32 above 1 with this property)
    whose scale fl(M / 127) rounds down, so that the maximum's x is
    +-(127 + 2^-17), and the first element indices below 2^19 whose uniform
    lies on the far side of the fraction: u >= p for -x (floor -128), u < p
    for +x. Returns (M, scale, J for -M, J for +M)."""
    M = F32(1.0)
    while F32(M / F32(M / F32(127))) <= F32(127):
        M = np.nextafter(M, F32(2), dtype=F32)
    scale = F32(M / F32(127))
    x = F32(M / scale)
    assert x > F32(127) and np.floor(-x) == -128
    u = uniforms(0, 1 << 19, seed, step)
    j_neg = int(np.nonzero(u >= F32(F32(-x) + F32(128)))[0][0])
    j_pos = int(np.nonzero(u < F32(x - F32(127)))[0][0])
    return M, scale, j_neg, j_pos


def test_codes_clamp_to_127_on_both_sides():
    """The clamp to [-127, 127] (tutorial, step 3) is reached: with the
    block maximum of clamp_case() at an element whose uniform lies on the
    far side of its fraction, the rounded value is -128 or +128, and the
    code must come out -127 or +127, with deq = +-127 scale and
    e = g' - deq."""
    seed, step = 3, 1
    M, scale, j_neg, j_pos = clamp_case(seed, step)
    for J, sign in ((j_neg, -1), (j_pos, 1)):
        b, j = divmod(J, 256)
        g = np.zeros(256, dtype=F32)
        g[j] = F32(sign) * M
        out = int8_sr(g, None, seed=seed, step=step, J0=256 * b)
        assert out["scales"][0] == scale
        assert int(out["codes"][j]) == 127 * sign
        deq = F32(F32(127 * sign) * scale)
        assert out["deq"][j] == deq and out["e"][j] == F32(g[j] - deq)


def test_nan_is_left_out_of_the_block_maximum():
    """M is the maximum of |g'| over the block's non-NaN elements, so a NaN
    leaves the other codes as they were; the NaN's own x is NaN, which the
    fmin/fmax clamp turns into -127."""
    g = np.zeros(256, dtype=F32)
    g[:4] = [127, np.nan, 5, -3]
    out = int8_sr(g, None, seed=1, step=1)
    assert out["scales"][0] == 1
    assert out["codes"][[0, 2, 3]].tolist() == [127, 5, -3]
    assert int(out["codes"][1]) == -127 and out["deq"][1] == -127
    assert np.isnan(out["e"][1])
