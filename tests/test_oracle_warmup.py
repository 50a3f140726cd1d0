"""Pins of the oracle's warmup phase (oracle/warmup.py).

Hand-evaluated steps fix the operand order, the sign of the update, where eps
sits and which x the trust ratio reads; a constant gradient with dyadic betas
gives the moments in closed form; beta2 = 1 reduces the Adam warmup step to
the frozen-variance step; the trust ratio is checked against numpy's norm
and for scale invariance; k_l against layers of constant magnitude.
"""

import math

import numpy as np

from oracle import optim as P
from oracle import warmup as W

F32 = np.float32


def a(*v):
    return np.array(v, dtype=F32)


def test_adam_warmup_hand_point():
    # beta1 = 1/2, beta2 = 3/4: m = (2 + 2)/2 = 2, v = 3 + 1 = 4;
    # x = 3 - 0.5 * (2 / (2 + 0)) = 2.5
    out = W.adam_warmup_step(a(3.0), a(2.0), a(4.0), a(2.0), lr=0.5, eps=0.0, beta1=0.5,
                             beta2=0.75)
    assert out["m"][0] == 2.0 and out["v"][0] == 4.0 and out["x"][0] == 2.5
    # eps outside the root: m = 1/2 g = 1, v = 0 -> x = 0 - 1 * (1 / 0.25) = -4
    out = W.adam_warmup_step(a(0.0), a(0.0), a(0.0), a(2.0), lr=1.0, eps=0.25, beta1=0.5,
                             beta2=1.0)
    assert out["m"][0] == 1.0 and out["v"][0] == 0.0 and out["x"][0] == -4.0


def test_moments_closed_form_constant_gradient():
    """g = 1, beta1 = beta2 = 1/2 from zero: m_t = v_t = 1 - 2^-t exactly."""
    m = v = np.zeros(3, dtype=F32)
    x = np.ones(3, dtype=F32)
    ref_x = 1.0
    lr = 2.0 ** -10
    for t in range(1, 21):
        out = W.adam_warmup_step(x, m, v, np.ones(3, dtype=F32), lr, 0.0, 0.5, 0.5)
        m, v, x = out["m"], out["v"], out["x"]
        assert np.all(m == 1 - 2.0 ** -t) and np.all(v == 1 - 2.0 ** -t)
        ref_x -= lr * (1 - 2.0 ** -t) / math.sqrt(1 - 2.0 ** -t)
        assert np.all(np.abs(x.astype(np.float64) - ref_x) <= t * 2.0 ** -23)


def test_beta2_one_is_frozen_step():
    rng = np.random.default_rng(0)
    x, m, g = (rng.standard_normal(500).astype(F32) for _ in range(3))
    v = np.abs(rng.standard_normal(500)).astype(F32)
    out = W.adam_warmup_step(x, m, v, g, 6e-5, 1e-6, 0.9, 1.0)
    assert np.array_equal(out["v"], v)
    b1 = F32(0.9)
    m_loc = ((b1 * m).astype(F32) + ((F32(1) - b1) * g).astype(F32)).astype(F32)
    assert np.array_equal(out["m"], m_loc)
    assert np.array_equal(out["x"], P.adam_frozen_step(x, m_loc, v, 6e-5, 1e-6))


def test_lamb_warmup_hand_layers():
    """Layer 0: x = (3, 4), u = (1, 0) -> c = 5; layer 1: x = 0 -> c = 1;
    layer 2: u = 0 -> c = 1 and x stays."""
    x = a(3.0, 4.0, 0.0, 0.0, 7.0, -2.0)
    m = a(0.5, 0.0, 0.5, 0.5, 0.0, 0.0)
    v = a(0.25, 0.25, 0.25, 0.25, 1.0, 1.0)
    g = a(0.5, 0.0, 0.5, 0.5, 0.0, 0.0)
    out = W.lamb_warmup_step(x, m, v, g, [0, 2, 4, 6], lr=0.25, eps=0.0, beta1=0.5, beta2=0.5)
    # m = (0.5, 0, 0.5, 0.5, 0, 0); v = (0.25, 0.125, 0.25, 0.25, 0.5, 0.5)
    assert np.array_equal(out["u"], a(1.0, 0.0, 1.0, 1.0, 0.0, 0.0))
    assert np.array_equal(out["c"], a(5.0, 1.0, 1.0))
    assert np.array_equal(out["x"], a(3.0 - 1.25, 4.0, -0.25, -0.25, 7.0, -2.0))
    assert np.array_equal(out["c_avg"], out["c"])  # first step starts the average


def test_trust_ratio_library_norm_and_scale():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(3000).astype(F32)
    u = (rng.standard_normal(3000) * 1e-3).astype(F32)
    c = W.trust_ratio(x, u)
    ref = np.linalg.norm(x.astype(np.float64)) / np.linalg.norm(u.astype(np.float64))
    assert abs(float(c) - ref) <= 2.0 ** -24 * ref * 1.01
    # powers of two scale the ratio exactly
    assert W.trust_ratio((x * F32(4)).astype(F32), u) == F32(4) * c
    assert W.trust_ratio(x, (u * F32(8)).astype(F32)) == c / F32(8)
    assert W.trust_ratio(np.zeros(4, F32), u[:4]) == 1 and W.trust_ratio(x[:4], np.zeros(4, F32)) == 1


def test_lamb_uses_x_before_update():
    """The ratio reads x before the step: with x = (3, 4) the update is lr * 5 * u,
    not a ratio of the updated x."""
    out = W.lamb_warmup_step(a(3.0, 4.0), a(0.5, 0.0), a(0.25, 0.25), a(0.5, 0.0), [0, 2],
                             lr=0.5, eps=0.0, beta1=0.5, beta2=0.5)
    assert out["x"][0] == F32(3.0 - 2.5)


def test_coefficient_average_by_hand():
    c1, c2, c3 = a(2.0, 8.0), a(4.0, 0.0), a(1.0, 1.0)
    avg = W.coefficient_average(None, c1, 0.5)
    assert np.array_equal(avg, c1)
    avg = W.coefficient_average(avg, c2, 0.5)
    assert np.array_equal(avg, a(3.0, 4.0))
    avg = W.coefficient_average(avg, c3, 0.75)
    assert np.array_equal(avg, a(2.5, 3.25))


def test_momentum_scale_constant_magnitude_layers():
    """RMS (1, 1, 4) over layers of 4, 16 and 8 elements: mean 2, k = (2, 2, 1/2).
    A wrong normalisation (norm instead of RMS) would split layers 0 and 1."""
    m = np.concatenate([a(1, -1, 1, -1), np.full(16, F32(-1.0)), np.full(8, F32(4.0))])
    off = [0, 4, 20, 28]
    assert np.array_equal(W.momentum_scale(m, off), a(2.0, 2.0, 0.5))
    # sign and scale (power of two) invariance; permutation within a layer
    assert np.array_equal(W.momentum_scale((-8 * m).astype(F32), off), a(2.0, 2.0, 0.5))
    perm = m.copy()
    perm[20:28] = perm[20:28][::-1]
    assert np.array_equal(W.momentum_scale(perm, off), a(2.0, 2.0, 0.5))


def test_momentum_scale_zero_and_empty_layers():
    m = np.concatenate([np.zeros(4, F32), np.full(4, F32(3.0)), np.full(4, F32(1.0))])
    off = [0, 4, 4, 8, 12]  # zero layer, empty layer, RMS 3, RMS 1
    k = W.momentum_scale(m, off)
    assert np.array_equal(k, a(1.0, 1.0, 2.0 / 3.0, 2.0))


def test_momentum_scale_equalises_rms():
    """After scaling by k_l every layer's RMS equals the mean RMS (to rounding)."""
    rng = np.random.default_rng(2)
    sizes = [5, 100, 1000, 64, 3000]
    sig = [1e-5, 1e-2, 3e-4, 1.0, 2e-3]
    m = np.concatenate([(rng.standard_normal(d) * s).astype(F32) for d, s in zip(sizes, sig)])
    off = np.concatenate([[0], np.cumsum(sizes)])
    k = W.momentum_scale(m, off)
    rms = [math.sqrt(float(W.exact_rms_ratio(m, off, l))) for l in range(len(sizes))]
    mean = sum(rms) / len(rms)
    for l in range(len(sizes)):
        assert abs(float(k[l]) * rms[l] / mean - 1.0) < 1e-6


def test_lamb_direction_uses_new_moments():
    """u reads the updated m and v: m = 0 -> 1/2, v = 0 -> 1/4 gives u = 1
    (the old moments would give 0/0)."""
    out = W.lamb_warmup_step(a(0.0, 2.0), a(0.0, 0.0), a(0.0, 1.0), a(1.0, 0.0), [0, 2],
                             lr=0.5, eps=0.0, beta1=0.5, beta2=0.75)
    assert np.array_equal(out["m"], a(0.5, 0.0)) and np.array_equal(out["v"], a(0.25, 0.75))
    assert np.array_equal(out["u"], a(1.0, 0.0))
    # ||x|| = 2, ||u|| = 1: c = 2, x = (0 - 0.5 * 2 * 1, 2)
    assert out["c"][0] == 2.0 and np.array_equal(out["x"], a(-1.0, 2.0))


# ------------------------------------------ rounding of the exact layer norms
# The readings fix how the exact sums become binary32 results: each squared
# norm is the exact sum rounded once to binary64; the trust ratio is the
# binary64 quotient of the two correctly rounded roots; the RMS is the
# correctly rounded root of the correctly rounded mean square.  The cases
# below are built (with exact integer arithmetic, independent of the oracle)
# so that the other natural compositions give a different binary32 result.

from fractions import Fraction  # noqa: E402

from tests._exactref import rn, rn64, sqrt_rn64  # noqa: E402


def _exact_sumsq(vals) -> Fraction:
    return sum(Fraction(float(v)) ** 2 for v in np.asarray(vals, dtype=F32))


def _complete_squares(target: Fraction, count: int = 4) -> list:
    """Up to `count` binary32 values whose squares sum to at most `target`,
    within about target 2^-90 of it (each the largest square that fits)."""
    vals, rem = [], target
    for _ in range(count):
        if rem <= 0:
            break
        y = F32(math.sqrt(float(rem)))
        while Fraction(float(y)) ** 2 > rem:
            y = np.nextafter(y, F32(0), dtype=F32)
        if y == 0:
            break
        vals.append(y)
        rem -= Fraction(float(y)) ** 2
    return vals


def _midpoint(k: int) -> Fraction:
    """The binary32 midpoint just above f = 1 + k 2^-15 + 2^-23, whose
    significand is odd, so that the tie rounds up (to even) while anything
    just below the midpoint rounds down."""
    f = F32(1.0 + k * 2.0 ** -15 + 2.0 ** -23)
    return (Fraction(float(f)) + Fraction(float(np.nextafter(f, F32(2), dtype=F32)))) / 2


def test_exact_rounding_helpers_match_ieee_binary64():
    """rn64 and sqrt_rn64, which the rounding pins below rest on, agree with
    the platform's correctly rounded binary64 division and square root on
    seeded operands over a wide exponent range, and on exact squares."""
    rng = np.random.default_rng(20)
    x = rng.uniform(1, 2, 3000) * 2.0 ** rng.integers(-300, 300, 3000)
    y = rng.uniform(1, 2, 3000) * 2.0 ** rng.integers(-300, 300, 3000)
    r = (rng.uniform(1, 2, 3000) * 2.0 ** rng.integers(-120, 120, 3000)).astype(F32)
    for a_, b_, r_ in zip(x, y, r):
        assert rn64(Fraction(a_) / Fraction(b_)) == Fraction(a_ / b_)
        assert sqrt_rn64(Fraction(a_)) == Fraction(math.sqrt(a_))
        assert sqrt_rn64(Fraction(float(r_)) ** 2) == Fraction(float(r_))


def test_sum_of_squares_is_exact_then_rounded_once():
    """Squares 1, eight of 2^-56 and 2^-200: the exact sum 1 + 2^-53 + 2^-200
    lies just above the midpoint between 1 and 1 + 2^-52, so its binary64
    rounding is 1 + 2^-52, while a running binary64 sum drops every small
    square and returns 1."""
    v = a(1.0, *([2.0 ** -28] * 8), 2.0 ** -100)
    want = rn64(_exact_sumsq(v))
    assert want == 1 + Fraction(2) ** -52
    assert W.exact_sumsq(v) == float(want)


def test_trust_ratio_is_the_quotient_of_the_roots():
    """||u||^2 = 2 and ||x|| / ||u|| within about 2^-80 of a binary32
    midpoint: the reading's fl32(fl64(fl64(sqrt Sx) / fl64(sqrt Su))) and
    the root of the quotient fl32(fl64(sqrt(fl64(Sx / Su)))) round to
    different binary32 values; the oracle must give the first."""
    u = a(1.0, 1.0)
    for k in range(1, 2000):
        M = _midpoint(k)
        x = a(*_complete_squares(2 * M * M))
        sx = rn64(_exact_sumsq(x))
        reading = rn(rn64(sqrt_rn64(sx) / sqrt_rn64(Fraction(2))))
        other = rn(sqrt_rn64(rn64(sx / 2)))
        if reading != other:
            break
    else:
        raise AssertionError("no discriminating case found")
    assert W.trust_ratio(x, u) == reading


def test_rms_is_the_root_of_the_rounded_mean_square():
    """Layer 0 holds the single value 1 and layer 1 three values whose RMS
    is within about 2^-70 of 2T - 1 - 2^-51 for a binary32 midpoint T (odd
    significand below it). The reading's a_1 = fl64(sqrt(fl64(S_1 / 3)))
    is that value, 1 + a_1 = 2T - 2^-51 is exact and k_0 = fl32(T - 2^-52)
    rounds down; where the quotient of roots fl64(fl64(sqrt S_1) /
    fl64(sqrt 3)) comes out one binary64 step higher, 1 + a_1 ties to the
    even 2T and k_0 = fl32(T) rounds up. The oracle must give the reading's
    k (the mean: the exact sum of the RMS values rounded once, then divided
    by the count)."""
    off = np.array([0, 1, 4], dtype=np.int64)

    def k_of(a1):
        mean = rn64(rn64(1 + a1) / 2)
        return np.array([rn(rn64(mean / 1)), rn(rn64(mean / a1))], dtype=F32)

    for k in range(1, 2000):
        T = _midpoint(k)
        m = np.zeros(4, dtype=F32)
        m[0] = 1.0
        fill = _complete_squares(3 * (2 * T - 1 - Fraction(2) ** -51) ** 2, count=3)
        m[1:1 + len(fill)] = fill
        s1 = rn64(_exact_sumsq(m[1:4]))
        want = k_of(sqrt_rn64(rn64(s1 / 3)))
        other = k_of(rn64(sqrt_rn64(s1) / sqrt_rn64(Fraction(3))))
        if not np.array_equal(want, other):
            break
    else:
        raise AssertionError("no discriminating case found")
    assert np.array_equal(W.momentum_scale(m, off), want)


def test_mean_of_rms_values_is_summed_exactly():
    """RMS values 1, y, delta, delta with 1 + y = 4T - 2^-50 (T a binary32
    midpoint with odd significand below it) and delta the binary32 value
    just below 2^-51: the exact sum rounds once to 4T, the mean over the
    four layers is T and k_0 = fl32(T) rounds up, while a running binary64
    sum drops both deltas (each under half a step of 1 + y), leaving the
    mean T - 2^-52 and k_0 rounding down."""
    off = np.array([0, 1, 4, 5, 6], dtype=np.int64)
    delta = np.nextafter(F32(2.0 ** -51), F32(0), dtype=F32)
    for k in range(1, 2000):
        T = _midpoint(k)
        y = 4 * T - 1 - Fraction(2) ** -50
        m = np.zeros(6, dtype=F32)
        m[0] = 1.0
        fill = _complete_squares(3 * y ** 2, count=3)
        m[1:1 + len(fill)] = fill
        m[4] = m[5] = delta
        if sqrt_rn64(rn64(_exact_sumsq(m[1:4]) / 3)) == y:
            break
    else:
        raise AssertionError("no layer with RMS exactly y found")
    d = Fraction(float(delta))
    want = np.array([rn(T), rn(rn64(T / y)), rn(rn64(T / d)), rn(rn64(T / d))],
                    dtype=F32)
    assert rn(T) != rn(T - Fraction(2) ** -52)
    assert np.array_equal(W.momentum_scale(m, off), want)


def test_lamb_step_takes_this_steps_coefficient_not_the_average():
    """With a running average already in place (c_avg = 2 from earlier
    steps), the step still moves x by lr * c_l * u with this step's c_l = 5
    (x = (3, 4), u = (1, 0)); the average moves to 1/2 * 2 + 1/2 * 5."""
    out = W.lamb_warmup_step(a(3.0, 4.0), a(0.5, 0.0), a(0.25, 0.25), a(0.5, 0.0), [0, 2],
                             lr=0.25, eps=0.0, beta1=0.5, beta2=0.5, c_avg=a(2.0), beta_c=0.5)
    assert out["c"][0] == 5
    assert np.array_equal(out["x"], a(3.0 - 1.25, 4.0))
    assert out["c_avg"][0] == F32(3.5)


def test_moments_and_average_rounding_sequences():
    """m = fl(fl(b1 m) + fl(fl(1 - b1) g)), v = fl(fl(b2 v) + fl(fl(1 - b2)
    fl(g g))) and c_avg = fl(fl(b_c c_avg) + fl(fl(1 - b_c) c)): each 1 - b
    formed from the binary32 b (exact for these b), the square before the
    product. Exact rationals on seeded values; the sample also separates the
    sequence from the square taken last and from 1 - b of the binary64 b."""
    rng = np.random.default_rng(30)
    n = 400
    m = (rng.standard_normal(n) * 1e-2).astype(F32)
    v = (np.abs(rng.standard_normal(n)) * 1e-4).astype(F32)
    v[::2] = 0  # fresh variance: the new term alone, so its rounding shows
    g = (rng.standard_normal(n) * 1e-2).astype(F32)
    b1, b2, bc = F32(0.9), F32(0.999), F32(0.9)
    fr = lambda t: Fraction(float(t))  # noqa: E731
    o1, o2, oc = fr(F32(1) - b1), fr(F32(1) - b2), fr(F32(1) - bc)
    want_m = [rn(fr(rn(fr(b1) * fr(mi))) + fr(rn(o1 * fr(gi)))) for mi, gi in zip(m, g)]
    want_v = [rn(fr(rn(fr(b2) * fr(vi))) + fr(rn(o2 * fr(rn(fr(gi) * fr(gi))))))
              for vi, gi in zip(v, g)]
    m_new, v_new = W.moments(m, v, g, 0.9, 0.999)  # the caller's binary64 betas
    assert np.array_equal(m_new, np.array(want_m, dtype=F32))
    assert np.array_equal(v_new, np.array(want_v, dtype=F32))
    square_last = [rn(fr(rn(fr(b2) * fr(vi))) + fr(rn(fr(rn(o2 * fr(gi))) * fr(gi))))
                   for vi, gi in zip(v, g)]
    assert want_v != square_last
    c_avg = (rng.uniform(0.5, 3, n)).astype(F32)
    c = (rng.uniform(0.5, 3, n)).astype(F32)
    want_c = [rn(fr(rn(fr(bc) * fr(ai))) + fr(rn(oc * fr(ci)))) for ai, ci in zip(c_avg, c)]
    assert np.array_equal(W.coefficient_average(c_avg, c, 0.9), np.array(want_c, dtype=F32))
    # 1 - b_c taken from the binary64 0.9 (0.09999999999999998), not from
    # binary32 b_c (1 - fl32(0.9) = 0.10000002384..., exact)
    unrounded = [rn(fr(rn(fr(bc) * fr(ai))) + fr(rn(Fraction(1.0 - 0.9) * fr(ci))))
                 for ai, ci in zip(c_avg, c)]
    assert want_c != unrounded
