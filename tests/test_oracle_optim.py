"""Pins of the oracle's frozen-variance steps (oracle/optim.py).

Hand-evaluated points fix operand order, the sign of the update and where
eps sits; the LAMB pieces are pinned by the momentum round trip of the
gradient reconstruction (1-bit LAMB algorithm paragraph), the clip bounds of
r_t, the basic-1-bit-LAMB special case r_min = r_max = 1, and a fixed point
where the fresh variance equals the frozen one.
"""

from fractions import Fraction

import numpy as np

from oracle import optim as P
from tests._exactref import rn

F32 = np.float32


def a(*v):
    return np.array(v, dtype=F32)


def test_adam_hand_points():
    # x=1, m=0.5, v=0.25, eps=0, lr=0.5: 1 - 0.5 * (0.5 / 0.5) = 0.5
    assert P.adam_frozen_step(a(1.0), a(0.5), a(0.25), 0.5, 0.0)[0] == F32(0.5)
    # eps outside the root: x=0, m=1, v=0, eps=0.25, lr=1 -> -(1/0.25) = -4
    assert P.adam_frozen_step(a(0.0), a(1.0), a(0.0), 1.0, 0.25)[0] == F32(-4.0)
    # sqrt(4) + 0 = 2: x=3, m=-4, lr=0.25 -> 3 + 0.25*2 = 3.5
    assert P.adam_frozen_step(a(3.0), a(-4.0), a(4.0), 0.25, 0.0)[0] == F32(3.5)


def test_adam_special_cases():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000).astype(F32)
    v = np.abs(rng.standard_normal(1000)).astype(F32)
    m = rng.standard_normal(1000).astype(F32)
    assert np.array_equal(P.adam_frozen_step(x, np.zeros_like(m), v, 6e-5, 1e-6), x)
    assert np.array_equal(P.adam_frozen_step(x, m, v, 0.0, 1e-6), x)
    up = P.adam_frozen_step(x, m, v, 6e-5, 1e-6)
    assert np.all(np.sign(x - up)[m != 0] == np.sign(m[m != 0]))  # moves against m


def test_gradient_reconstruction_round_trip_exact():
    """beta1 = 1/2 keeps every operation exact: m = b1 m_prev + (1-b1) g
    reconstructs g bit for bit."""
    rng = np.random.default_rng(1)
    g = (rng.integers(-1000, 1000, size=500) / 1024).astype(F32)
    mp = (rng.integers(-1000, 1000, size=500) / 1024).astype(F32)
    m = (F32(0.5) * mp + F32(0.5) * g).astype(F32)
    assert np.array_equal(P.reconstruct_gradient(m, mp, 0.5), g)


def test_gradient_reconstruction_round_trip_beta09():
    """beta1 = 0.9: the momentum recursion evaluated in binary32 is inverted up
    to its roundings, which the division by 1 - beta1 amplifies tenfold."""
    rng = np.random.default_rng(2)
    g = rng.standard_normal(2000).astype(F32)
    mp = rng.standard_normal(2000).astype(F32)
    b1 = F32(0.9)
    m = ((b1 * mp).astype(F32) + ((F32(1) - b1) * g).astype(F32)).astype(F32)
    rec = P.reconstruct_gradient(m, mp, 0.9).astype(np.float64)
    u = 2.0 ** -24
    tol = 10 * 2 * u * (np.abs(m) + np.abs(mp)) + 4 * u * np.abs(g)
    assert np.all(np.abs(rec - g) <= tol)
    # a wrong formula (e.g. dividing by beta1) is far outside that band
    assert np.median(np.abs(rec - g) / np.abs(g)) < 1e-5


def test_fresh_variance_hand_point():
    assert P.fresh_variance(a(4.0), a(2.0), 0.5)[0] == F32(4.0)
    assert P.fresh_variance(a(0.0), a(3.0), 0.75)[0] == F32(2.25)


def test_ratio_clip_bounds():
    rng = np.random.default_rng(3)
    R = np.exp(rng.uniform(-3, 3, size=5000)).astype(F32)
    r_prev = np.exp(rng.uniform(np.log(0.5), np.log(4.0), size=5000)).astype(F32)
    r, c = P.lamb_ratio_update(R, r_prev, np.ones_like(R), 0.1, 0.5, 4.0)
    lo = np.maximum(F32(0.5), F32(0.9) * r_prev)
    hi = np.minimum(F32(4.0), F32(1.1) * r_prev)
    assert np.all(r >= F32(0.5)) and np.all(r <= F32(4.0))
    ok = lo <= hi
    assert np.all((r >= lo)[ok]) and np.all((r <= hi)[ok])
    inside = ok & (R >= lo) & (R <= hi)
    assert np.array_equal(r[inside], R[inside])
    assert np.array_equal(c, r)


def test_ratio_outer_clip_is_hard():
    """The page nests the soft clip inside the hard one, so with r_{t-1}
    outside [r_min, r_max] the hard bounds win: r_{t-1} = 1.3 with
    r_min = r_max = 1 gives 1 (the other nesting would give 1.17), and
    r_{t-1} = 5 with r_max = 4 gives 4 (not 4.5)."""
    r, _ = P.lamb_ratio_update(a(0.2, 1.0, 10.0), a(1.3, 1.3, 5.0), a(1.0, 1.0, 1.0), 0.1,
                               1.0, 1.0)
    assert r.tolist() == [1.0, 1.0, 1.0]
    r, c = P.lamb_ratio_update(a(10.0, 1.0), a(5.0, 5.0), a(2.0, 2.0), 0.1, 0.5, 4.0)
    assert r.tolist() == [4.0, 4.0] and c.tolist() == [8.0, 8.0]


def test_ratio_no_valid_keeps_previous():
    r, c = P.lamb_ratio_update(a(np.nan), a(1.7), a(2.0), 0.1, 0.5, 4.0)
    assert r[0] == F32(1.7) and c[0] == F32(3.4)


def test_basic_onebit_lamb_special_case():
    """r_min = r_max = 1 freezes the coefficient at c_avg."""
    rng = np.random.default_rng(4)
    R = np.exp(rng.uniform(-5, 5, size=100)).astype(F32)
    cav = rng.uniform(0.5, 2, size=100).astype(F32)
    r, c = P.lamb_ratio_update(R, np.ones(100, dtype=F32), cav, 0.1, 1.0, 1.0)
    assert np.all(r == 1) and np.array_equal(c, cav)


def test_layer_max_semantics():
    vals = a(1.0, np.nan, 3.0, np.nan, np.nan, -0.0, 0.0, np.inf, 2.0)
    R = P.layer_max(vals, [0, 3, 5, 7, 9])
    assert R[0] == 3.0 and np.isnan(R[1]) and R[2] == 0.0 and not np.signbit(R[2]) and R[3] == np.inf


def test_lamb_fixed_point_and_step():
    """g^2 = v_Tw with v = v_Tw and beta2 = 1/2: the fresh variance stays v_Tw,
    every ratio is 1 and r_t = r_{t-1} = 1; the update uses c_{t-1}."""
    g = a(2.0, -2.0, 0.5, 0.5)
    mp = a(0.0, 0.0, 0.0, 0.0)
    b1 = 0.5
    m = (F32(1 - b1) * g).astype(F32)
    v = (g * g).astype(F32)
    x = a(1.0, 1.0, 1.0, 1.0)
    out = P.lamb_frozen_step(x, m, mp, v, v, [0, 2, 4], c_avg=a(2.0, 3.0), r_prev=a(1.0, 1.0),
                             c_prev=a(0.5, 0.25), lr=1.0, eps=0.0, beta1=b1, beta2=0.5,
                             thr=0.1, r_min=0.5, r_max=4.0)
    assert np.array_equal(out["v"], v)
    assert np.array_equal(out["R"], a(1.0, 1.0)) and np.array_equal(out["r"], a(1.0, 1.0))
    assert np.array_equal(out["c"], a(2.0, 3.0))
    # x - (lr c_prev) * m / sqrt(v): layer 0 step 0.5 * (1/2 or -1/2) ; layer 1 step 0.25 * 0.5
    assert np.array_equal(out["x"], a(0.75, 1.25, 0.875, 0.875))
    out_b = P.lamb_frozen_step(x, m, mp, v, v, [0, 2, 4], c_avg=a(2.0, 3.0), r_prev=a(1.0, 1.0),
                               c_prev=a(0.5, 0.25), lr=1.0, eps=0.0, beta1=b1, beta2=0.5,
                               thr=0.1, r_min=0.5, r_max=4.0, use_c_t=True)
    assert np.array_equal(out_b["x"], a(0.0, 2.0, -0.5, -0.5))


def test_lamb_error_ratio_output():
    """The factor for the next step's error feedback is c_{t-1} / c_t."""
    out = P.lamb_frozen_step(a(1.0, 1.0), a(0.5, 0.5), a(0.0, 0.0), a(1.0, 1.0), a(1.0, 1.0),
                             [0, 1, 2], c_avg=a(2.0, 3.0), r_prev=a(1.0, 1.0), c_prev=a(1.0, 6.0),
                             lr=1.0, eps=0.0, beta1=0.5, beta2=0.5, thr=0.1, r_min=1.0, r_max=1.0)
    assert np.array_equal(out["c"], a(2.0, 3.0))
    assert np.array_equal(out["err_ratio"], a(0.5, 2.0))


def test_lamb_step_by_hand():
    """One layer by hand, every value dyadic: beta1 = beta2 = 1/2, m = 1,
    m_prev = 0 give g = 2 and v = (0 + 4) / 2 = 2; v_Tw = 16 gives the ratio
    v_Tw / v = 8 (frozen over fresh, 1-bit LAMB page, algorithm), clipped to
    1.1 r_{t-1} = fl(1.1); the step uses the frozen variance and c_{t-1}:
    x = 1 - (1 * 1/2) * (1 / sqrt(16)) = 0.875."""
    one = np.ones(4, dtype=F32)
    out = P.lamb_frozen_step(one, one, 0 * one, 0 * one, 16 * one, [0, 4],
                             c_avg=np.array([2], F32), r_prev=np.array([1], F32),
                             c_prev=np.array([0.5], F32), lr=1.0, eps=0.0, beta1=0.5,
                             beta2=0.5, thr=0.1, r_min=0.5, r_max=4.0)
    assert np.all(out.get("g", 2) == 2) and np.all(out["v"] == 2)
    assert out["R"][0] == 8
    r = F32(F32(1) + F32(0.1))
    assert out["r"][0] == r and out["c"][0] == F32(2 * r)
    assert np.all(out["x"] == F32(0.875))
    assert out["err_ratio"][0] == F32(F32(0.5) / F32(2 * r))


# ------------------------------------------------ rounding sequences, exactly
# The pages fix no rounding order; the step formulas are read as the
# sequences below (one binary32 rounding per operation, true division, the
# square root correctly rounded). Each pin evaluates its sequence on seeded
# values with exact rationals and one explicit rounding per step, and checks
# that the sample separates it from the plausible other orders.

def _fr(a):
    return [Fraction(float(t)) for t in np.asarray(a, dtype=F32).ravel()]


def _sample(seed, n=400, lo=-3.0, hi=3.0):
    rng = np.random.default_rng(seed)
    return (rng.uniform(lo, hi, n) * 2.0 ** rng.integers(-4, 5, n)).astype(F32)


def test_adam_step_rounding_sequence():
    """x - fl(lr fl(m / fl(sqrt(v) + eps))); half of x is 0, so that the
    update's own rounding shows."""
    x, m = _sample(1), _sample(2)
    x[::2] = 0
    v = np.abs(_sample(3)) + F32(1e-3)
    lr, eps = F32(0.37), F32(1e-6)
    den = [rn(Fraction(float(np.sqrt(vi))) + Fraction(float(eps))) for vi in v]
    q = [rn(mi / Fraction(float(d))) for mi, d in zip(_fr(m), den)]
    want = [rn(xi - Fraction(float(rn(Fraction(float(lr)) * Fraction(float(qi))))))
            for xi, qi in zip(_fr(x), q)]
    got = P.adam_frozen_step(x, m, v, lr, eps)
    assert np.array_equal(got, np.array(want, dtype=F32))
    lr_first = [rn(xi - Fraction(float(rn(Fraction(float(rn(Fraction(float(lr)) * mi)))
                                             / Fraction(float(d))))))
                for xi, mi, d in zip(_fr(x), _fr(m), den)]
    recip = [rn(xi - Fraction(float(rn(Fraction(float(lr)) * Fraction(float(
        rn(mi * Fraction(float(rn(1 / Fraction(float(d))))))))))))
        for xi, mi, d in zip(_fr(x), _fr(m), den)]
    assert want != lr_first and want != recip


def test_gradient_reconstruction_rounding_sequence():
    """fl(fl(m - fl(beta1 m_prev)) / fl(1 - beta1)), a true division."""
    m, mp = _sample(4), _sample(5)
    b1 = F32(0.9)
    omb1 = Fraction(float(F32(F32(1) - b1)))
    num = [rn(mi - Fraction(float(rn(Fraction(float(b1)) * pi)))) for mi, pi in zip(_fr(m), _fr(mp))]
    want = [rn(Fraction(float(t)) / omb1) for t in num]
    assert np.array_equal(P.reconstruct_gradient(m, mp, b1), np.array(want, dtype=F32))
    recip = Fraction(float(rn(1 / omb1)))
    assert want != [rn(Fraction(float(t)) * recip) for t in num]


def test_fresh_variance_rounding_sequence():
    """fl(fl(beta2 v) + fl(fl(1 - beta2) fl(g g))): the square first."""
    v = np.abs(_sample(6))
    g = _sample(7)
    b2 = F32(0.999)
    omb2 = Fraction(float(F32(F32(1) - b2)))
    a = [rn(Fraction(float(b2)) * vi) for vi in _fr(v)]
    want = [rn(Fraction(float(ai)) + Fraction(float(rn(omb2 * Fraction(float(rn(gi * gi)))))))
            for ai, gi in zip(a, _fr(g))]
    assert np.array_equal(P.fresh_variance(v, g, b2), np.array(want, dtype=F32))
    other = [rn(Fraction(float(ai)) + Fraction(float(rn(Fraction(float(rn(omb2 * gi))) * gi))))
             for ai, gi in zip(a, _fr(g))]
    assert want != other


def test_lamb_apply_rounding_sequence():
    """x - fl(fl(lr c_l) fl(m / fl(sqrt(v_Tw) + eps))) per layer."""
    x, m = _sample(8), _sample(9)
    x[::2] = 0
    v = np.abs(_sample(10)) + F32(1e-3)
    off = [0, 150, 400]
    c = np.array([0.7, 1.3], dtype=F32)
    lr, eps = F32(1e-3), F32(1e-6)
    den = [rn(Fraction(float(np.sqrt(vi))) + Fraction(float(eps))) for vi in v]
    q = [rn(mi / Fraction(float(d))) for mi, d in zip(_fr(m), den)]
    want, other = [], []
    for l in range(2):
        step = Fraction(float(rn(Fraction(float(lr)) * Fraction(float(c[l])))))
        for j in range(off[l], off[l + 1]):
            xj, qj = Fraction(float(x[j])), Fraction(float(q[j]))
            want.append(rn(xj - Fraction(float(rn(step * qj)))))
            cq = Fraction(float(rn(Fraction(float(c[l])) * qj)))
            other.append(rn(xj - Fraction(float(rn(Fraction(float(lr)) * cq)))))
    assert np.array_equal(P.lamb_apply(x, m, v, off, c, lr, eps), np.array(want, dtype=F32))
    assert want != other
