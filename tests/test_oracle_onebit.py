"""Pins of the oracle's 1-bit worker/server compression (oracle/onebit.py).

Each test fixes the oracle against something it does not compute itself:
exact rational arithmetic on tiny inputs, the error identity and the
telescoping property the 1-bit Adam article states for error compensation
(section 2.1), optimality of the mean-|.| scale for a fixed sign vector, the
clamp bound the article's troubleshooting section asks for (error below
clip_value), and closed forms of the server in degenerate cases.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bits as B
from oracle import cref as R
from oracle import onebit as O
from tests._exactref import frac, rn, ulp

F32 = np.float32


def _draw(rng, shape, scale=1e-3):
    return (rng.standard_normal(shape) * scale).astype(F32)


def _brute_worker(m, e, clip, k):
    """Element-by-element exact evaluation of compensation, scale, sign,
    error, written from the equations with Fractions."""
    n, N = m.shape
    L = N // n
    gc = np.empty_like(m)
    s = np.empty((n, n), dtype=F32)
    e_new = np.empty_like(m)
    for i in range(n):
        for j in range(N):
            km = frac(m[i, j]) if k is None else frac(rn(frac(k[j]) * frac(m[i, j])))
            v = rn(km + frac(e[i, j]))
            if clip > 0:
                v = min(max(v, F32(-clip)), F32(clip))
            gc[i, j] = v
        for c in range(n):
            chunk = gc[i, c * L:(c + 1) * L]
            s[i, c] = rn(sum(abs(frac(v)) for v in chunk) / L)
            for j in range(L):
                v = chunk[j]
                q = frac(s[i, c]) if v >= 0 else -frac(s[i, c])
                e_new[i, c * L + j] = rn(frac(v) - q)
    return gc, s, e_new


IMPLS = {"numpy": O, "cpp": R}  # both oracles against the same brute force


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("clip,use_k", [(0.0, False), (2.5e-3, False), (0.0, True)])
def test_worker_matches_exact_arithmetic(clip, use_k, impl):
    rng = np.random.default_rng(7)
    n, N = 2, 128
    m = _draw(rng, (n, N))
    e = _draw(rng, (n, N), 3e-4)
    # zeros of both signs must encode +1 (sign(0) = +1)
    m[:, :4] = np.array([0.0, -0.0, 0.0, -0.0], dtype=F32)
    e[:, :4] = np.array([0.0, 0.0, -0.0, -0.0], dtype=F32)
    k = (2.0 ** rng.integers(-3, 4, size=N) * rng.uniform(0.5, 1.5, size=N)).astype(F32) if use_k else None
    out = IMPLS[impl].worker_compress(m, e, clip=clip, k=k)
    gc, s, e_new = _brute_worker(m, e, clip, k)
    assert np.array_equal(out["gc"], gc)
    assert np.array_equal(out["s"], s)
    assert np.array_equal(out["e"], e_new)
    assert np.all(out["bits"][:, 0] & np.uint32(0xF) == 0xF)
    want_bits = np.zeros((n, N // 32), dtype=np.uint32)
    for i in range(n):
        for j in range(N):
            if gc[i, j] >= 0:
                want_bits[i, j >> 5] |= np.uint32(1 << (j & 31))
    assert np.array_equal(out["bits"], want_bits)


def test_reset_ignores_error():
    rng = np.random.default_rng(3)
    m = _draw(rng, (2, 128))
    e = _draw(rng, (2, 128))
    a = O.worker_compress(m, e, reset=True)
    b = O.worker_compress(m, np.zeros_like(e))
    for key in ("gc", "s", "e", "bits"):
        assert np.array_equal(a[key], b[key])


def test_server_reset_ignores_error():
    """The error reset (1-bit Adam article, section 4.1) drops the server's
    carried error too: a reset step equals a step from zero error, both for
    one chunk and for the whole buffer."""
    rng = np.random.default_rng(31)
    n, N = 4, 512
    L = N // n
    w = O.worker_compress(_draw(rng, (n, N)), np.zeros((n, N), dtype=F32))
    E = _draw(rng, N)
    zero = np.zeros(N, dtype=F32)
    a = O.server_reduce(w["bits"], w["s"], E, reset=True)
    b = O.server_reduce(w["bits"], w["s"], zero)
    for key in ("g2", "S", "E", "bits"):
        assert np.array_equal(a[key], b[key])
    words = slice(L // 32, 2 * L // 32)
    a = O.server_chunk(w["bits"][:, words], w["s"][:, 1], E[L:2 * L], reset=True)
    b = O.server_chunk(w["bits"][:, words], w["s"][:, 1], zero[L:2 * L])
    for key in ("g2", "S", "E", "bits"):
        assert np.array_equal(a[key], b[key])


def test_error_identity_within_one_rounding():
    """e_t = g'_t - q_t up to the one binary32 rounding of the subtraction."""
    rng = np.random.default_rng(11)
    n, N = 4, 1024
    out = O.worker_compress(_draw(rng, (n, N)), _draw(rng, (n, N), 1e-4))
    L = N // n
    for i in range(n):
        for c in range(n):
            sl = slice(c * L, (c + 1) * L)
            q = B.signed(B.sign_bit(out["gc"][i, sl]), out["s"][i, c])
            for gv, qv, ev in zip(out["gc"][i, sl][::7], q[::7], out["e"][i, sl][::7]):
                assert abs(frac(ev) - (frac(gv) - frac(qv))) <= ulp(ev) / 2


def _run_steps(ms, clip=0.0):
    n, N = ms[0].shape
    e = np.zeros((n, N), dtype=F32)
    hist = []
    for m in ms:
        out = O.worker_compress(m, e, clip=clip)
        hist.append((m, e, out))
        e = out["e"]
    return hist


def test_telescoping_exact_on_dyadic_inputs():
    """sum_t q_t + e_T = sum_t m_t exactly when no operation rounds: inputs
    on a 2^-8 grid in (-1, 1), L = 64, two steps keep every value on a grid
    binary32 represents."""
    rng = np.random.default_rng(5)
    n, N, T = 2, 128, 2
    ms = [(rng.integers(-255, 256, size=(n, N)) / 256.0).astype(F32) for _ in range(T)]
    hist = _run_steps(ms)
    L = N // n
    for i in range(n):
        for j in range(N):
            c = j // L
            total_q = sum(frac(out["s"][i, c]) * (1 if out["gc"][i, j] >= 0 else -1) for _, _, out in hist)
            total_m = sum(frac(m[i, j]) for m in ms)
            assert total_q + frac(hist[-1][2]["e"][i, j]) == total_m


@pytest.mark.parametrize("clip", [0.0, 1.5e-3])
def test_telescoping_bounded_by_roundings(clip):
    """Random inputs: |sum q + e_T - sum m + sum clipped| <= sum of half-ulps
    of every rounded compensation and error."""
    rng = np.random.default_rng(9)
    n, N, T = 2, 256, 6
    ms = [_draw(rng, (n, N)) for _ in range(T)]
    hist = _run_steps(ms, clip=clip)
    L = N // n
    for i in range(n):
        for j in range(0, N, 5):
            c = j // L
            lhs = frac(hist[-1][2]["e"][i, j])
            rhs = Fraction(0)
            bound = Fraction(0)
            for m, e_prev, out in hist:
                g = out["gc"][i, j]
                lhs += frac(out["s"][i, c]) * (1 if g >= 0 else -1)
                rhs += frac(m[i, j])
                raw = F32(m[i, j] + e_prev[i, j])
                rhs -= frac(raw) - frac(g)  # clipped-off amount
                bound += (ulp(raw) + ulp(out["e"][i, j])) / 2
            assert abs(lhs - rhs) <= bound


def test_scale_is_the_l2_optimal_magnitude():
    """For fixed signs, sum (g' - s sgn)^2 is minimal at s = mean|g'|: moving
    s by one binary32 step in either direction must not lower it."""
    rng = np.random.default_rng(21)
    n, N = 4, 4096
    out = O.worker_compress(_draw(rng, (n, N)) * np.float32(3), _draw(rng, (n, N)))
    L = N // n
    for i in range(n):
        for c in range(n):
            g = out["gc"][i, c * L:(c + 1) * L].astype(np.float64)
            s = out["s"][i, c]
            abs_sum = sum(abs(Fraction(float(x))) for x in g)
            sq = sum(Fraction(float(x)) ** 2 for x in g)

            def cost(sv):
                sv = Fraction(float(sv))
                return sq - 2 * sv * abs_sum + L * sv * sv

            here = cost(s)
            assert here <= cost(np.nextafter(s, F32(np.inf), dtype=F32))
            assert here <= cost(np.nextafter(s, F32(0), dtype=F32))
            # and the orthogonality <e, sgn> = sum|g'| - L s vanishes up to rounding of s
            assert abs(float(np.sum(np.abs(g)) - L * float(s))) <= L * float(ulp(s))


def test_clamp_bounds_error():
    rng = np.random.default_rng(4)
    n, N, clip = 4, 1024, 2e-3
    e = np.zeros((n, N), dtype=F32)
    for t in range(5):
        m = _draw(rng, (n, N), 4e-3)
        m[0, :8] = [np.inf, -np.inf, 1e30, -1e30, np.nan, 0, -0.0, 5]
        out = O.worker_compress(m, e, clip=clip)
        assert np.all(np.abs(out["gc"]) <= F32(clip))
        assert np.all(np.abs(out["e"]) <= F32(clip))
        assert out["gc"][0, 4] == F32(-clip)  # NaN clamps to -clip
        e = out["e"]


def test_server_single_worker_is_identity():
    rng = np.random.default_rng(8)
    N = 256
    w = O.worker_compress(_draw(rng, (1, N)), np.zeros((1, N), dtype=F32))
    sv = O.server_reduce(w["bits"], w["s"], np.zeros(N, dtype=F32))
    assert np.array_equal(sv["bits"], w["bits"][0])
    assert sv["S"][0] == w["s"][0, 0]
    assert np.all(sv["E"] == 0)
    assert np.array_equal(O.decompress(sv["bits"], sv["S"]), B.signed(B.sign_bit(w["gc"][0]), w["s"][0, 0]))


def test_server_unanimous_signs():
    rng = np.random.default_rng(12)
    n, N = 4, 1024
    base = O.worker_compress(_draw(rng, (1, N)), np.zeros((1, N), dtype=F32))["bits"][0]
    bits = np.stack([base] * n)
    s = np.abs(_draw(rng, (n, n))) + F32(1e-4)
    sv = O.server_reduce(bits, s, np.zeros(N, dtype=F32))
    assert np.array_equal(sv["bits"], base)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_server_average_exact_sequence(impl):
    """n = 3 (not a power of two): sequential binary32 accumulation in worker
    order, then one rounding of the division."""
    rng = np.random.default_rng(13)
    n, N = 3, 192
    L = N // n
    bits = rng.integers(0, 2**32, size=(n, N // 32), dtype=np.uint64).astype(np.uint32)
    s = np.abs(_draw(rng, (n, n))).astype(F32)
    sv = IMPLS[impl].server_reduce(bits, s, np.zeros(N, dtype=F32))
    for c in range(n):
        for j in range(0, L, 3):
            J = c * L + j
            acc = F32(0.0)
            for i in range(n):
                bit = (int(bits[i, J >> 5]) >> (J & 31)) & 1
                acc = rn(frac(acc) + (frac(s[i, c]) if bit else -frac(s[i, c])))
            assert sv["avg"][J] == rn(frac(acc) / n)


def test_two_level_momentum_identity():
    """1-bit LAMB analysis paragraph with a unit step ratio: the transmitted
    global momentum equals the workers' average momentum plus the previous
    combined error minus the new one, delta = E + mean_i e_i.  Dyadic inputs,
    n = 2, two steps: every operation is exact, so the identity is exact."""
    rng = np.random.default_rng(17)
    n, N, T = 2, 128, 2
    e = np.zeros((n, N), dtype=F32)
    E = np.zeros(N, dtype=F32)
    delta_prev = [Fraction(0)] * N
    for t in range(T):
        m = (rng.integers(-255, 256, size=(n, N)) / 256.0).astype(F32)
        w = O.worker_compress(m, e)
        sv = O.server_reduce(w["bits"], w["s"], E)
        mbar = O.decompress(sv["bits"], sv["S"])
        for j in range(N):
            delta = frac(sv["E"][j]) + (frac(w["e"][0, j]) + frac(w["e"][1, j])) / 2
            avg_m = (frac(m[0, j]) + frac(m[1, j])) / 2
            assert frac(mbar[j]) == avg_m + delta_prev[j] - delta
            delta_prev[j] = delta
        e, E = w["e"], sv["E"]


def test_layer_scale_power_of_two_is_transparent():
    """Uniform k = 2^p: scaling before compression and dividing after gives
    exactly the unscaled path (positive homogeneity of the method)."""
    rng = np.random.default_rng(19)
    n, N = 4, 1024
    m = _draw(rng, (n, N))
    k = np.full(N, F32(8.0))
    a = O.worker_compress(m, np.zeros_like(m), k=k)
    b = O.worker_compress(m, np.zeros_like(m))
    assert np.array_equal(a["bits"], b["bits"])
    assert np.array_equal(a["s"], b["s"] * F32(8.0))
    sa = O.server_reduce(a["bits"], a["s"], np.zeros(N, dtype=F32))
    sb = O.server_reduce(b["bits"], b["s"], np.zeros(N, dtype=F32))
    assert np.array_equal(O.decompress(sa["bits"], sa["S"], k=k), O.decompress(sb["bits"], sb["S"]))


def test_layer_scale_segments():
    buf = np.arange(1, 11, dtype=F32)
    off = [0, 3, 4, 10]
    k = np.array([2, 0.5, 4], dtype=F32)
    assert list(O.layer_scale(buf, off, k, False)) == [2, 4, 6, 2, 20, 24, 28, 32, 36, 40]
    assert list(O.layer_scale(buf, off, k, True)) == [0.5, 1, 1.5, 8, 1.25, 1.5, 1.75, 2, 2.25, 2.5]


def test_per_element_k_layout():
    """Layer l's coefficient on elements seg_off[l] .. seg_off[l+1]-1, empty
    layers taking none; it agrees with the segment-wise layer scale."""
    off = [0, 2, 2, 5, 6]
    k = np.array([3, 7, 5, 9], dtype=F32)
    assert list(O.per_element_k(off, k)) == [3, 3, 5, 5, 5, 9]
    buf = np.arange(1, 7, dtype=F32)
    assert np.array_equal(O.layer_scale(buf, off, k, False), buf * O.per_element_k(off, k))


def test_local_momentum_closed_forms():
    """beta1 = 0 gives the gradient; beta1 = 1/2 the exact midpoint on dyadic
    inputs; beta1 = 0.9 matches the recursion within two roundings."""
    rng = np.random.default_rng(23)
    g = (rng.integers(-512, 512, size=(3, 256)) / 1024).astype(F32)
    mb = (rng.integers(-512, 512, size=256) / 1024).astype(F32)
    assert np.array_equal(O.local_momentum(g, mb, 0.0), g)
    half = O.local_momentum(g, mb, 0.5)
    for i in range(3):
        for j in range(0, 256, 7):
            assert frac(half[i, j]) == (frac(g[i, j]) + frac(mb[j])) / 2
    g9 = _draw(rng, (2, 512))
    mb9 = _draw(rng, (512,))
    m9 = O.local_momentum(g9, mb9, 0.9)
    b1 = Fraction(float(F32(0.9)))
    for i in range(2):
        for j in range(0, 512, 5):
            exact = b1 * frac(mb9[j]) + (1 - b1) * frac(g9[i, j])
            assert abs(frac(m9[i, j]) - exact) <= ulp(m9[i, j]) + ulp(F32(0.9) * mb9[j]) / 2 + \
                ulp(F32(F32(1) - F32(0.9)) * g9[i, j]) / 2 + abs(frac(g9[i, j])) * (
                    abs(Fraction(float(F32(1) - F32(0.9))) - (1 - b1)))


def test_unit_scale_is_the_plain_sign():
    """The 1-bit Adam article's q = sign(g'): every scale is 1 and the error
    is g' -+ 1 (exact on dyadic inputs); the server's scales are 1 too."""
    rng = np.random.default_rng(29)
    n, N = 4, 512
    m = (rng.integers(-255, 256, size=(n, N)) / 256.0).astype(F32)
    w = O.worker_compress(m, np.zeros_like(m), unit_scale=True)
    assert np.all(w["s"] == 1)
    for i in range(n):
        for j in range(0, N, 3):
            q = 1 if m[i, j] >= 0 else -1
            assert frac(w["e"][i, j]) == frac(m[i, j]) - q
    sv = O.server_reduce(w["bits"], w["s"], np.zeros(N, dtype=F32), unit_scale=True)
    assert np.all(sv["S"] == 1)
    # the average of +-1 over 4 workers takes values in {-1, -1/2, 0, 1/2, 1}
    assert set(np.unique(sv["avg"]).tolist()) <= {-1.0, -0.5, 0.0, 0.5, 1.0}


def test_error_ratio_one_is_transparent():
    rng = np.random.default_rng(31)
    n, N = 4, 1024
    m = _draw(rng, (n, N))
    e = _draw(rng, (n, N), 3e-4)
    a = O.worker_compress(m, e, err_ratio=np.ones(N, dtype=F32))
    b = O.worker_compress(m, e)
    for key in ("gc", "s", "e", "bits"):
        assert np.array_equal(a[key], b[key])


def test_two_level_identity_with_step_ratio():
    """1-bit LAMB analysis paragraph: with the carried errors scaled by the
    step ratio rho at both levels, m_bar_t = mean_i m_t^(i) + rho
    delta_{t-1} - delta_t.  Inputs on a 2^-4 grid in (-1/4, 1/4), chunks of
    64 and two steps keep every operation exact (each chunk mean adds six
    binary digits), so the identity holds exactly for rho = 1/2 and 2."""
    rng = np.random.default_rng(37)
    n, N = 2, 128
    for rho in (0.5, 2.0):
        e = np.zeros((n, N), dtype=F32)
        E = np.zeros(N, dtype=F32)
        delta_prev = [Fraction(0)] * N
        for t in range(2):
            m = (rng.integers(-3, 4, size=(n, N)) / 16.0).astype(F32)
            ratio = np.full(N, F32(rho))
            w = O.worker_compress(m, e, err_ratio=ratio)
            sv = O.server_reduce(w["bits"], w["s"], E, err_ratio=ratio)
            mbar = O.decompress(sv["bits"], sv["S"])
            for j in range(N):
                delta = frac(sv["E"][j]) + (frac(w["e"][0, j]) + frac(w["e"][1, j])) / 2
                avg_m = (frac(m[0, j]) + frac(m[1, j])) / 2
                assert frac(mbar[j]) == avg_m + Fraction(rho) * delta_prev[j] - delta
                delta_prev[j] = delta
            e, E = w["e"], sv["E"]


def test_layer_coefficient_scales_the_momentum_not_the_error():
    """g' = k_l m + e: the 1-bit LAMB page (layer-scaling paragraph) scales
    each layer's local momentum before the compressed exchange, and the
    carried error, formed on scaled values, is added as it is. With m = 1,
    e = 1/2 and k = 2 on the first layer, 4 on the second, g' is 2.5 and
    4.5, the chunk mean 3.5 and the new error -1 and +1."""
    m = np.ones((1, 64), dtype=F32)
    e = np.full((1, 64), 0.5, dtype=F32)
    k = np.repeat(np.array([2, 4], dtype=F32), 32)
    out = O.worker_compress(m, e, k=k)
    assert np.all(out["gc"][0, :32] == 2.5) and np.all(out["gc"][0, 32:] == 4.5)
    assert out["s"][0, 0] == 3.5
    assert np.all(out["e"][0, :32] == -1) and np.all(out["e"][0, 32:] == 1)
    assert np.all(out["bits"] == 0xFFFFFFFF)


def test_division_by_the_layer_coefficient_is_a_true_division():
    """x / k_l is one correctly rounded division, in the layer scale and in
    the decompression (1-bit LAMB page, layer-scaling paragraph: divide by
    the same coefficient afterwards), never x * fl(1 / k_l); the sample's
    coefficients are not powers of two, so the two differ on some elements."""
    rng = np.random.default_rng(12)
    N = 512
    off = [0, 100, 300, 512]
    k = np.array([3.0, 0.7, 10.3], dtype=F32)
    x = (rng.uniform(-2, 2, N)).astype(F32)
    kk = O.per_element_k(off, k)
    want = np.array([rn(frac(a) / frac(b)) for a, b in zip(x, kk)], dtype=F32)
    recip = np.array([rn(frac(a) * frac(rn(1 / frac(b)))) for a, b in zip(x, kk)], dtype=F32)
    assert not np.array_equal(want, recip)
    assert np.array_equal(O.layer_scale(x, off, k, divide=True), want)
    # decompression: +-S[c] / k_l with two chunks
    S = np.array([0.3, 1.7], dtype=F32)
    words = rng.integers(0, 2 ** 32, N // 32, dtype=np.uint64).astype(np.uint32)
    b = B.unpack(words)
    sc = np.repeat(S, N // 2)
    dec = np.array([rn(frac(s if bit else -s) / frac(kv)) for bit, s, kv in zip(b, sc, kk)],
                   dtype=F32)
    assert np.array_equal(O.decompress(words, S, kk), dec)
