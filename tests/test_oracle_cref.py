"""The C++ oracle (oracle/cpp) against the numpy oracle and against the pins
that do not depend on either.

Two implementations written apart from the same passages must agree bit for
bit on every output, on seeded inputs that reach each branch: resets, the
clamp (with NaN and infinities), layer coefficients, the unit scale, the
step-ratio factor, ties of the mean, subnormals, every INT8 block size and
both roundings. The independent pins (brute force with fractions for the
exact mean, numpy's own float64 -> float32 rounding for midpoints, closed
forms of the server) run on the C++ oracle directly.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import cref as R
from oracle import int8 as I
from oracle import onebit as O
from oracle import optim as P
from oracle import philox as PH
from oracle.exact import mean_abs_f32
from tests.test_oracle_int8 import _tie_block

F32 = np.float32


def _eq(got, want, name):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.dtype == np.float32:
        g, w = got.view(np.uint32), want.astype(F32).view(np.uint32)
        nan_g, nan_w = np.isnan(got), np.isnan(want)
        assert np.array_equal(nan_g, nan_w), f"{name}: NaN positions differ"
        ok = (g == w) | nan_g
    else:
        ok = got == want
    assert ok.all(), f"{name}: {int((~ok).sum())} of {ok.size} differ"


def _momentum(rng, n, N, spread=3.0):
    sig = 10.0 ** rng.uniform(-5, -5 + spread, size=-(-N // 64))
    return (rng.standard_normal((n, N)) * np.repeat(sig, 64)[None, :N]).astype(F32)


# ------------------------------------------------------------------ exact mean

@pytest.mark.parametrize("L", [1, 2, 3, 64, 257, 4096])
def test_mean_matches_fractions(L):
    rng = np.random.default_rng(100 + L)
    trials = 30 if L <= 257 else 4
    for trial in range(trials):
        x = (rng.standard_normal(L) * 10.0 ** rng.uniform(-40, 35, size=L)).astype(F32)
        if trial % 3 == 0:
            x[: L // 2] = F32(1e-45) * rng.integers(0, 50, size=L // 2)  # subnormals
        exact = sum((abs(Fraction(float(v))) for v in x), Fraction(0)) / L
        got = R.mean_abs_f32(x)
        # nearest binary32 to the exact mean: no binary32 value is closer
        lo, hi = np.nextafter(got, F32(0)), np.nextafter(got, F32(np.inf))
        d = abs(Fraction(float(got)) - exact)
        assert d <= abs(Fraction(float(lo)) - exact)
        if np.isfinite(hi):
            assert d <= abs(Fraction(float(hi)) - exact)
        assert got == mean_abs_f32(x)


def test_mean_ties_round_to_even():
    """Two neighbours a < b average to their exact midpoint: the tie goes to
    the one with an even significand (numpy's float64 -> float32 cast, one
    correct rounding, gives the same)."""
    rng = np.random.default_rng(7)
    a = rng.integers(1, 0x7F000000, size=4000, dtype=np.int64).astype(np.uint32)
    lo, hi = a.view(F32), (a + 1).view(F32)
    for x, y in zip(lo, hi):
        got = R.mean_abs_f32(np.array([x, y], dtype=F32))
        mid = (float(x) + float(y)) / 2  # exact in float64
        assert got == F32(mid)
        even = x if (x.view(np.uint32) & 1) == 0 else y
        assert got == even


def test_mean_special_values():
    assert np.isnan(R.mean_abs_f32(np.array([1.0, np.nan, np.inf], dtype=F32)))
    assert R.mean_abs_f32(np.array([1.0, -np.inf], dtype=F32)) == np.inf
    assert R.mean_abs_f32(np.zeros(96, dtype=F32)) == 0.0
    assert R.mean_abs_f32(np.array([-0.0, 0.0], dtype=F32)) == 0.0
    big = np.full(1000, np.finfo(F32).max, dtype=F32)
    assert R.mean_abs_f32(big) == np.finfo(F32).max  # the sum overflows binary32, the mean not
    tiny = np.array([2.0 ** -149, 0.0], dtype=F32)  # mean 2^-150: a tie with 0, even is 0
    assert R.mean_abs_f32(tiny) == 0.0
    tiny3 = np.array([2.0 ** -149, 2.0 ** -148], dtype=F32)  # 1.5 units: tie, even is 2 units
    assert R.mean_abs_f32(tiny3) == F32(2.0 ** -148)


def test_mean_matches_numpy_oracle_random():
    rng = np.random.default_rng(11)
    for trial in range(200):
        L = int(rng.integers(1, 3000))
        x = (rng.standard_normal(L) * 10.0 ** rng.uniform(-45, 38, size=L)).astype(F32)
        assert R.mean_abs_f32(x).view(np.uint32) == mean_abs_f32(x).view(np.uint32), trial


# --------------------------------------------------------------- worker, server

CASES = [
    dict(n=1, N=64 * 7, clip=0.0),
    dict(n=4, N=4 * 3136, clip=0.0),
    dict(n=3, N=3 * 64 * 33, clip=2e-3),
    dict(n=8, N=8 * 1024, clip=0.0, k=True),
    dict(n=5, N=5 * 64 * 9, clip=0.0, unit=True),
    dict(n=6, N=6 * 640, clip=1e-3, ratio=True),
    dict(n=16, N=16 * 128, clip=0.0, k=True, ratio=True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_compressed_steps_match_numpy_oracle(case):
    """Four steps of worker compress, server reduce and decompression, the
    first a reset, fed back into themselves on both sides."""
    cfg = CASES[case]
    n, N = cfg["n"], cfg["N"]
    rng = np.random.default_rng(case)
    k = (10.0 ** rng.uniform(-1, 1, size=N)).astype(F32) if cfg.get("k") else None
    unit = cfg.get("unit", False)
    e_np = e_c = np.zeros((n, N), dtype=F32)
    E_np = E_c = np.zeros(N, dtype=F32)
    for t in range(4):
        m = _momentum(rng, n, N)
        if t == 2:
            m[0, :5] = [np.nan, np.inf, -np.inf, 0.0, -0.0]  # clamp and sign conventions
        ratio = (1.0 + 0.1 * rng.standard_normal(N)).astype(F32) if cfg.get("ratio") else None
        reset = t == 0
        w_np = O.worker_compress(m, e_np, clip=cfg["clip"], reset=reset, k=k, unit_scale=unit,
                                 err_ratio=ratio)
        w_c = R.worker_compress(m, e_c, clip=cfg["clip"], reset=reset, k=k, unit_scale=unit,
                                err_ratio=ratio, threads=2)
        for key in ("gc", "bits", "s", "e"):
            _eq(w_c[key], w_np[key], f"case {case} t={t} worker {key}")
        s_np = O.server_reduce(w_np["bits"], w_np["s"], E_np, reset=reset, unit_scale=unit,
                               err_ratio=ratio)
        s_c = R.server_reduce(w_c["bits"], w_c["s"], E_c, reset=reset, unit_scale=unit,
                              err_ratio=ratio, threads=3)
        for key in ("avg", "g2", "bits", "S", "E"):
            _eq(s_c[key], s_np[key], f"case {case} t={t} server {key}")
        _eq(R.decompress(s_c["bits"], s_c["S"], k), O.decompress(s_np["bits"], s_np["S"], k),
            f"case {case} t={t} decompressed")
        e_np, e_c, E_np, E_c = w_np["e"], w_c["e"], s_np["E"], s_c["E"]


def test_worker_without_compensated_values():
    rng = np.random.default_rng(3)
    m = _momentum(rng, 4, 4 * 256)
    a = R.worker_compress(m, None, reset=True)
    b = R.worker_compress(m, None, reset=True, keep_gc=False, threads=4)
    assert "gc" not in b
    for key in ("bits", "s", "e"):
        _eq(b[key], a[key], key)


def test_server_closed_forms():
    """n = 1: the server sees +-s, so with a zero error its output is the
    worker's own scaled sign (scale s, same bits). Unanimous workers with
    scales s_i average to sum(s_i)/n on every element."""
    rng = np.random.default_rng(5)
    m = _momentum(rng, 1, 64 * 40)
    w = R.worker_compress(m, None, reset=True)
    s = R.server_reduce(w["bits"], w["s"], None, reset=True)
    assert np.array_equal(s["bits"], w["bits"][0])
    assert s["S"][0] == w["s"][0, 0]
    assert not s["E"].any()
    n, N = 4, 4 * 64
    bits = np.full((n, N // 32), 0xFFFFFFFF, dtype=np.uint32)
    sc = np.array([[1.0, 2.0, 4.0, 8.0]] * n, dtype=F32).T.copy()  # s[i][c] = 2^i
    out = R.server_reduce(bits, sc, None, reset=True)
    assert np.all(out["avg"] == F32(15.0 / 4))
    assert np.all(out["S"] == F32(15.0 / 4))


def test_local_momentum_matches_numpy_oracle():
    rng = np.random.default_rng(9)
    g = _momentum(rng, 3, 3 * 512)
    mb = _momentum(rng, 1, 3 * 512)[0]
    _eq(R.local_momentum(g, mb, 0.9), O.local_momentum(g, mb, 0.9), "local momentum")


# ----------------------------------------------------------------------- steps

def test_adam_step_matches_numpy_oracle_and_closed_form():
    rng = np.random.default_rng(12)
    N = 4096
    x = rng.standard_normal(N).astype(F32)
    m = _momentum(rng, 1, N)[0]
    v = (np.abs(rng.standard_normal(N)) * 1e-6 + 1e-8).astype(F32)
    v[:4] = [0.0, np.inf, 1.0, 4.0]
    _eq(R.adam_frozen_step(x, m, v, 6e-5, 1e-6), P.adam_frozen_step(x, m, v, 6e-5, 1e-6), "adam")
    # v = 4, eps = 0, m = 2, lr = 1/2: x - 1/2 * (2 / 2) = x - 1/2, exact
    out = R.adam_frozen_step(np.array([3.0] * 4, F32), np.array([2.0] * 4, F32),
                             np.array([4.0] * 4, F32), 0.5, 0.0)
    assert np.all(out == F32(2.5))


@pytest.mark.parametrize("use_c_t", [False, True])
def test_lamb_step_matches_numpy_oracle(use_c_t):
    rng = np.random.default_rng(20 + use_c_t)
    sizes = [64, 1, 300, 1024, 4, 0, 77, 2048]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N = int(off[-1])
    L = len(sizes)
    x = rng.standard_normal(N).astype(F32)
    m_prev = _momentum(rng, 1, N)[0]
    m = (0.9 * m_prev + 0.1 * _momentum(rng, 1, N)[0]).astype(F32)
    v_tw = (np.abs(rng.standard_normal(N)) * 1e-6 + 1e-9).astype(F32)
    v_f = (v_tw * (1 + 0.3 * rng.standard_normal(N))).astype(F32)
    # a layer of ratio 0/0 (no valid ratio: r stays), one with signed zeros
    lay1 = slice(off[1], off[2])
    m[lay1], m_prev[lay1], v_f[lay1], v_tw[lay1] = 0, 0, 0, 0
    lay4 = slice(off[4], off[5])
    v_tw[lay4] = [-0.0, -0.0, 0.0, -0.0]  # the first valid ratio is -0, a later one +0
    c_avg = (10.0 ** rng.uniform(-1, 1, size=L)).astype(F32)
    r_prev = (1 + 0.2 * rng.standard_normal(L)).astype(F32)
    c_prev = (c_avg * r_prev).astype(F32)
    args = (x, m, m_prev, v_f, v_tw, off, c_avg, r_prev, c_prev, 1e-3, 1e-6, 0.9, 0.999,
            0.1, 0.5, 4.0, use_c_t)
    got, want = R.lamb_frozen_step(*args), P.lamb_frozen_step(*args)
    for key in ("x", "v", "R", "r", "c", "err_ratio"):
        _eq(got[key], want[key], f"lamb {key}")
    assert np.isnan(got["R"][1]) and got["r"][1] == r_prev[1]
    assert got["R"][4] == 0.0 and not np.signbit(got["R"][4])
    lo = (F32(0.9) * r_prev).astype(F32)
    hi = (F32(1.1) * r_prev).astype(F32)
    assert np.all(got["r"] >= np.maximum(np.minimum(lo, 4.0), 0.5))
    assert np.all(got["r"] <= np.minimum(np.maximum(hi, 0.5), 4.0))


def test_lamb_gradient_round_trip():
    """With v_f = 0 and beta2 = 0 the fresh variance is g^2 of the rebuilt
    gradient; m built from m_prev and a dyadic g by exact operations gives
    back that g exactly (beta1 = 1/2)."""
    rng = np.random.default_rng(30)
    N = 256
    g = (rng.integers(-64, 64, size=N) / 64).astype(F32)
    m_prev = (rng.integers(-64, 64, size=N) / 64).astype(F32)
    m = (F32(0.5) * m_prev + F32(0.5) * g).astype(F32)
    off = np.array([0, N], dtype=np.int64)
    one = np.ones(1, F32)
    out = R.lamb_frozen_step(np.zeros(N, F32), m, m_prev, np.zeros(N, F32), np.ones(N, F32), off,
                             one, one, one, 0.0, 0.0, 0.5, 0.0, 0.1, 0.5, 4.0)
    assert np.array_equal(out["v"], (g * g).astype(F32))


# ------------------------------------------------------------------ INT8, Philox

def test_philox_matches_numpy_oracle():
    rng = np.random.default_rng(40)
    ctr = rng.integers(0, 2**32, size=(300, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(300, 2), dtype=np.uint64).astype(np.uint32)
    got = np.stack([R.philox4x32_10(ctr[i], key[i])[0] for i in range(300)])
    assert np.array_equal(got, PH.philox4x32_10(ctr, key))
    J0 = (1 << 33) + 5
    assert np.array_equal(R.uniforms(J0, 40, 0xDEADBEEF12345, 7), PH.uniforms(J0, 40, 0xDEADBEEF12345, 7))


@pytest.mark.parametrize("block", [0, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("rounding", ["stochastic", "nearest"])
def test_int8_matches_numpy_oracle(block, rounding):
    rng = np.random.default_rng(block + (rounding == "nearest"))
    N = 4096
    g = rng.laplace(0, 1e-3, size=N).astype(F32)
    out_idx = rng.choice(N, size=4, replace=False)
    g[out_idx] *= 100  # outliers
    e = (rng.standard_normal(N) * 1e-5).astype(F32)
    g[64:128] = 0.0
    e[64:128] = 0.0  # an all-zero block of 64: scale 0, code 0
    g[300], g[301] = np.nan, -0.0
    J0 = 12345 * 4
    for err in (None, e):
        got = R.int8_sr(g, err, 77, 3, block=block, J0=J0, rounding=rounding)
        want = I.int8_sr(g, err, 77, 3, block=block, J0=J0, rounding=rounding)
        for key in ("codes", "scales", "deq", "e"):
            _eq(got[key], want[key], f"int8 block={block} {rounding} {key}")
        assert np.all(np.abs(got["codes"].astype(int)) <= 127)


def test_int8_fraction_equal_to_its_uniform_rounds_down():
    """The pin of the numpy oracle's comparison u < p, on the C++ oracle: a
    fraction equal to its own uniform rounds down, one 2^-24 above it up."""
    for above, code in ((False, 0), (True, 1)):
        g, idx = _tie_block(5, 2, above=above)
        out = R.int8_sr(g, None, 5, 2)
        assert out["scales"][0] == 1
        assert np.all(out["codes"][idx] == code)


def test_int8_threaded_slices_equal_one_call():
    rng = np.random.default_rng(50)
    g = rng.laplace(0, 1e-3, size=256 * 37).astype(F32)
    e = (rng.standard_normal(g.size) * 1e-5).astype(F32)
    one = R.int8_sr(g, e, 9, 4, block=256, J0=1 << 33)
    for threads in (2, 5, 37, 64):
        many = R.int8_sr(g, e, 9, 4, block=256, J0=1 << 33, threads=threads)
        for key in ("codes", "scales", "deq", "e"):
            _eq(many[key], one[key], f"int8 threads={threads} {key}")


def test_row_chunks_threaded_equal_one_call():
    """The chunk-parallel worker row, slice-parallel decompression and Adam
    step give the same bytes as one call (chunks and elements are
    independent), with clamp, k, the step-ratio error and a reset."""
    rng = np.random.default_rng(51)
    n, L = 5, 64 * 7
    N = n * L
    m = (rng.standard_normal(N) * 1e-3).astype(F32)
    e = (rng.standard_normal(N) * 1e-4).astype(F32)
    k = np.exp(rng.uniform(-3, 3, N)).astype(F32)
    ratio = np.exp(rng.uniform(-1, 1, N)).astype(F32)
    for kw in (dict(), dict(clip=2e-3, k=k), dict(err_ratio=ratio), dict(reset=True),
               dict(unit_scale=True)):
        one = R.worker_compress_row(m, e.copy(), n, **kw)
        gc, eo = np.empty(N, dtype=F32), np.empty(N, dtype=F32)
        many = R.worker_compress_row(m, e.copy(), n, threads=3, gc_out=gc, e_out=eo, **kw)
        for key in ("gc", "bits", "s", "e"):
            _eq(many[key], one[key], f"row threads {kw.keys()} {key}")
        assert many["gc"] is gc and many["e"] is eo
    sb = rng.integers(0, 1 << 32, N // 32, dtype=np.uint32)
    S = rng.uniform(0, 1e-3, n).astype(F32)
    for kk in (None, k):
        _eq(R.decompress(sb, S, kk, threads=4), R.decompress(sb, S, kk), "decompress threads")
    wb = rng.integers(0, 1 << 32, (n, N // 32), dtype=np.uint32)
    ws = rng.uniform(0, 1e-3, (n, n)).astype(F32)
    E = (rng.standard_normal(N) * 1e-4).astype(F32)
    for reset in (False, True):
        full = R.server_reduce(wb, ws, E, reset=reset)
        for c in (0, 2, n - 1):
            one = R.server_reduce_chunk(wb, ws, E[:(c + 1) * L], c, reset=reset)
            sl = slice(c * L, (c + 1) * L)
            for key in ("avg", "g2", "E"):
                _eq(one[key][sl], full[key][sl], f"server chunk {c} {key}")
            _eq(one["bits"][c * L // 32:], full["bits"][c * L // 32:(c + 1) * L // 32],
                f"server chunk {c} words")
            assert one["S"][c] == full["S"][c]
    N2 = 4096 * 3 + 64  # long enough for three slices
    x = (rng.standard_normal(N2) * 0.02).astype(F32)
    v = (np.abs(rng.standard_normal(N2)) * 1e-6 + 1e-8).astype(F32)
    mb = (rng.standard_normal(N2) * 1e-3).astype(F32)
    _eq(R.adam_frozen_step(x, mb, v, 6e-5, 1e-6, threads=3),
        R.adam_frozen_step(x, mb, v, 6e-5, 1e-6), "adam threads")


# ------------------------------------- pins the pages fix, run on the C++ oracle

def _frac(x):
    return Fraction(float(x))


def test_telescoping_exact_on_dyadic_inputs_both_levels():
    """With inputs on a 2^-8 grid no operation rounds, so what was sent plus
    what is still owed equals what came in, exactly: per worker element
    sum_t q_t + e_T = sum_t m_t, and at the server sum_t Q_t + E_T =
    sum_t avg_t (1-bit Adam article, section 2.1, error compensation)."""
    rng = np.random.default_rng(60)
    n, N, T = 2, 128, 2  # each step's mean over 64 adds 6 bits: two steps stay exact
    L = N // n
    e = E = None
    sum_m = np.zeros((n, N), dtype=object)
    sum_q = np.zeros((n, N), dtype=object)
    sum_avg = np.zeros(N, dtype=object)
    sum_Q = np.zeros(N, dtype=object)
    sum_m[:] = Fraction(0)
    sum_q[:] = Fraction(0)
    sum_avg[:] = Fraction(0)
    sum_Q[:] = Fraction(0)
    for t in range(T):
        m = (rng.integers(-255, 256, size=(n, N)) / 256.0).astype(F32)
        w = R.worker_compress(m, e, reset=t == 0)
        sv = R.server_reduce(w["bits"], w["s"], E, reset=t == 0)
        for i in range(n):
            for j in range(N):
                sign = 1 if w["gc"][i, j] >= 0 else -1
                sum_q[i, j] += sign * _frac(w["s"][i, j // L])
                sum_m[i, j] += _frac(m[i, j])
        for j in range(N):
            sign = 1 if sv["g2"][j] >= 0 else -1
            sum_Q[j] += sign * _frac(sv["S"][j // L])
            sum_avg[j] += _frac(sv["avg"][j])
        e, E = w["e"], sv["E"]
    for i in range(n):
        for j in range(N):
            assert sum_q[i, j] + _frac(e[i, j]) == sum_m[i, j], (i, j)
    for j in range(N):
        assert sum_Q[j] + _frac(E[j]) == sum_avg[j], j


def test_sign_words_match_numpy_packbits():
    """Bit j of a row is (g'_j >= 0), least significant bit first: the same
    bytes as numpy's packbits with little bit order, read as little-endian
    32-bit words. The decompression inverts it: its sign is the bit."""
    rng = np.random.default_rng(61)
    n, N = 3, 3 * 64 * 5
    m = _momentum(rng, n, N)
    m[0, :4] = [0.0, -0.0, np.nan, -1e-30]
    w = R.worker_compress(m, None, reset=True)
    for i in range(n):
        want = np.packbits(w["gc"][i] >= 0, bitorder="little").view("<u4")
        assert np.array_equal(w["bits"][i], want)
    S = np.ones(1, dtype=F32)
    dec = R.decompress(w["bits"][0], S)
    assert np.array_equal(dec > 0, w["gc"][0] >= 0)


def test_error_is_the_nearest_binary32_to_g_minus_q():
    """e = g' - q rounded once: no binary32 value lies closer to the exact
    difference (checked with fractions on a sample)."""
    rng = np.random.default_rng(62)
    n, N = 2, 2 * 640
    m = _momentum(rng, n, N, spread=6.0)
    w = R.worker_compress(m, None, reset=True)
    L = N // n
    for i in range(n):
        for j in range(0, N, 7):
            s = _frac(w["s"][i, j // L])
            g = _frac(w["gc"][i, j])
            exact = g - (s if w["gc"][i, j] >= 0 else -s)
            got = w["e"][i, j]
            d = abs(_frac(got) - exact)
            for nb in (np.nextafter(got, F32(-np.inf)), np.nextafter(got, F32(np.inf))):
                assert d <= abs(_frac(nb) - exact)


# ----------------------------------------------------------------------- warmup

from oracle import warmup as W  # noqa: E402


def _layers(rng, sizes):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return off, int(off[-1])


def test_warmup_steps_match_numpy_oracle():
    """Four free-running warmup steps of Adam and of LAMB (layers of 1 to
    3000 elements, an empty layer, an all-zero layer, values spanning 1e-30
    to 1e3), and k_l at the end."""
    rng = np.random.default_rng(70)
    off, N = _layers(rng, [64, 1, 3000, 0, 257, 128, 4, 1024])
    hp = dict(lr=1e-3, eps=1e-6, beta1=0.9, beta2=0.999)
    x = (rng.standard_normal(N) * 10.0 ** rng.uniform(-30, 3, size=N)).astype(F32)
    m = np.zeros(N, F32)
    v = np.zeros(N, F32)
    xa, ma, va = x.copy(), m.copy(), v.copy()
    c_np = c_c = None
    for t in range(4):
        g = (rng.standard_normal(N) * 1e-3).astype(F32)
        g[off[5]:off[6]] = 0.0  # the layer's u stays 0: c = 1
        a_np = W.adam_warmup_step(xa, ma, va, g, **hp)
        a_c = R.adam_warmup_step(xa, ma, va, g, **hp)
        for key in ("x", "m", "v"):
            _eq(a_c[key], a_np[key], f"adam warmup t={t} {key}")
        xa, ma, va = a_np["x"], a_np["m"], a_np["v"]
        l_np = W.lamb_warmup_step(x, m, v, g, off, c_avg=c_np, beta_c=0.9, **hp)
        l_c = R.lamb_warmup_step(x, m, v, g, off, c_avg=c_c, beta_c=0.9, **hp)
        for key in ("x", "m", "v", "c", "c_avg"):
            _eq(l_c[key], l_np[key], f"lamb warmup t={t} {key}")
        x, m, v, c_np, c_c = l_np["x"], l_np["m"], l_np["v"], l_np["c_avg"], l_c["c_avg"]
    assert l_c["c"][3] == 1 and l_c["c"][5] == 1
    _eq(R.momentum_scale(m, off), W.momentum_scale(m, off), "k_l")


def test_momentum_scale_pins():
    """Layers of constant magnitude 1, 4 and 2 (RMS 1, 4, 2, mean 7/3) give
    k = (7/3, 7/12, 7/6), each rounded once; an empty and an all-zero layer
    give 1. The RMS uses an exact sum: the squares of 2^20 copies of 2^-75
    vanish in binary32 (2^-150), but their RMS is 2^-75, so the layer counts:
    k = (0.5 / 2^-75, 0.5 / 1) with mean (2^-75 + 1) / 2 = 0.5 in binary64."""
    m = np.array([1, -1, 4, 4, -4, 2, 0, 0], dtype=F32)
    off = np.array([0, 2, 5, 6, 6, 8], dtype=np.int64)
    k = R.momentum_scale(m, off)
    assert np.array_equal(k, np.array([7 / 3, 7 / 12, 7 / 6, 1, 1], dtype=F32))
    tiny = np.full(1 << 20, 2.0 ** -75, dtype=F32)
    m2 = np.concatenate([tiny, np.array([1.0], dtype=F32)])
    k2 = R.momentum_scale(m2, np.array([0, 1 << 20, (1 << 20) + 1], dtype=np.int64))
    assert np.array_equal(k2, np.array([2.0 ** 74, 0.5], dtype=F32))
    assert np.array_equal(W.momentum_scale(m2, [0, 1 << 20, (1 << 20) + 1]), k2)


def test_trust_ratio_pins():
    """One layer x = (3, 4), and m, v chosen so that u = (1, 0) exactly: the
    coefficient is ||x|| / ||u|| = 5, and x moves by lr * 5 * u. A layer
    whose x is 0 keeps c = 1."""
    x = np.array([3, 4, 0, 0], dtype=F32)
    m0 = np.array([1, 0, 1, 1], dtype=F32)
    v0 = np.ones(4, dtype=F32)
    g = np.array([1, 0, 1, 1], dtype=F32)
    off = np.array([0, 2, 4], dtype=np.int64)
    # beta1 = 1/2 keeps m = 1 (or 0); beta2 = 1/2 keeps v = 1; eps = 0: u = m
    out = R.lamb_warmup_step(x, m0, v0, g, off, lr=0.25, eps=0.0, beta1=0.5, beta2=0.5)
    assert np.array_equal(out["c"], np.array([5, 1], dtype=F32))
    assert np.array_equal(out["x"], np.array([3 - 1.25, 4, -0.25, -0.25], dtype=F32))
    assert np.array_equal(out["c_avg"], out["c"])


def test_exact_binary64_sums_against_fsum():
    """The squared norms are the exact sums rounded once to binary64, which
    math.fsum gives independently: checked through the coefficient of a
    layer whose update direction has norm 1 exactly."""
    import math

    rng = np.random.default_rng(71)
    for trial in range(20):
        d = int(rng.integers(1, 500))
        x = (rng.standard_normal(d) * 10.0 ** rng.uniform(-20, 20, size=d)).astype(F32)
        # u = (1, 0, ..., 0) exactly: m = g = e0, v = 1, betas 1/2, eps 0
        e0 = np.zeros(d, dtype=F32)
        e0[0] = 1
        out = R.lamb_warmup_step(x, e0, np.ones(d, F32), e0, np.array([0, d]), lr=0.0, eps=0.0,
                                 beta1=0.5, beta2=0.5)
        sx = math.fsum((x.astype(np.float64) ** 2).tolist())
        assert out["c"][0] == F32(math.sqrt(sx)), trial


def test_exact_sums_against_fsum_and_ties():
    """The binary64 sums directly: math.fsum (an independent exact summation,
    rounded once) on random data over 60 decades and subnormals, and
    hand-made ties: 1 + 2^-52 + 2^-53 lies halfway between two binary64
    values and goes to the even one, 1 + 2^-51; 1 + 2^-53 goes to 1."""
    import math

    rng = np.random.default_rng(72)
    for trial in range(100):
        d = int(rng.integers(1, 2000))
        x = (rng.standard_normal(d) * 10.0 ** rng.uniform(-45, 15, size=d)).astype(F32)
        assert R.exact_sumsq(x) == math.fsum((x.astype(np.float64) ** 2).tolist()), trial
        y = np.abs(rng.standard_normal(d) * 10.0 ** rng.uniform(-300, 300, size=d))
        y[: d // 7] = 5e-324 * rng.integers(0, 1000, size=d // 7)
        assert R.exact_sum_f64(y) == math.fsum(y.tolist()), trial
    assert R.exact_sumsq(np.array([1, 2.0 ** -26, 2.0 ** -27, 2.0 ** -27], F32)) == 1 + 2.0 ** -51
    assert R.exact_sumsq(np.array([1, 2.0 ** -27, 2.0 ** -27], F32)) == 1.0
    assert R.exact_sum_f64(np.array([1.0, 2.0 ** -52, 2.0 ** -53])) == 1 + 2.0 ** -51
    assert np.isnan(R.exact_sumsq(np.array([1, np.nan, np.inf], F32)))
    assert R.exact_sumsq(np.array([1, -np.inf], F32)) == np.inf


def test_exact_sums_at_the_extreme_exponents():
    """The wide-integer sums at the ends of their ranges: the largest binary32
    squared (2^256 ulp-scale terms) and the smallest subnormal squared
    (2^-298), the largest and smallest binary64 values, and the exact mean
    of binary32 values at both ends, each against an independent exact sum
    (math.fsum, Fractions)."""
    import math

    fmax, tiny32 = np.finfo(F32).max, F32(2.0 ** -149)
    for x in (np.full(3000, fmax, F32), np.array([fmax, tiny32, -fmax, tiny32], F32),
              np.full(777, tiny32, F32), np.array([tiny32, 1, fmax], F32)):
        assert R.exact_sumsq(x) == math.fsum((x.astype(np.float64) ** 2).tolist())
    dmax, dtiny = np.finfo(np.float64).max, 5e-324
    for y in (np.array([dmax / 4, dmax / 4, dmax / 8]), np.full(999, dtiny),
              np.array([dmax / 2, dtiny, dtiny]), np.array([dtiny, 1.0, dtiny])):
        assert R.exact_sum_f64(y) == math.fsum(y.tolist())
    for x in (np.array([fmax, fmax, tiny32, fmax], F32), np.array([tiny32] * 5 + [0] * 59, F32)):
        exact = sum((abs(Fraction(float(v))) for v in x), Fraction(0)) / x.size
        got = R.mean_abs_f32(x)
        lo, hi = np.nextafter(got, F32(0)), np.nextafter(got, F32(np.inf))
        d = abs(Fraction(float(got)) - exact)
        assert d <= abs(Fraction(float(lo)) - exact)
        if np.isfinite(hi):
            assert d <= abs(Fraction(float(hi)) - exact)


def _cpp_trust_ratio(x_l, u_l):
    """The C++ oracle's coefficient of one layer, taken through its warm-up
    step: with u's entries 0 or 1, m = g = u, v = 1, beta1 = beta2 = 1/2 and
    eps = 0 leave the update direction equal to u; zero padding to a common
    length changes neither norm."""
    x = np.asarray(x_l, dtype=F32)
    u = np.asarray(u_l, dtype=F32)
    assert np.all((u == 0) | (u == 1))
    n = max(x.size, u.size)
    xp, up = np.zeros(n, F32), np.zeros(n, F32)
    xp[:x.size], up[:u.size] = x, u
    out = R.lamb_warmup_step(xp, up, np.ones(n, F32), up, np.array([0, n], dtype=np.int64),
                             lr=0.0, eps=0.0, beta1=0.5, beta2=0.5)
    return out["c"][0]


_CPP_PINS = [
    ("tests.test_oracle_warmup", "test_sum_of_squares_is_exact_then_rounded_once", W, "exact_sumsq",
     R.exact_sumsq),
    ("tests.test_oracle_warmup", "test_trust_ratio_is_the_quotient_of_the_roots", W, "trust_ratio",
     _cpp_trust_ratio),
    ("tests.test_oracle_warmup", "test_rms_is_the_root_of_the_rounded_mean_square", W,
     "momentum_scale", R.momentum_scale),
    ("tests.test_oracle_warmup", "test_mean_of_rms_values_is_summed_exactly", W, "momentum_scale",
     R.momentum_scale),
    ("tests.test_oracle_int8", "test_codes_clamp_to_127_on_both_sides", None, "int8_sr", R.int8_sr),
    ("tests.test_oracle_int8", "test_nan_is_left_out_of_the_block_maximum", None, "int8_sr",
     R.int8_sr),
    ("tests.test_oracle_optim", "test_lamb_step_by_hand", P, "lamb_frozen_step", R.lamb_frozen_step),
    ("tests.test_oracle_onebit", "test_layer_coefficient_scales_the_momentum_not_the_error", O,
     "worker_compress", R.worker_compress),
    ("tests.test_oracle_optim", "test_adam_step_rounding_sequence", P, "adam_frozen_step",
     R.adam_frozen_step),
    ("tests.test_oracle_onebit", "test_division_by_the_layer_coefficient_is_a_true_division", O,
     "decompress", R.decompress),
    ("tests.test_oracle_warmup", "test_lamb_step_takes_this_steps_coefficient_not_the_average", W,
     "lamb_warmup_step", R.lamb_warmup_step),
    ("tests.test_oracle_exact", "test_mean_abs_is_rounded_once_from_the_exact_value", None,
     "mean_abs_f32", R.mean_abs_f32),
]


@pytest.mark.parametrize("pin", _CPP_PINS, ids=[p[1] for p in _CPP_PINS])
def test_cpp_oracle_passes_the_rounding_and_edge_pins(pin):
    """The numpy oracle's pins for rounding compositions and sequences, the
    INT8 clamp and NaN, the LAMB step by hand and the layer coefficient, run
    with the C++ oracle's function in place of the numpy one (the pin
    module's own name where it imported the function)."""
    import importlib
    from unittest import mock

    mod_name, test_name, module, attr, cpp_fn = pin
    tm = importlib.import_module(mod_name)
    target = tm if module is None else module
    with mock.patch.object(target, attr, cpp_fn):
        getattr(tm, test_name)()


def test_cpp_oracle_passes_every_applicable_pin():
    """Every pin of the numpy oracle's modules, run with every function the
    C++ oracle offers put in place of its numpy counterpart at once (also
    where a pin module imported it by name). A pin that reads an output the
    C++ binding leaves out (the LAMB warm-up's update direction u) does not
    apply; every other pin must pass."""
    import contextlib
    import importlib
    from unittest import mock

    from oracle import exact as X
    from tests.test_oracle_mutations import _pin_calls
    from tests.test_oracle_philox import build_rocrand_dump

    subs = [(O, "worker_compress", R.worker_compress), (O, "server_reduce", R.server_reduce),
            (O, "decompress", R.decompress), (O, "local_momentum", R.local_momentum),
            (P, "adam_frozen_step", R.adam_frozen_step),
            (P, "lamb_frozen_step", R.lamb_frozen_step), (I, "int8_sr", R.int8_sr),
            (PH, "philox4x32_10", R.philox4x32_10), (PH, "uniforms", R.uniforms),
            (W, "momentum_scale", R.momentum_scale), (W, "exact_sumsq", R.exact_sumsq),
            (W, "lamb_warmup_step", R.lamb_warmup_step),
            (W, "adam_warmup_step", R.adam_warmup_step), (X, "mean_abs_f32", R.mean_abs_f32)]
    names = ["tests.test_oracle_bits", "tests.test_oracle_exact", "tests.test_oracle_onebit",
             "tests.test_oracle_optim", "tests.test_oracle_int8", "tests.test_oracle_philox",
             "tests.test_oracle_warmup"]
    mods = [importlib.import_module(m) for m in names]
    run = build_rocrand_dump()
    fixtures = {} if run is None else {"rocrand_dump": run}
    passed, not_applicable = 0, []
    with contextlib.ExitStack() as stack:
        for mod, attr, fn in subs:
            orig = getattr(mod, attr)
            stack.enter_context(mock.patch.object(mod, attr, fn))
            for tm in mods:
                if getattr(tm, attr, None) is orig:
                    stack.enter_context(mock.patch.object(tm, attr, fn))
        for m in names:
            for name, fn, kw in _pin_calls(m, fixtures):
                try:
                    fn(**kw)
                    passed += 1
                except KeyError as e:  # an output the C++ binding does not return
                    not_applicable.append((name, str(e)))
    assert passed >= 80
    assert all(key == "'u'" for _, key in not_applicable), not_applicable
