"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in the oracle -- a flipped sign, a
wrong bit order, a swapped factor, a missing term -- for the duration of the
case only (on the CPU, through the module attribute the oracle itself looks
up at call time, and for the cases so marked also where a pin module
imported the function by name), runs the pins of the affected oracle
modules, and asserts that at least one of them fails.  A case that no pin caught would mean the
oracle could carry that mistake unnoticed.

The Philox cases rerun the rocRAND cross-check pins with the cross-check
built once for this module.
"""

import contextlib
import importlib
import inspect
import math
from unittest import mock

import numpy as np
import pytest

from oracle import bits as B
from oracle import exact as X
from oracle import int8 as I
from oracle import onebit as O
from oracle import optim as P
from oracle import philox as PH
from oracle import warmup as W

F32 = np.float32


def _pin_calls(module_name, fixtures):
    """(name, function, kwargs) for every pin of a module: no arguments, the
    fixtures given, or a single parametrize mark expanded into its cases."""
    mod = importlib.import_module(module_name)
    for name, fn in sorted(vars(mod).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        params = list(inspect.signature(fn).parameters)
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            yield name, fn, {}
        elif set(params) <= set(fixtures):
            yield name, fn, {p: fixtures[p] for p in params}
        elif len(marks) == 1:
            names = [p.strip() for p in marks[0].args[0].split(",")]
            if set(names) != set(params):
                continue
            for vals in marks[0].args[1]:
                vals = vals if isinstance(vals, (tuple, list)) else (vals,)
                yield name, fn, dict(zip(names, vals))


def _first_failing(modules, fixtures):
    for m in modules:
        for name, fn, kw in _pin_calls(m, fixtures):
            try:
                with np.errstate(all="ignore"):
                    fn(**kw)
            except AssertionError:  # only a failed pin counts (a broken mutant does not)
                return f"{m}.{name}"
    return None


# ---------------------------------------------------------------- mutants

def sign_gt(x):  # sign(0) = -1
    return np.asarray(x) > 0


def pack_msb_first(b):  # numpy's default bit order
    b = np.asarray(b, dtype=bool).ravel()
    weights = np.uint64(1) << np.arange(31, -1, -1, dtype=np.uint64)
    return (b.reshape(-1, 32).astype(np.uint64) * weights).sum(axis=1).astype(np.uint32)


def error_wrong_sign(gc, s):
    s = F32(s)
    return np.where(B.sign_bit(gc), gc + s, gc - s).astype(F32)


def mean_over_n_minus_1(x):
    a = np.asarray(x, dtype=F32).ravel()
    return X.round_rational_to_f32(X.abs_units(a), max(1, a.size - 1) << 149)


def round_truncating(num, den):  # toward zero instead of to nearest
    q = F32(num / den)
    if abs(float(q)) > num / den:
        q = np.nextafter(q, F32(0))
    return F32(q)


def clamp_half(x, clip):
    c = F32(clip)
    if not (c > 0) or np.isinf(c):
        return x
    return np.fmin(np.fmax(x, -c / 2), c / 2).astype(F32)


def local_momentum_swapped(g, mbar_prev, beta1):
    b1 = F32(beta1)
    omb1 = F32(F32(1.0) - b1)
    a = (omb1 * np.asarray(mbar_prev, dtype=F32)).astype(F32)
    return (a[None, :] + (b1 * np.asarray(g, dtype=F32)).astype(F32)).astype(F32)


def decompress_times_k(sbits, S, k=None):
    d = O.__dict__["_orig_decompress"](sbits, S)
    return d if k is None else (d * np.asarray(k, dtype=F32)).astype(F32)


def adam_eps_inside(x, m, v, lr, eps):
    den = np.sqrt((np.asarray(v, dtype=F32) + F32(eps)).astype(F32)).astype(F32)
    upd = (np.asarray(m, dtype=F32) / den).astype(F32)
    return (np.asarray(x, dtype=F32) - (F32(lr) * upd).astype(F32)).astype(F32)


def reconstruct_over_beta1(m, m_prev, beta1):
    b1 = F32(beta1)
    num = (np.asarray(m, dtype=F32) - (b1 * np.asarray(m_prev, dtype=F32)).astype(F32)).astype(F32)
    return (num / b1).astype(F32)


def fresh_variance_swapped(v_f, g, beta2):
    b2 = F32(beta2)
    omb2 = F32(F32(1.0) - b2)
    g = np.asarray(g, dtype=F32)
    return ((omb2 * np.asarray(v_f, dtype=F32)).astype(F32)
            + (b2 * (g * g).astype(F32)).astype(F32)).astype(F32)


def ratio_hard_clip_first(R, r_prev, c_avg, thr, r_min, r_max):
    R = np.asarray(R, dtype=F32)
    r_prev = np.asarray(r_prev, dtype=F32)
    R = np.where(np.isnan(R), r_prev, R).astype(F32)
    r = np.fmin(np.fmax(R, F32(r_min)), F32(r_max)).astype(F32)
    lo = (F32(F32(1.0) - F32(thr)) * r_prev).astype(F32)
    hi = (F32(F32(1.0) + F32(thr)) * r_prev).astype(F32)
    r = np.fmin(np.fmax(r, lo), hi).astype(F32)
    return r, (np.asarray(c_avg, dtype=F32) * r).astype(F32)


def layer_max_keeps_nan(vals, seg_off):
    out = np.full(len(seg_off) - 1, np.nan, dtype=F32)
    for l in range(len(seg_off) - 1):
        seg = np.asarray(vals[int(seg_off[l]):int(seg_off[l + 1])], dtype=F32)
        if seg.size:
            out[l] = seg.max()
    return out


def trust_ratio_inverted(x_l, u_l):
    sx, su = W.exact_sumsq(x_l), W.exact_sumsq(u_l)
    if sx == 0.0 or su == 0.0:
        return F32(1.0)
    return F32(np.sqrt(su) / np.sqrt(sx))


def average_swapped(c_avg, c, beta_c):
    c = np.asarray(c, dtype=F32)
    if c_avg is None:
        return c.copy()
    return ((W._omb(beta_c) * np.asarray(c_avg, dtype=F32)).astype(F32)
            + (F32(beta_c) * c).astype(F32)).astype(F32)


def momentum_scale_by_norm(m, seg_off):
    m = np.asarray(m, dtype=F32)
    S = len(seg_off) - 1
    nrm = [np.sqrt(W.exact_sumsq(m[int(seg_off[l]):int(seg_off[l + 1])])) for l in range(S)]
    valid = [a for a in nrm if a > 0]
    mean = sum(valid) / len(valid) if valid else 0.0
    return np.array([F32(mean / a) if a > 0 else F32(1.0) for a in nrm], dtype=F32)


def moments_abs_g(m, v, g, beta1, beta2):
    b1, b2 = F32(beta1), F32(beta2)
    g = np.asarray(g, dtype=F32)
    m_new = ((b1 * np.asarray(m, dtype=F32)).astype(F32) + (W._omb(beta1) * g).astype(F32)).astype(F32)
    v_new = ((b2 * np.asarray(v, dtype=F32)).astype(F32)
             + (W._omb(beta2) * np.abs(g)).astype(F32)).astype(F32)
    return m_new, v_new


def uniforms_squared(J0, count, seed, step):
    u = I.__dict__["_orig_uniforms"](J0, count, seed, step)
    return (u * u).astype(F32)


def round_half_even(x):
    return np.rint(np.asarray(x, dtype=F32)).astype(F32)


def unpack_msb_first(words, count=None):
    w = np.asarray(words, dtype=np.uint32).ravel()
    pos = np.arange(31, -1, -1, dtype=np.uint32)
    b = ((w[:, None] >> pos[None, :]) & np.uint32(1)).astype(bool).ravel()
    return b if count is None else b[:count]


def signed_swapped(b, s):
    s = F32(s)
    return np.where(b, -s, s).astype(F32)


def _server_chunk_variant(order="up", reciprocal=False, keep_error_on_reset=False):
    def server_chunk(bits_c, s_c, E_c, reset=False, unit_scale=False, err_ratio_c=None):
        bits_c = np.asarray(bits_c, dtype=np.uint32)
        s_c = np.asarray(s_c, dtype=F32)
        n = s_c.shape[0]
        L = bits_c.shape[1] * 32
        acc = np.zeros(L, dtype=F32)
        for i in (range(n) if order == "up" else range(n - 1, -1, -1)):
            acc = (acc + B.signed(B.unpack(bits_c[i]), s_c[i])).astype(F32)
        avg = ((acc * F32(F32(1.0) / F32(n))) if reciprocal else (acc / F32(n))).astype(F32)
        E_in = np.zeros(L, dtype=F32) if (reset and not keep_error_on_reset) else np.asarray(E_c, dtype=F32)
        if err_ratio_c is not None and not reset:
            E_in = (np.asarray(err_ratio_c, dtype=F32) * E_in).astype(F32)
        g2 = (avg + E_in).astype(F32)
        S = F32(1.0) if unit_scale else O.mean_abs_f32(g2)
        return {"avg": avg, "g2": g2, "bits": B.pack(B.sign_bit(g2)), "S": S,
                "E": O.error_from(g2, S)}
    return server_chunk


def _worker_variant(clip_before=False, ignore_reset=False):
    def worker_compress(m, e, clip=0.0, reset=False, k=None, unit_scale=False, err_ratio=None):
        m = np.asarray(m, dtype=F32)
        n, N = m.shape
        L = N // n
        e_in = np.zeros_like(m) if (reset and not ignore_reset) else np.asarray(e, dtype=F32)
        if err_ratio is not None and not reset:
            e_in = (np.asarray(err_ratio, dtype=F32)[None, :] * e_in).astype(F32)
        gc = np.empty_like(m)
        e_out = np.empty_like(m)
        s = np.empty((n, n), dtype=F32)
        bits = np.empty((n, N // 32), dtype=np.uint32)
        for i in range(n):
            mi = m[i] if k is None else (np.asarray(k, dtype=F32) * m[i]).astype(F32)
            if clip_before:
                gi = (O.clamp(mi, clip) + e_in[i]).astype(F32)
            else:
                gi = O.clamp((mi + e_in[i]).astype(F32), clip)
            gc[i] = gi
            for c in range(n):
                sl = slice(c * L, (c + 1) * L)
                s[i, c] = F32(1.0) if unit_scale else O.mean_abs_f32(gi[sl])
                e_out[i, sl] = O.error_from(gi[sl], s[i, c])
            bits[i] = B.pack(B.sign_bit(gi))
        return {"gc": gc, "bits": bits, "s": s, "e": e_out}
    return worker_compress


def decompress_first_scale(sbits, S, k=None):
    S = np.asarray(S, dtype=F32)
    return O.__dict__["_orig_decompress"](sbits, np.full_like(S, S[0]), k)


def layer_scale_swapped(buf, seg_off, k, divide):
    return O.__dict__["_orig_layer_scale"](buf, seg_off, k, not divide)


def per_element_k_shifted(seg_off, k):
    k = np.asarray(k, dtype=F32)
    sizes = np.diff(np.asarray(seg_off, dtype=np.int64))
    return np.repeat(np.roll(k, 1), sizes).astype(F32)


def local_momentum_unrounded(g, mbar_prev, beta1):
    b1 = F32(beta1)
    a = (b1 * np.asarray(mbar_prev, dtype=F32)).astype(F32)
    t = ((1.0 - float(beta1)) * np.asarray(g, dtype=F32).astype(np.float64)).astype(F32)
    return (a[None, :] + t).astype(F32)


def lamb_apply_without_c(x, m, v_tw, seg_off, c_used, lr, eps):
    return P.__dict__["_orig_lamb_apply"](x, m, v_tw, seg_off, np.ones_like(np.asarray(c_used, dtype=F32)),
                                           lr, eps)


def lamb_step_ratio_inverted(*args, **kw):
    out = P.__dict__["_orig_lamb_frozen_step"](*args, **kw)
    out["err_ratio"] = (F32(1.0) / out["err_ratio"]).astype(F32)
    return out


def philox_nine_rounds(ctr, key):
    x = np.asarray(ctr, dtype=np.uint32).astype(np.uint64)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint32), x.shape[:-1] + (2,)).astype(np.uint64)
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    mask = np.uint64(0xFFFFFFFF)
    for rnd in range(9):
        if rnd:
            k0 = (k0 + PH.W0) & mask
            k1 = (k1 + PH.W1) & mask
        p0, p1 = PH.M0 * x0, PH.M1 * x2
        x0, x1, x2, x3 = (p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & mask, (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & mask
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def uniforms_down_half_step(J0, count, seed, step):  # u <= p in place of u < p
    u = I.__dict__["_orig_uniforms"](J0, count, seed, step)
    return (u.astype(np.float64) - 2.0 ** -25).astype(F32)


def sumsq_binary32(a):
    acc = F32(0.0)
    for t in np.asarray(a, dtype=F32):
        acc = F32(acc + F32(t * t))
    return float(acc)


def trust_ratio_zero_norm_zero(x_l, u_l):
    sx, su = W.exact_sumsq(x_l), W.exact_sumsq(u_l)
    if sx == 0.0 or su == 0.0:
        return F32(0.0)
    return F32(np.sqrt(sx) / np.sqrt(su))


def average_started_at_one(c_avg, c, beta_c):
    if c_avg is None:
        c_avg = np.ones_like(np.asarray(c, dtype=F32))
    return W.__dict__["_orig_coefficient_average"](c_avg, c, beta_c)


def momentum_scale_counts_empty(m, seg_off):
    import math
    m = np.asarray(m, dtype=F32)
    S = len(seg_off) - 1
    rms = []
    for l in range(S):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        rms.append(math.sqrt(W.exact_sumsq(m[a:b]) / (b - a)) if b > a else 0.0)
    valid = [r for r in rms if r > 0.0]
    k = np.ones(S, dtype=F32)
    if not valid:
        return k
    mean = math.fsum(rms) / S
    for l in range(S):
        if rms[l] > 0.0:
            k[l] = F32(mean / rms[l])
    return k


def trust_ratio_root_of_quotient(x_l, u_l):
    import math
    sx, su = W.exact_sumsq(x_l), W.exact_sumsq(u_l)
    if sx == 0.0 or su == 0.0:
        return F32(1.0)
    return F32(math.sqrt(sx / su))


def sumsq_binary64_running(a):
    acc = 0.0
    for t in np.asarray(a, dtype=F32).astype(np.float64):
        acc += t * t
    return acc


def _momentum_scale_variant(root_over_root=False, running_mean=False):
    import math

    def f(m, seg_off):
        m = np.asarray(m, dtype=F32)
        S = len(seg_off) - 1
        rms = [0.0] * S
        for l in range(S):
            a, b = int(seg_off[l]), int(seg_off[l + 1])
            if b > a:
                s = W.exact_sumsq(m[a:b])
                rms[l] = math.sqrt(s) / math.sqrt(b - a) if root_over_root else math.sqrt(s / (b - a))
        valid = [r for r in rms if r > 0.0]
        k = np.ones(S, dtype=F32)
        if not valid:
            return k
        if running_mean:
            acc = 0.0
            for r in valid:
                acc += r
        else:
            acc = math.fsum(valid)
        mean = acc / len(valid)
        for l in range(S):
            if rms[l] > 0.0:
                k[l] = F32(mean / rms[l])
        return k
    return f


def _int8_variant(clamp_lo=-127.0, div=127.0, err_flip=False, nan_in_max=False):
    """The block quantiser with one planted change (stochastic rounding)."""
    def f(g, e, seed, step, block=256, J0=0, rounding="stochastic"):
        g = np.asarray(g, dtype=F32).ravel()
        N = g.size
        block = block or N
        gc = g if e is None else (g + np.asarray(e, dtype=F32).ravel()).astype(F32)
        a = np.abs(gc).reshape(-1, block)
        if not nan_in_max:
            a = np.where(np.isnan(a), F32(0.0), a)
        scale = (np.fmax(a.max(axis=1).astype(F32), F32(0.0)) / F32(div)).astype(F32)
        sc = np.repeat(scale, block)
        with np.errstate(divide="ignore", invalid="ignore"):
            x = (gc / sc).astype(F32)
            if rounding == "nearest":
                q = I.round_half_away(x)
            else:
                u = I.uniforms(J0, N, seed, step)
                fl = np.floor(x).astype(F32)
                q = (fl + np.where(u < (x - fl).astype(F32), F32(1.0), F32(0.0))).astype(F32)
            q = np.fmin(np.fmax(q, F32(clamp_lo)), F32(127.0))
        zero = sc == 0
        q = np.where(zero, F32(0.0), q)
        with np.errstate(invalid="ignore", over="ignore"):
            deq = np.where(zero, F32(0.0), (q * sc).astype(F32)).astype(F32)
            e_new = ((deq - gc) if err_flip else (gc - deq)).astype(F32)
        return {"gc": gc, "codes": q.astype(np.int8), "scales": scale, "deq": deq, "e": e_new}
    return f


def _uniforms_variant(step_word=2, key_swapped=False, words_reversed=False, low_bits=False,
                      half_step=False):
    """Element uniforms with one planted change in the counter, key, word
    choice or the mapping of the word to [0, 1)."""
    mask = np.uint64(0xFFFFFFFF)

    def f(J0, count, seed, step):
        J = np.arange(J0, J0 + count, dtype=np.uint64)
        blk = J >> np.uint64(2)
        cols = [blk & mask, blk >> np.uint64(32), np.zeros_like(blk), np.zeros_like(blk)]
        cols[step_word] = np.full_like(blk, np.uint64(step) & mask)
        key = [seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF]
        if key_swapped:
            key = key[::-1]
        words = PH.philox4x32_10(np.stack(cols, axis=-1).astype(np.uint32),
                                 np.array(key, dtype=np.uint32))
        idx = (J & np.uint64(3)).astype(np.int64)
        w = words[np.arange(count), 3 - idx if words_reversed else idx]
        v = ((w & np.uint32(0xFFFFFF)) if low_bits else (w >> np.uint32(8))).astype(np.float64)
        v = v * 2.0 ** -24 + (2.0 ** -25 if half_step else 0.0)
        return v.astype(F32)
    return f


def _ratio_update_variant(nan_to_one=False, band_around_one=False):
    def f(R, r_prev, c_avg, thr, r_min, r_max):
        R = np.asarray(R, dtype=F32)
        r_prev = np.asarray(r_prev, dtype=F32)
        R = np.where(np.isnan(R), F32(1.0) if nan_to_one else r_prev, R).astype(F32)
        base = np.ones_like(r_prev) if band_around_one else r_prev
        lo = (F32(F32(1.0) - F32(thr)) * base).astype(F32)
        hi = (F32(F32(1.0) + F32(thr)) * base).astype(F32)
        r = np.fmin(np.fmax(np.fmin(np.fmax(R, lo), hi), F32(r_min)), F32(r_max)).astype(F32)
        return r, (np.asarray(c_avg, dtype=F32) * r).astype(F32)
    return f


def _lamb_step_variant(ratio_inverted=False, fresh_v_in_step=False, c_t_always=None):
    def f(x, m, m_prev, v_f, v_tw, seg_off, c_avg, r_prev, c_prev, lr, eps, beta1, beta2,
          thr, r_min, r_max, use_c_t=False):
        g = P.reconstruct_gradient(m, m_prev, beta1)
        v_new = P.fresh_variance(v_f, g, beta2)
        vt = np.asarray(v_tw, dtype=F32)
        ratio = ((v_new / vt) if ratio_inverted else (vt / v_new)).astype(F32)
        R = P.layer_max(ratio, seg_off)
        r, c = P.lamb_ratio_update(R, r_prev, c_avg, thr, r_min, r_max)
        use = use_c_t if c_t_always is None else c_t_always
        c_used = c if use else np.asarray(c_prev, dtype=F32)
        x_new = P.lamb_apply(x, m, v_new if fresh_v_in_step else v_tw, seg_off, c_used, lr, eps)
        rho = (np.asarray(c_prev, dtype=F32) / c).astype(F32)
        return {"x": x_new, "v": v_new, "R": R, "r": r, "c": c, "g": g, "err_ratio": rho}
    return f


def adam_step_adds(x, m, v, lr, eps):
    x = np.asarray(x, dtype=F32)
    den = (np.sqrt(np.asarray(v, dtype=F32)) + F32(eps)).astype(F32)
    upd = (np.asarray(m, dtype=F32) / den).astype(F32)
    return (x + (F32(lr) * upd).astype(F32)).astype(F32)


def clamp_nan_to_plus(x, clip):
    c = F32(clip)
    if not (c > 0) or np.isinf(c):
        return x
    return np.where(np.isnan(x), c, np.fmin(np.fmax(x, -c), c)).astype(F32)


def clamp_keeps_nan(x, clip):
    c = F32(clip)
    if not (c > 0) or np.isinf(c):
        return x
    return np.minimum(np.maximum(x, -c), c).astype(F32)


def worker_k_on_the_sum(m, e, clip=0.0, reset=False, k=None, unit_scale=False, err_ratio=None):
    """k_l (m + e) in place of k_l m + e: the scaled momentum's error scaled again."""
    orig = O.__dict__["_orig_worker_compress"]
    if k is None or reset:
        return orig(m, e, clip, reset, k, unit_scale, err_ratio)
    e = np.asarray(e, dtype=F32)
    if err_ratio is not None:
        e = (np.asarray(err_ratio, dtype=F32)[None, :] * e).astype(F32)
    kk = np.asarray(k, dtype=F32)
    # fold the extra factor into the error: k m + (k e) == k (m + e) up to rounding
    return orig(m, (kk[None, :] * e).astype(F32), clip, reset, k, unit_scale, None)


def server_scales_divided_first(bits_c, s_c, E_c, reset=False, unit_scale=False, err_ratio_c=None):
    """The average as the ordered sum of +-s_i / n in place of (sum of +-s_i) / n."""
    s_c = np.asarray(s_c, dtype=F32)
    n = s_c.shape[0]
    acc = np.zeros(np.asarray(bits_c).shape[1] * 32, dtype=F32)
    for i in range(n):
        acc = (acc + B.signed(B.unpack(bits_c[i]), F32(s_c[i] / F32(n)))).astype(F32)
    E_in = np.zeros_like(acc) if reset else np.asarray(E_c, dtype=F32)
    if err_ratio_c is not None and not reset:
        E_in = (np.asarray(err_ratio_c, dtype=F32) * E_in).astype(F32)
    g2 = (acc + E_in).astype(F32)
    S = F32(1.0) if unit_scale else X.mean_abs_f32(g2)
    return {"avg": acc, "g2": g2, "bits": B.pack(B.sign_bit(g2)), "S": S, "E": O.error_from(g2, S)}


def layer_scale_by_reciprocal(buf, seg_off, k, divide):
    buf = np.asarray(buf, dtype=F32)
    out = np.empty_like(buf)
    k = np.asarray(k, dtype=F32)
    for l in range(len(seg_off) - 1):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        out[..., a:b] = buf[..., a:b] * (F32(F32(1) / k[l]) if divide else k[l])
    return out


def decompress_by_reciprocal(sbits, S, k=None):
    out = O.__dict__["_orig_decompress"](sbits, S)
    if k is not None:
        out = (out * (F32(1) / np.asarray(k, dtype=F32)).astype(F32)).astype(F32)
    return out


def reconstruct_by_reciprocal(m, m_prev, beta1):
    b1 = F32(beta1)
    omb1 = F32(F32(1) - b1)
    num = (np.asarray(m, dtype=F32) - (b1 * np.asarray(m_prev, dtype=F32)).astype(F32)).astype(F32)
    return (num * F32(F32(1) / omb1)).astype(F32)


def fresh_variance_square_last(v_f, g, beta2):
    b2 = F32(beta2)
    omb2 = F32(F32(1) - b2)
    g = np.asarray(g, dtype=F32)
    return ((b2 * np.asarray(v_f, dtype=F32)).astype(F32)
            + ((omb2 * g).astype(F32) * g).astype(F32)).astype(F32)


def adam_lr_times_m_first(x, m, v, lr, eps):
    den = (np.sqrt(np.asarray(v, dtype=F32)) + F32(eps)).astype(F32)
    upd = ((F32(lr) * np.asarray(m, dtype=F32)).astype(F32) / den).astype(F32)
    return (np.asarray(x, dtype=F32) - upd).astype(F32)


def adam_by_reciprocal(x, m, v, lr, eps):
    den = (np.sqrt(np.asarray(v, dtype=F32)) + F32(eps)).astype(F32)
    upd = (np.asarray(m, dtype=F32) * (F32(1) / den).astype(F32)).astype(F32)
    return (np.asarray(x, dtype=F32) - (F32(lr) * upd).astype(F32)).astype(F32)


def lamb_apply_c_times_update_first(x, m, v_tw, seg_off, c_used, lr, eps):
    x = np.asarray(x, dtype=F32)
    den = (np.sqrt(np.asarray(v_tw, dtype=F32)) + F32(eps)).astype(F32)
    upd = (np.asarray(m, dtype=F32) / den).astype(F32)
    out = np.empty_like(x)
    for l in range(len(seg_off) - 1):
        a, b = int(seg_off[l]), int(seg_off[l + 1])
        cu = (F32(c_used[l]) * upd[a:b]).astype(F32)
        out[a:b] = (x[a:b] - (F32(lr) * cu).astype(F32)).astype(F32)
    return out


def momentum_scale_inverted(m, seg_off):
    k = W.__dict__["_orig_momentum_scale"](m, seg_off)
    return (F32(1) / k).astype(F32)


def adam_warmup_with_old_moments(x, m, v, g, lr, eps, beta1, beta2):
    m_new, v_new = W.moments(m, v, g, beta1, beta2)
    u = W.adam_direction(m, v, eps)
    return {"x": (np.asarray(x, dtype=F32) - (F32(lr) * u).astype(F32)).astype(F32),
            "m": m_new, "v": v_new}


def moments_square_last(m, v, g, beta1, beta2):
    b1, b2 = F32(beta1), F32(beta2)
    g = np.asarray(g, dtype=F32)
    m_new = ((b1 * np.asarray(m, dtype=F32)).astype(F32)
             + (F32(F32(1) - b1) * g).astype(F32)).astype(F32)
    v_new = ((b2 * np.asarray(v, dtype=F32)).astype(F32)
             + ((F32(F32(1) - b2) * g).astype(F32) * g).astype(F32)).astype(F32)
    return m_new, v_new


def direction_eps_inside_the_root(m, v, eps):
    den = np.sqrt((np.asarray(v, dtype=F32) + F32(eps)).astype(F32)).astype(F32)
    return (np.asarray(m, dtype=F32) / den).astype(F32)


def lamb_warmup_step_scaled_by_the_average(x, m, v, g, seg_off, lr, eps, beta1, beta2,
                                           c_avg=None, beta_c=0.9):
    r = dict(W.__dict__["_orig_lamb_warmup_step"](x, m, v, g, seg_off, lr, eps, beta1, beta2,
                                                    c_avg, beta_c))
    if c_avg is not None:
        x = np.asarray(x, dtype=F32)
        r["x"] = x.copy()
        for l in range(len(seg_off) - 1):
            a, b = int(seg_off[l]), int(seg_off[l + 1])
            step = F32(F32(lr) * F32(np.asarray(c_avg, dtype=F32)[l]))
            r["x"][a:b] = (x[a:b] - (step * r["u"][a:b]).astype(F32)).astype(F32)
    return r


def average_with_binary64_one_minus_beta(c_avg, c, beta_c):
    c = np.asarray(c, dtype=F32)
    if c_avg is None:
        return c.copy()
    return ((F32(beta_c) * np.asarray(c_avg, dtype=F32)).astype(F32)
            + (np.float64(1.0 - beta_c) * c.astype(np.float64)).astype(F32)).astype(F32)


def server_error_before_the_divide(bits_c, s_c, E_c, reset=False, unit_scale=False, err_ratio_c=None):
    s_c = np.asarray(s_c, dtype=F32)
    n = s_c.shape[0]
    acc = np.zeros(np.asarray(bits_c).shape[1] * 32, dtype=F32)
    for i in range(n):
        acc = (acc + B.signed(B.unpack(bits_c[i]), s_c[i])).astype(F32)
    E_in = np.zeros_like(acc) if reset else np.asarray(E_c, dtype=F32)
    if err_ratio_c is not None and not reset:
        E_in = (np.asarray(err_ratio_c, dtype=F32) * E_in).astype(F32)
    g2 = ((acc + E_in).astype(F32) / F32(n)).astype(F32)
    S = F32(1.0) if unit_scale else X.mean_abs_f32(g2)
    return {"avg": (acc / F32(n)).astype(F32), "g2": g2, "bits": B.pack(B.sign_bit(g2)), "S": S,
            "E": O.error_from(g2, S)}


def mean_through_binary64_sum(x):
    a = np.abs(np.asarray(x, dtype=F32)).astype(np.float64)
    return F32(math.fsum(a.tolist()) / a.size)


def mean_by_numpy_pairwise(x):
    return F32(np.mean(np.abs(np.asarray(x, dtype=F32)).astype(np.float64)))


CASES = [
    # (id, module, attribute, replacement, pin modules)
    ("sign(0) = -1", B, "sign_bit", sign_gt, ["tests.test_oracle_bits", "tests.test_oracle_onebit"]),
    ("bit order MSB first", B, "pack", pack_msb_first, ["tests.test_oracle_bits"]),
    ("error with the wrong sign", O, "error_from", error_wrong_sign, ["tests.test_oracle_onebit"]),
    ("mean over L - 1", O, "mean_abs_f32", mean_over_n_minus_1, ["tests.test_oracle_onebit"]),
    ("truncating rounding", X, "round_rational_to_f32", round_truncating, ["tests.test_oracle_exact"]),
    ("clamp at half the bound", O, "clamp", clamp_half, ["tests.test_oracle_onebit"]),
    ("momentum factors swapped", O, "local_momentum", local_momentum_swapped, ["tests.test_oracle_onebit"]),
    ("decompress multiplies by k", O, "decompress", decompress_times_k, ["tests.test_oracle_onebit"]),
    ("eps inside the root", P, "adam_frozen_step", adam_eps_inside,
     ["tests.test_oracle_optim", "tests.test_oracle_warmup"]),
    ("gradient over beta1", P, "reconstruct_gradient", reconstruct_over_beta1, ["tests.test_oracle_optim"]),
    ("variance factors swapped", P, "fresh_variance", fresh_variance_swapped, ["tests.test_oracle_optim"]),
    ("hard clip before soft clip", P, "lamb_ratio_update", ratio_hard_clip_first, ["tests.test_oracle_optim"]),
    ("layer max keeps NaN", P, "layer_max", layer_max_keeps_nan, ["tests.test_oracle_optim"]),
    ("trust ratio inverted", W, "trust_ratio", trust_ratio_inverted, ["tests.test_oracle_warmup"]),
    ("average factors swapped", W, "coefficient_average", average_swapped, ["tests.test_oracle_warmup"]),
    ("k from the norm, not the RMS", W, "momentum_scale", momentum_scale_by_norm,
     ["tests.test_oracle_warmup"]),
    ("variance from |g|", W, "moments", moments_abs_g, ["tests.test_oracle_warmup"]),
    ("biased uniforms", I, "uniforms", uniforms_squared, ["tests.test_oracle_int8"]),
    ("halves to even", I, "round_half_away", round_half_even, ["tests.test_oracle_int8"]),
    ("Weyl constant", PH, "W0", np.uint64(0x9E3779BB), ["tests.test_oracle_philox"]),
    ("multiplier", PH, "M1", np.uint64(0xCD9E8D59), ["tests.test_oracle_philox"]),
    ("unpack MSB first", B, "unpack", unpack_msb_first, ["tests.test_oracle_bits", "tests.test_oracle_onebit"]),
    ("scaled sign swapped", B, "signed", signed_swapped, ["tests.test_oracle_onebit"]),
    ("server sums workers in reverse", O, "server_chunk", _server_chunk_variant(order="down"),
     ["tests.test_oracle_onebit"]),
    ("server average by a reciprocal", O, "server_chunk", _server_chunk_variant(reciprocal=True),
     ["tests.test_oracle_onebit"]),
    ("server error kept at reset", O, "server_chunk", _server_chunk_variant(keep_error_on_reset=True),
     ["tests.test_oracle_onebit"]),
    ("clip before compensation", O, "worker_compress", _worker_variant(clip_before=True),
     ["tests.test_oracle_onebit"]),
    ("worker reset ignored", O, "worker_compress", _worker_variant(ignore_reset=True),
     ["tests.test_oracle_onebit"]),
    ("decompress with chunk 0's scale", O, "decompress", decompress_first_scale, ["tests.test_oracle_onebit"]),
    ("layer scale multiply / divide swapped", O, "layer_scale", layer_scale_swapped, ["tests.test_oracle_onebit"]),
    ("layer coefficient one layer off", O, "per_element_k", per_element_k_shifted, ["tests.test_oracle_onebit"]),
    ("1 - beta1 unrounded", O, "local_momentum", local_momentum_unrounded, ["tests.test_oracle_onebit"]),
    ("LAMB step without c", P, "lamb_apply", lamb_apply_without_c, ["tests.test_oracle_optim"]),
    ("error ratio inverted", P, "lamb_frozen_step", lamb_step_ratio_inverted, ["tests.test_oracle_optim"]),
    ("Philox with 9 rounds", PH, "philox4x32_10", philox_nine_rounds, ["tests.test_oracle_philox"]),
    ("u <= p", I, "uniforms", uniforms_down_half_step, ["tests.test_oracle_int8"]),
    ("sum of squares in binary32", W, "exact_sumsq", sumsq_binary32, ["tests.test_oracle_warmup"]),
    ("zero norm gives c = 0", W, "trust_ratio", trust_ratio_zero_norm_zero, ["tests.test_oracle_warmup"]),
    ("average started at 1", W, "coefficient_average", average_started_at_one, ["tests.test_oracle_warmup"]),
    ("k averages empty layers", W, "momentum_scale", momentum_scale_counts_empty, ["tests.test_oracle_warmup"]),
    ("trust ratio as the root of the quotient", W, "trust_ratio", trust_ratio_root_of_quotient,
     ["tests.test_oracle_warmup"]),
    ("sum of squares in running binary64", W, "exact_sumsq", sumsq_binary64_running,
     ["tests.test_oracle_warmup"]),
    ("RMS as a root over a root", W, "momentum_scale", _momentum_scale_variant(root_over_root=True),
     ["tests.test_oracle_warmup"]),
    ("mean of RMS values by a running sum", W, "momentum_scale", _momentum_scale_variant(running_mean=True),
     ["tests.test_oracle_warmup"]),
    # the cases below also replace the name where a pin module imported it
    ("INT8 codes clamped at -128", I, "int8_sr", _int8_variant(clamp_lo=-128.0),
     ["tests.test_oracle_int8"], True),
    ("INT8 scale max/128", I, "int8_sr", _int8_variant(div=128.0), ["tests.test_oracle_int8"], True),
    ("INT8 error with the wrong sign", I, "int8_sr", _int8_variant(err_flip=True),
     ["tests.test_oracle_int8"], True),
    ("INT8 NaN kept in the block maximum", I, "int8_sr", _int8_variant(nan_in_max=True),
     ["tests.test_oracle_int8"], True),
    ("Philox step in counter word 3", PH, "uniforms", _uniforms_variant(step_word=3),
     ["tests.test_oracle_philox"], True),
    ("Philox key halves swapped", PH, "uniforms", _uniforms_variant(key_swapped=True),
     ["tests.test_oracle_philox"], True),
    ("Philox words in reverse order", PH, "uniforms", _uniforms_variant(words_reversed=True),
     ["tests.test_oracle_philox"], True),
    ("uniform from the low 24 bits", PH, "uniforms", _uniforms_variant(low_bits=True),
     ["tests.test_oracle_philox"], True),
    ("uniform offset by half a step", PH, "uniforms", _uniforms_variant(half_step=True),
     ["tests.test_oracle_philox"], True),
    ("no valid ratio gives r = 1", P, "lamb_ratio_update", _ratio_update_variant(nan_to_one=True),
     ["tests.test_oracle_optim"]),
    ("ratio band around 1", P, "lamb_ratio_update", _ratio_update_variant(band_around_one=True),
     ["tests.test_oracle_optim"]),
    ("LAMB ratio fresh over frozen", P, "lamb_frozen_step", _lamb_step_variant(ratio_inverted=True),
     ["tests.test_oracle_optim"]),
    ("LAMB step with the fresh variance", P, "lamb_frozen_step",
     _lamb_step_variant(fresh_v_in_step=True), ["tests.test_oracle_optim"]),
    ("LAMB step always with c_t", P, "lamb_frozen_step", _lamb_step_variant(c_t_always=True),
     ["tests.test_oracle_optim"]),
    ("LAMB step never with c_t", P, "lamb_frozen_step", _lamb_step_variant(c_t_always=False),
     ["tests.test_oracle_optim"]),
    ("Adam step adds the update", P, "adam_frozen_step", adam_step_adds, ["tests.test_oracle_optim"]),
    ("clamp sends NaN to +clip", O, "clamp", clamp_nan_to_plus, ["tests.test_oracle_onebit"]),
    ("clamp keeps NaN", O, "clamp", clamp_keeps_nan, ["tests.test_oracle_onebit"]),
    ("k on momentum plus error", O, "worker_compress", worker_k_on_the_sum, ["tests.test_oracle_onebit"]),
    ("server divides the scales first", O, "server_chunk", server_scales_divided_first,
     ["tests.test_oracle_onebit"]),
    ("layer scale divides by a reciprocal", O, "layer_scale", layer_scale_by_reciprocal,
     ["tests.test_oracle_onebit"]),
    ("decompression divides by a reciprocal", O, "decompress", decompress_by_reciprocal,
     ["tests.test_oracle_onebit"]),
    ("gradient reconstruction by a reciprocal", P, "reconstruct_gradient", reconstruct_by_reciprocal,
     ["tests.test_oracle_optim"]),
    ("fresh variance squares last", P, "fresh_variance", fresh_variance_square_last,
     ["tests.test_oracle_optim"]),
    ("Adam step with lr m first", P, "adam_frozen_step", adam_lr_times_m_first,
     ["tests.test_oracle_optim"]),
    ("Adam step by a reciprocal", P, "adam_frozen_step", adam_by_reciprocal, ["tests.test_oracle_optim"]),
    ("LAMB step with c times the update first", P, "lamb_apply", lamb_apply_c_times_update_first,
     ["tests.test_oracle_optim"]),
    ("k_l inverted", W, "momentum_scale", momentum_scale_inverted, ["tests.test_oracle_warmup"]),
    ("Adam warm-up step with the old moments", W, "adam_warmup_step", adam_warmup_with_old_moments,
     ["tests.test_oracle_warmup"]),
    ("variance with the square last", W, "moments", moments_square_last, ["tests.test_oracle_warmup"]),
    ("warm-up direction with eps inside the root", W, "adam_direction", direction_eps_inside_the_root,
     ["tests.test_oracle_warmup"]),
    ("LAMB warm-up step scaled by the average", W, "lamb_warmup_step",
     lamb_warmup_step_scaled_by_the_average, ["tests.test_oracle_warmup"]),
    ("coefficient average with a binary64 1 - beta", W, "coefficient_average",
     average_with_binary64_one_minus_beta, ["tests.test_oracle_warmup"]),
    ("server adds its error before dividing by n", O, "server_chunk", server_error_before_the_divide,
     ["tests.test_oracle_onebit"]),
    ("chunk mean through a binary64 sum", X, "mean_abs_f32", mean_through_binary64_sum,
     ["tests.test_oracle_exact"], True),
    ("chunk mean by numpy's pairwise sum", X, "mean_abs_f32", mean_by_numpy_pairwise,
     ["tests.test_oracle_exact"], True),
]


@pytest.fixture(scope="module")
def fixtures():
    from tests.test_oracle_philox import build_rocrand_dump

    run = build_rocrand_dump()
    return {} if run is None else {"rocrand_dump": run}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_planted_mistake(case, fixtures):
    _, module, attr, mutant, pins = case[:5]
    by_name = len(case) > 5 and case[5]
    if "tests.test_oracle_philox" in pins and "rocrand_dump" not in fixtures:
        pytest.skip("hipcc not available to build the rocRAND cross-check")
    # imported before any patching, so that no pin module binds a mutant
    pin_mods = [importlib.import_module(m) for m in pins]
    original = getattr(module, attr)
    extra = {f"_orig_{attr}": original}
    if attr == "uniforms":
        extra = {"_orig_uniforms": PH.uniforms}
    with contextlib.ExitStack() as stack:
        stack.enter_context(mock.patch.dict(module.__dict__, extra))
        stack.enter_context(mock.patch.object(module, attr, mutant))
        if by_name:  # pin modules that imported the function by name
            for tm in pin_mods:
                if getattr(tm, attr, None) is original:
                    stack.enter_context(mock.patch.object(tm, attr, mutant))
        caught = _first_failing(pins, fixtures)
    assert caught is not None, f"no pin caught the planted mistake in {module.__name__}.{attr}"
    # and the unmodified oracle is back in place everywhere
    assert getattr(module, attr) is original
    assert all(getattr(tm, attr, original) is not mutant for tm in pin_mods)
