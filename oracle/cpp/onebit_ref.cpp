// Plain, slow C++ CPU implementation of the compressed phase of 1-bit Adam
// and 1-bit LAMB, and of the block-wise INT8 stochastic rounding.
//
// TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
// benchmark's CPU baseline load this library. The GPU library never does, and
// the two share no source, header, table or helper.
//
// It is a second oracle beside the numpy one in this directory. It is written
// from the same passages, as straight loops over elements, so that whole
// full-size buffers can be checked. The numpy oracle and this one must agree
// bit for bit; the tests check that on seeded inputs that reach every branch,
// and they run the numpy oracle's independent pins (brute force with
// fractions, closed forms) on this one too.
//
// Conventions:
// * IEEE binary32 buffers. Each arithmetic operation is one correctly rounded
//   binary32 operation, in the order the formula is written. The file is
//   compiled with -ffp-contract=off and without fast-math, so nothing is
//   fused or reassociated.
// * sign bit = (x >= 0): +0 and -0 count as +1, NaN as -1. Element j of a
//   packed row is bit (j & 31) of 32-bit word (j >> 5).
// * A scale that is a mean of |x| is the exact real mean of the binary32
//   inputs, rounded once to binary32, ties to even.
//
// Sources (page titles and sections):
// * 1-bit Adam article, section 2.1 (error compensation): g' = g + e, the
//   1-bit quantisation of g', the new error e = g' - q.
// * gradient-quantisation tutorial, "1-bit gradient quantisation": the scaled
//   sign mean(|g'|) sign(g') with error feedback (taken per chunk of the
//   fused buffer, one chunk per server).
// * 1-bit Adam article, section 4.1: the periodic error reset and the clamp of
//   the compensated value.
// * 1-bit LAMB page, layer-scaling paragraph: the fixed coefficient k_l
//   multiplies the local momentum before compression and divides the
//   decompressed global momentum.
// * 1-bit LAMB page, experiments paragraph: every server averages its chunk
//   over the n workers, compensates it with its own error and re-compresses.
// * 1-bit LAMB page, algorithm paragraph: frozen v, the gradient rebuilt from
//   two compressed momenta, the fresh variance, the clipped ratio r_t and
//   c_t = c_avg r_t; analysis paragraph: the step uses c_{t-1}, and the
//   carried errors are multiplied by c_{t-1}/c_t.
// * gradient-quantisation tutorial, "FP32 -> INT8", steps 1-3 and the PyTorch
//   example: scale = max|g|/127 per block, stochastic rounding, codes in
//   [-127, 127], dequantisation, error feedback.
// * Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
//   3" (SC'11), section 4: the Philox4x32 bijection with 10 rounds.
// * 1-bit Adam article, section 2.1 and its warmup setting: uncompressed Adam
//   steps first. 1-bit LAMB page, algorithm paragraph: LAMB's layer
//   coefficient and its warmup average c_avg; layer-scaling paragraph: k_l
//   from the average momentum norm at the end of warmup.
//
// Readings where the pages are silent are the ones the numpy oracle states
// (chunk = N/n consecutive elements; ascending worker order in the server
// sum, from +0, then one division by n; clamp = fmin(fmax(x, -clip), clip);
// the layer maximum skips NaN; and so on). Each function repeats the ones it
// uses.

#include <cmath>
#include <cstdint>
#include <cstring>

namespace {

bool sign_bit(float x) { return x >= 0.0f; }

void put_bit(uint32_t* words, int64_t j, bool b) {
    const uint32_t mask = 1u << (j & 31);
    words[j >> 5] = (words[j >> 5] & ~mask) | (b ? mask : 0u);
}

// the scaled sign q = +s for bit 1, -s for bit 0
float scaled_sign(bool b, float s) {
    const float q[2] = {-s, s};
    return q[b ? 1 : 0];
}

bool get_bit(const uint32_t* words, int64_t j) { return (words[j >> 5] >> (j & 31)) & 1u; }

// ---------------------------------------------------------------- exact mean
//
// Every finite binary32 value is an integer multiple of 2^-149:
// |x| = M * 2^(E-1) units for biased exponent E >= 1 (M with its hidden bit)
// and M units for a subnormal (E = 0). The sum of the |x| is therefore an
// integer number of units. It is built in a little-endian array of 32-bit
// limbs; 16 limbs hold 512 bits, far above the 2^31 * 2^128 * 2^149 bound.

constexpr int kLimbs = 16;

struct Big {
    uint32_t w[kLimbs];
};

void big_zero(Big& a) { std::memset(a.w, 0, sizeof a.w); }

// a += v * 2^shift
void big_add_shifted(Big& a, uint64_t v, int shift) {
    int limb = shift / 32;
    const int bit = shift % 32;
    // v < 2^64 shifted by < 32 bits spans at most three limbs
    unsigned __int128 part = (unsigned __int128)v << bit;
    uint64_t carry = 0;
    for (int i = limb; i < kLimbs; ++i) {
        const uint64_t add = (uint64_t)(uint32_t)part;
        part >>= 32;
        const uint64_t s = (uint64_t)a.w[i] + add + carry;
        a.w[i] = (uint32_t)s;
        carry = s >> 32;
        if (part == 0 && carry == 0) break;
    }
}

// a /= d (d > 0), returns the remainder
uint64_t big_div_small(Big& a, uint64_t d) {
    uint64_t rem = 0;
    for (int i = kLimbs - 1; i >= 0; --i) {
        const unsigned __int128 cur = ((unsigned __int128)rem << 32) | a.w[i];
        a.w[i] = (uint32_t)(cur / d);
        rem = (uint64_t)(cur % d);
    }
    return rem;
}

int big_bitlen(const Big& a) {
    for (int i = kLimbs - 1; i >= 0; --i)
        if (a.w[i]) return 32 * i + (32 - __builtin_clz(a.w[i]));
    return 0;
}

bool big_bit(const Big& a, int i) { return (a.w[i / 32] >> (i % 32)) & 1u; }

// the value 0 <= v < 2^24 of bits [lo, lo + 24) (lo may be negative: the
// missing low bits are zero)
uint64_t big_window24(const Big& a, int lo) {
    uint64_t v = 0;
    for (int i = 23; i >= 0; --i) {
        const int b = lo + i;
        v = (v << 1) | (b >= 0 && big_bit(a, b) ? 1u : 0u);
    }
    return v;
}

// binary32 nearest to (Q + r/d) * 2^-149, ties to even, for 0 <= r < d
float round_units(const Big& Q, uint64_t r, uint64_t d) {
    const int p = big_bitlen(Q);
    // keep 24 significant bits, but never finer than one unit (2^-149)
    const int lo = p > 24 ? p - 24 : 0;
    uint64_t top = big_window24(Q, lo);
    // compare what is dropped -- bits [0, lo) of Q plus r/d -- with half of
    // 2^lo units
    int cmp;  // -1 below half, 0 exactly half, +1 above
    if (lo == 0) {
        // dropped part is r/d alone
        const unsigned __int128 twice = (unsigned __int128)r * 2;
        cmp = twice < d ? -1 : (twice == d ? 0 : 1);
    } else if (!big_bit(Q, lo - 1)) {
        cmp = -1;
    } else {
        bool rest = r != 0;
        for (int i = 0; i < lo - 1 && !rest; ++i) rest = big_bit(Q, i);
        cmp = rest ? 1 : 0;
    }
    if (cmp > 0 || (cmp == 0 && (top & 1))) top += 1;
    // top <= 2^24: exact in binary32; the exponent stays in range because a
    // mean of finite values never exceeds the largest of them
    return (float)std::ldexp((double)top, lo - 149);
}

// ------------------------------------------------- exact binary64 sums
//
// A wide unsigned integer (2304 bits) that holds any exact sum of up to 2^31
// non-negative binary64 values, or of squares of binary32 values, in units of
// a fixed power of two; it is rounded once to binary64, ties to even.

constexpr int kWide = 72;

struct Wide {
    uint32_t w[kWide];
};

void wide_zero(Wide& a) { std::memset(a.w, 0, sizeof a.w); }

void wide_add_shifted(Wide& a, uint64_t v, int shift) {
    const int limb = shift / 32;
    unsigned __int128 part = (unsigned __int128)v << (shift % 32);
    uint64_t carry = 0;
    for (int i = limb; i < kWide; ++i) {
        const uint64_t s = (uint64_t)a.w[i] + (uint64_t)(uint32_t)part + carry;
        part >>= 32;
        a.w[i] = (uint32_t)s;
        carry = s >> 32;
        if (part == 0 && carry == 0) break;
    }
}

bool wide_bit(const Wide& a, int i) { return (a.w[i / 32] >> (i % 32)) & 1u; }

// binary64 nearest to a * 2^unit_exp, ties to even (no overflow for the sums
// formed here)
double wide_to_double(const Wide& a, int unit_exp) {
    int p = 0;
    for (int i = kWide - 1; i >= 0; --i)
        if (a.w[i]) {
            p = 32 * i + (32 - __builtin_clz(a.w[i]));
            break;
        }
    if (p == 0) return 0.0;
    // keep 53 significant bits, never finer than 2^-1074
    int lo = p > 53 ? p - 53 : 0;
    if (unit_exp + lo < -1074) lo = -1074 - unit_exp;
    uint64_t top = 0;
    for (int i = p - 1; i >= lo; --i) top = (top << 1) | (wide_bit(a, i) ? 1u : 0u);
    if (lo > 0 && wide_bit(a, lo - 1)) {
        bool rest = false;
        for (int i = 0; i < lo - 1 && !rest; ++i) rest = wide_bit(a, i);
        if (rest || (top & 1)) top += 1;
    }
    return std::ldexp((double)top, unit_exp + lo);
}

// sum of squares of binary32 values, exact, rounded once to binary64. A
// square of M * 2^e (M < 2^24, e >= -149) is M^2 * 2^(2e), an integer number
// of units 2^-298.
// (a NaN gives NaN, else an infinity gives +inf)
double exact_sumsq(const float* x, int64_t n) {
    Wide acc;
    wide_zero(acc);
    bool nan = false, inf = false;
    for (int64_t j = 0; j < n; ++j) {
        uint32_t b;
        std::memcpy(&b, &x[j], 4);
        b &= 0x7FFFFFFFu;
        const uint32_t E = b >> 23;
        if (E == 255) {
            if (b & 0x7FFFFFu) nan = true;
            else inf = true;
            continue;
        }
        const uint64_t M = E ? ((b & 0x7FFFFFu) | 0x800000u) : (b & 0x7FFFFFu);
        const int e = E ? (int)E - 150 : -149;
        if (M) wide_add_shifted(acc, M * M, 2 * e + 298);
    }
    if (nan) return NAN;
    if (inf) return INFINITY;
    return wide_to_double(acc, -298);
}

// sum of non-negative binary64 values, exact, rounded once to binary64
// (units 2^-1074; a NaN gives NaN, else an infinity gives +inf)
double exact_sum_f64(const double* x, int64_t n) {
    Wide acc;
    wide_zero(acc);
    bool nan = false, inf = false;
    for (int64_t j = 0; j < n; ++j) {
        uint64_t b;
        std::memcpy(&b, &x[j], 8);
        const int E = (int)(b >> 52) & 0x7FF;
        if (E == 0x7FF) {
            if (b & 0xFFFFFFFFFFFFFull) nan = true;
            else inf = true;
            continue;
        }
        const uint64_t M = E ? ((b & 0xFFFFFFFFFFFFFull) | (1ull << 52)) : (b & 0xFFFFFFFFFFFFFull);
        if (M) wide_add_shifted(acc, M, E ? E - 1 : 0);
    }
    if (nan) return NAN;
    if (inf) return INFINITY;
    return wide_to_double(acc, -1074);
}

}  // namespace

extern "C" {

// binary32 nearest to mean(|x_0|, ..., |x_{L-1}|), exact, ties to even.
// NaN anywhere gives NaN; otherwise an infinity gives +inf. 1 <= L < 2^39.
float ref_mean_abs(const float* x, int64_t L) {
    bool nan = false, inf = false;
    // per-exponent sums of significands, in 4 interleaved sets (integer sums:
    // the split changes nothing); each below 2^24 * 2^39 = 2^63 for L < 2^39
    uint64_t per_exp[4][256];
    std::memset(per_exp, 0, sizeof per_exp);
    for (int64_t j = 0; j < L; ++j) {
        uint32_t b;
        std::memcpy(&b, &x[j], 4);
        b &= 0x7FFFFFFFu;
        const uint32_t E = b >> 23;
        const uint32_t M = b & 0x7FFFFFu;
        if (E == 255) {
            if (M) nan = true;
            else inf = true;
            continue;
        }
        per_exp[j & 3][E] += E ? (M | 0x800000u) : M;
    }
    if (nan) return NAN;
    if (inf) return INFINITY;
    Big S;
    big_zero(S);
    for (int set = 0; set < 4; ++set)
        for (int E = 0; E < 255; ++E)
            if (per_exp[set][E]) big_add_shifted(S, per_exp[set][E], E ? E - 1 : 0);
    const uint64_t r = big_div_small(S, (uint64_t)L);
    return round_units(S, r, (uint64_t)L);
}

// ------------------------------------------------------------- worker side

// Worker compression of one worker row (length N, n chunks of L = N/n).
//   m         the worker's momentum
//   e_in      its carried error (ignored when reset)
//   k         optional per-element layer coefficient: the row is k * m
//   err_ratio optional per-element factor on the carried error (not on reset)
//   clip      clamp bound; clip <= 0 or infinite turns the clamp off
//   unit      scale 1 instead of the chunk mean (unscaled sign)
// Outputs: gc (the compensated, clamped values), e_out (new error; may alias
// e_in), bits (N/32 words), s (n scales).
int ref_worker_compress_row(const float* m, const float* e_in, const float* k,
                            const float* err_ratio, int64_t N, int32_t n, float clip,
                            int32_t reset, int32_t unit, float* gc, float* e_out, uint32_t* bits,
                            float* s) {
    if (n < 1 || N % (64 * (int64_t)n)) return 1;
    const int64_t L = N / n;
    const bool clamp = clip > 0.0f && !std::isinf(clip);
    for (int64_t j = 0; j < N; ++j) {
        float e = 0.0f;
        if (!reset) {
            e = e_in[j];
            if (err_ratio) e = err_ratio[j] * e;
        }
        const float mk = k ? k[j] * m[j] : m[j];
        float g = mk + e;
        if (clamp) g = std::fmin(std::fmax(g, -clip), clip);
        gc[j] = g;
        put_bit(bits, j, sign_bit(g));
    }
    for (int32_t c = 0; c < n; ++c) {
        const float sc = unit ? 1.0f : ref_mean_abs(gc + c * L, L);
        s[c] = sc;
        for (int64_t j = c * L; j < (c + 1) * L; ++j) e_out[j] = gc[j] - scaled_sign(sign_bit(gc[j]), sc);
    }
    return 0;
}

// A worker's momentum formed from its gradient and the previous global
// momentum: fl(fl(beta1 mbar) + fl(fl(1 - beta1) g)) (1-bit Adam article,
// section 2.1; mbar is the same on every worker).
void ref_local_momentum(const float* g, const float* mbar, float beta1, int64_t N, float* out) {
    const float omb1 = 1.0f - beta1;
    for (int64_t j = 0; j < N; ++j) {
        const float a = beta1 * mbar[j];
        const float b = omb1 * g[j];
        out[j] = a + b;
    }
}

// ------------------------------------------------------------- server side

// Server side of chunk c (elements [cL, (c+1)L) of the buffer, L = N/n).
//   wbits  worker sign words, [n][N/32] row-major
//   ws     worker scales, [n][n] row-major (ws[i*n + c]: worker i, chunk c)
//   E_in   the server error over the whole buffer (ignored when reset)
// The average sums +-ws[i][c] over workers i = 0, 1, ..., n-1 in binary32
// from +0, then divides by n once. Writes, for chunk c only: avg, g2 (the
// compensated value), E_out (may alias E_in), sbits, and S[c].
int ref_server_chunk(const uint32_t* wbits, const float* ws, const float* E_in,
                     const float* err_ratio, int64_t N, int32_t n, int32_t c, int32_t reset,
                     int32_t unit, float* avg, float* g2, float* E_out, uint32_t* sbits,
                     float* S) {
    if (n < 1 || N % (64 * (int64_t)n) || c < 0 || c >= n) return 1;
    const int64_t L = N / n, W = N / 32;
    const float nf = (float)n;
    for (int64_t j = c * L; j < (c + 1) * L; ++j) {
        float acc = 0.0f;
        for (int32_t i = 0; i < n; ++i) {
            const float si = ws[(int64_t)i * n + c];
            acc = acc + scaled_sign(get_bit(wbits + (int64_t)i * W, j), si);
        }
        const float a = acc / nf;
        float e = 0.0f;
        if (!reset) {
            e = E_in[j];
            if (err_ratio) e = err_ratio[j] * e;
        }
        avg[j] = a;
        g2[j] = a + e;
        put_bit(sbits, j, sign_bit(g2[j]));
    }
    const float sc = unit ? 1.0f : ref_mean_abs(g2 + c * L, L);
    S[c] = sc;
    for (int64_t j = c * L; j < (c + 1) * L; ++j) E_out[j] = g2[j] - scaled_sign(sign_bit(g2[j]), sc);
    return 0;
}

// The global momentum every worker rebuilds: +-S[c] on chunk c, divided by
// k[j] when k is given.
int ref_decompress(const uint32_t* sbits, const float* S, const float* k, int64_t N, int32_t n,
                   float* out) {
    if (n < 1 || N % (64 * (int64_t)n)) return 1;
    const int64_t L = N / n;
    for (int32_t c = 0; c < n; ++c) {
        for (int64_t j = c * L; j < (c + 1) * L; ++j) {
            float v = scaled_sign(get_bit(sbits, j), S[c]);
            if (k) v = v / k[j];
            out[j] = v;
        }
    }
    return 0;
}

// ------------------------------------------------------- parameter steps

// Adam with frozen v: x <- x - lr * (m / (sqrt(v) + eps)) (1-bit Adam
// article, section 2.1; eps outside the root, no bias correction).
void ref_adam_frozen_step(float* x, const float* m, const float* v, int64_t N, float lr,
                          float eps) {
    for (int64_t j = 0; j < N; ++j) {
        const float den = std::sqrt(v[j]) + eps;
        const float upd = m[j] / den;
        x[j] = x[j] - lr * upd;
    }
}

// One 1-bit LAMB step with frozen v_tw over layers [seg_off[l], seg_off[l+1]).
//   g_t = (m - beta1 m_prev) / (1 - beta1); v_f <- beta2 v_f + (1 - beta2) g^2;
//   R_l = max over the layer of v_tw / v_f, skipping NaN (+0 above -0);
//   r_l = clip(clip(R_l, (1-thr) r_prev, (1+thr) r_prev), r_min, r_max),
//   r_prev where the layer has no valid ratio; c_l = c_avg r_l;
//   x <- x - (lr c) * (m / (sqrt(v_tw) + eps)) with c = c_prev (or c_t when
//   use_c_t); rho_l = c_prev / c_l.
// Updates x and v_f in place; writes R, r, c and rho per layer.
int ref_lamb_frozen_step(float* x, const float* m, const float* m_prev, float* v_f,
                         const float* v_tw, const int64_t* seg_off, int32_t n_seg,
                         const float* c_avg, const float* r_prev, const float* c_prev, float lr,
                         float eps, float beta1, float beta2, float thr, float r_min, float r_max,
                         int32_t use_c_t, float* R, float* r, float* c, float* rho) {
    if (n_seg < 1) return 1;
    const float omb1 = 1.0f - beta1, omb2 = 1.0f - beta2;
    for (int32_t l = 0; l < n_seg; ++l) {
        bool have = false;
        float best = 0.0f;
        for (int64_t j = seg_off[l]; j < seg_off[l + 1]; ++j) {
            const float num = m[j] - beta1 * m_prev[j];
            const float g = num / omb1;
            const float vn = beta2 * v_f[j] + omb2 * (g * g);
            v_f[j] = vn;
            const float q = v_tw[j] / vn;
            if (std::isnan(q)) continue;
            if (!have || q > best || (q == 0.0f && best == 0.0f && !std::signbit(q))) best = q;
            have = true;
        }
        R[l] = have ? best : NAN;
        const float Rl = have ? best : r_prev[l];
        const float lo = (1.0f - thr) * r_prev[l];
        const float hi = (1.0f + thr) * r_prev[l];
        float rl = std::fmin(std::fmax(Rl, lo), hi);
        rl = std::fmin(std::fmax(rl, r_min), r_max);
        r[l] = rl;
        c[l] = c_avg[l] * rl;
        rho[l] = c_prev[l] / c[l];
        const float step = lr * (use_c_t ? c[l] : c_prev[l]);
        for (int64_t j = seg_off[l]; j < seg_off[l + 1]; ++j) {
            const float den = std::sqrt(v_tw[j]) + eps;
            const float upd = m[j] / den;
            x[j] = x[j] - step * upd;
        }
    }
    return 0;
}

// ---------------------------------------------------------------- Philox

// Philox4x32-10: 10 rounds of the S-box on a 4-word counter with a 2-word key.
// Each round multiplies words 0 and 2 by the two round multipliers; the new
// words are (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)).
// The key is bumped by the two Weyl constants before every round after the
// first.
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t p0 = M0 * x0, p1 = M1 * x2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        x0 = n0;
        x1 = n1;
        x2 = n2;
        x3 = n3;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

// The uniform of element J: counter (J/4 low word, J/4 high word, step, 0),
// key (seed low word, seed high word); word J mod 4, top 24 bits, times 2^-24.
float ref_uniform(uint64_t J, uint64_t seed, uint32_t step) {
    const uint64_t blk = J >> 2;
    const uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), step, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    ref_philox4x32_10(ctr, key, w);
    return (float)(w[J & 3] >> 8) * 0x1p-24f;
}

// ------------------------------------------------------------------ INT8

// Block-wise INT8 quantisation of g' = g + e (g alone when e is NULL).
//   block   elements per scale (0: the whole tensor); N a multiple of it
//   rounding 0: stochastic (floor(x) + [u < x - floor(x)]), 1: nearest,
//            halves away from zero
//   J0      global index of element 0 (the Philox counter of element j is
//           J0 + j)
// Per block: M = largest |g'| skipping NaN (0 if none); scale = M / 127.
// Per element: x = g' / scale; code clamped to [-127, 127] with fmin/fmax;
// scale 0 gives code 0 and dequantised 0; deq = code * scale;
// e_out = g' - deq. Outputs: codes, scales (N/block), deq, e_out (each but
// codes and scales may be NULL).
int ref_int8_quantize(const float* g, const float* e, int64_t N, int64_t block, int32_t rounding,
                      uint64_t seed, uint32_t step, int64_t J0, int8_t* codes, float* scales,
                      float* deq, float* e_out) {
    if (block == 0) block = N;
    if (block <= 0 || N % block) return 1;
    for (int64_t b0 = 0; b0 < N; b0 += block) {
        float M = 0.0f;
        for (int64_t j = b0; j < b0 + block; ++j) {
            const float gc = e ? g[j] + e[j] : g[j];
            const float a = std::fabs(gc);
            if (!std::isnan(a) && a > M) M = a;
        }
        const float sc = M / 127.0f;
        scales[b0 / block] = sc;
        for (int64_t j = b0; j < b0 + block; ++j) {
            const float gc = e ? g[j] + e[j] : g[j];
            float q;
            if (sc == 0.0f) {
                q = 0.0f;
            } else {
                const float x = gc / sc;
                if (rounding == 1) {
                    const float t = std::trunc(x);
                    const float frac = std::fabs(x - t);
                    q = frac >= 0.5f ? t + std::copysign(1.0f, x) : t;
                } else {
                    const float f = std::floor(x);
                    const float p = x - f;
                    const float u = ref_uniform((uint64_t)(J0 + j), seed, step);
                    q = f + (u < p ? 1.0f : 0.0f);
                }
                q = std::fmin(std::fmax(q, -127.0f), 127.0f);
            }
            const float dq = sc == 0.0f ? 0.0f : q * sc;
            codes[j] = (int8_t)q;
            if (deq) deq[j] = dq;
            if (e_out) e_out[j] = gc - dq;
        }
    }
    return 0;
}

// ---------------------------------------------------------------- warmup
//
// Readings where the pages are silent: no bias correction and no weight
// decay; u = m / (sqrt(v) + eps) from the new moments; LAMB's coefficient is
// c_l = ||x_l|| / ||u_l|| with x before the update, 1 when either norm is 0,
// the squared norms exact sums rounded once to binary64 and the ratio
// sqrt(Sx) / sqrt(Su) in binary64 rounded once to binary32; c_avg starts at
// the first coefficient, then c_avg <- beta_c c_avg + (1 - beta_c) c; k_l =
// (mean over layers with a_l > 0 of a_l) / a_l with the RMS
// a_l = sqrt(||m_l||^2 / d_l) in binary64, 1 for a layer with a_l = 0.

namespace {

void moments(float& m, float& v, float g, float beta1, float beta2) {
    const float omb1 = 1.0f - beta1, omb2 = 1.0f - beta2;
    const float m1 = beta1 * m;
    const float m2 = omb1 * g;
    const float v1 = beta2 * v;
    const float v2 = omb2 * (g * g);
    m = m1 + m2;
    v = v1 + v2;
}

float direction(float m, float v, float eps) {
    const float den = std::sqrt(v) + eps;
    return m / den;
}

}  // namespace

// The exact sums on their own, for pins against an independent exact sum.
double ref_exact_sumsq(const float* x, int64_t n) { return exact_sumsq(x, n); }
double ref_exact_sum_f64(const double* x, int64_t n) { return exact_sum_f64(x, n); }

// One uncompressed Adam step on the averaged gradient g (x, m, v in place).
void ref_adam_warmup_step(float* x, float* m, float* v, const float* g, int64_t N, float lr,
                          float eps, float beta1, float beta2) {
    for (int64_t j = 0; j < N; ++j) {
        moments(m[j], v[j], g[j], beta1, beta2);
        const float u = direction(m[j], v[j], eps);
        x[j] = x[j] - lr * u;
    }
}

// One uncompressed LAMB step over layers [seg_off[l], seg_off[l+1]) (x, m, v
// in place); writes each layer's coefficient c and advances c_avg (c_avg_in
// NULL: the first step, which starts the average at c).
int ref_lamb_warmup_step(float* x, float* m, float* v, const float* g, const int64_t* seg_off,
                         int32_t n_seg, float lr, float eps, float beta1, float beta2,
                         const float* c_avg_in, float beta_c, float* c, float* c_avg_out) {
    if (n_seg < 1) return 1;
    const float ombc = 1.0f - beta_c;
    for (int32_t l = 0; l < n_seg; ++l) {
        const int64_t a = seg_off[l], b = seg_off[l + 1];
        if (b < a) return 1;
        float* u = new float[b > a ? b - a : 1];
        for (int64_t j = a; j < b; ++j) {
            moments(m[j], v[j], g[j], beta1, beta2);
            u[j - a] = direction(m[j], v[j], eps);
        }
        const double sx = exact_sumsq(x + a, b - a);
        const double su = exact_sumsq(u, b - a);
        const float cl = (sx == 0.0 || su == 0.0) ? 1.0f : (float)(std::sqrt(sx) / std::sqrt(su));
        c[l] = cl;
        const float step = lr * cl;
        for (int64_t j = a; j < b; ++j) x[j] = x[j] - step * u[j - a];
        delete[] u;
        if (c_avg_in) {
            const float p = beta_c * c_avg_in[l];
            const float q = ombc * cl;
            c_avg_out[l] = p + q;
        } else {
            c_avg_out[l] = cl;
        }
    }
    return 0;
}

// k_l of every layer from the momentum m at the end of warmup.
int ref_momentum_scale(const float* m, const int64_t* seg_off, int32_t n_seg, float* k) {
    if (n_seg < 1) return 1;
    double* rms = new double[n_seg];
    double* valid = new double[n_seg];
    int32_t nv = 0;
    for (int32_t l = 0; l < n_seg; ++l) {
        const int64_t a = seg_off[l], b = seg_off[l + 1];
        rms[l] = 0.0;
        if (b > a) rms[l] = std::sqrt(exact_sumsq(m + a, b - a) / (double)(b - a));
        if (rms[l] > 0.0) valid[nv++] = rms[l];
    }
    const double mean = nv ? exact_sum_f64(valid, nv) / (double)nv : 0.0;
    for (int32_t l = 0; l < n_seg; ++l) k[l] = rms[l] > 0.0 ? (float)(mean / rms[l]) : 1.0f;
    delete[] rms;
    delete[] valid;
    return 0;
}

}  // extern "C"
