// Warmup phase and the transition to compressed training.
//
// Adam warmup (1-bit Adam article, section 2.1 recursions; its configuration
// block runs the first steps without quantisation), one streaming pass:
//   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;  x -= lr * (m / (sqrtf(v)+eps)).
//
// LAMB warmup (1-bit LAMB page: LAMB's layer coefficient c and its warmup
// moving average c_avg), two passes around a per-layer finalize:
//   pass 1: m, v as above, u = m / (sqrtf(v)+eps); per layer Sx = sum x^2
//           (x before the step) and Su = sum u^2 in binary64;
//   finalize: c = (Sx == 0 || Su == 0) ? 1 : float(sqrt(Sx) / sqrt(Su)),
//           c_avg = first ? c : b_c c_avg + (1-b_c) c;
//   pass 2: u again from the stored m and v, x -= (lr c_l) u.
//
// Momentum scale (1-bit LAMB page, layer-scaling paragraph): per layer the
// RMS a_l = sqrt(sum m^2 / d_l) in binary64, k_l = mean(a) / a_l over layers
// with a_l > 0, else 1.
//
// The squared norms are defined as exact sums rounded once to binary64.  The
// passes above sum them in binary64 in a fixed order, with a relative error
// below gamma_D for D additions per term (the terms are exact squares, all
// non-negative).  The binary32 result (c_l, k_l) is certified when every
// value within the resulting error bound rounds to the same binary32 value,
// so it equals the one the exact sums give.  Where that fails (a result
// within about D 2^-53 of a binary32 rounding boundary, or exactly on one),
// an exact pass recomputes the layer's sums: every square is an integer
// number of units 2^-298, accumulated per exponent in 64-bit LDS counters,
// folded per workgroup into a 640-bit integer, summed per layer and rounded
// once to binary64; c_l or k_l is then computed from those sums exactly as
// the definition states.  For k_l the mean over layers needs every layer's
// RMS, so all layers take the exact path together, and the mean of the RMS
// values is an exact sum too.
//
// Layout of the layer passes: every workgroup lies inside one layer (a plan
// kernel gives each layer ceil(quads / 1024) workgroups of 4 tiles), so each
// workgroup reduces into a slot of its own and a layer's slots are summed in
// a fixed order: the binary64 norms do not depend on scheduling.  Layer
// offsets may take any value: a layer starting or ending inside a float4
// masks the foreign elements of that quad and stores its own elements one by
// one, so neighbouring layers never write the same element.  Offsets are
// clamped to [0, N] and to non-decreasing order before use, so a malformed
// table gives wrong layers but no access outside the buffers.
#include "common.h"

namespace onebit {

namespace {

constexpr int64_t kSpan = (int64_t)kLambTiles * kTile;  // elements (quads x 4) per workgroup

__device__ __forceinline__ int64_t layer_wgs(int64_t a, int64_t b) {
    if (b <= a) return 0;
    const int64_t qa = a & ~(int64_t)3, qb = (b + 3) & ~(int64_t)3;
    return (qb - qa + kSpan - 1) / kSpan;
}

// offsets of layer l clamped to 0 <= lo <= hi <= N
__device__ __forceinline__ void layer_bounds(const int64_t* __restrict__ seg_off, int l, int64_t N,
                                             int64_t& lo, int64_t& hi) {
    lo = seg_off[l];
    hi = seg_off[l + 1];
    lo = lo < 0 ? 0 : (lo > N ? N : lo);
    hi = hi < lo ? lo : (hi > N ? N : hi);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Fixed-order sum of a double over the workgroup (wave butterflies, then the
// 4 wave sums in order); the result is valid in thread 0.
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
    v = wave_sum_f64(v);
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
        s = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) s += red[w];
    }
    return s;
}

// Sum over the workgroup of part[w].x (and .y) for w in [w0, w1), in a fixed
// order: each thread adds the slots w0 + tid + 256 q in ascending q (8 loads
// in flight), then block_sum_f64; valid in thread 0.
__device__ __forceinline__ double2 slot_sum(const double2* __restrict__ part, int64_t w0,
                                            int64_t w1, double* red) {
    constexpr int kBatch = 8;
    double sx = 0.0, sy = 0.0;
    for (int64_t wb = w0; wb < w1; wb += (int64_t)kThreads * kBatch) {
        double2 p[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t w = wb + (int64_t)q * kThreads + threadIdx.x;
            p[q] = w < w1 ? part[w] : make_double2(0.0, 0.0);
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            sx += p[q].x;
            sy += p[q].y;
        }
    }
    const double tx = block_sum_f64(sx, red);
    __syncthreads();  // red is reused
    const double ty = block_sum_f64(sy, red);
    return make_double2(tx, ty);
}

// The workgroup's layer and element range; false for the spare workgroups of
// the launch (the grid is an upper bound on the plan's total).
struct WgRange {
    int layer;
    int64_t lo, hi;   // elements of the layer
    int64_t base;     // first quad (element index, multiple of 4) of this workgroup
    int64_t qend;     // end of this workgroup's quads
};

__device__ __forceinline__ bool wg_range(const int64_t* __restrict__ seg_off,
                                         const int64_t* __restrict__ wg_first, int32_t n_seg,
                                         int64_t N, WgRange& r) {
    const int64_t w = blockIdx.x;
    if (w >= wg_first[n_seg]) return false;
    const int l = find_segment(wg_first, n_seg, w);
    r.layer = l;
    layer_bounds(seg_off, l, N, r.lo, r.hi);
    r.base = (r.lo & ~(int64_t)3) + (w - wg_first[l]) * kSpan;
    const int64_t qb = (r.hi + 3) & ~(int64_t)3;
    r.qend = r.base + kSpan < qb ? r.base + kSpan : qb;
    return true;
}

// Store the elements of quad J that lie in [lo, hi): whole float4 when the
// quad is inside, element by element at a layer edge.
__device__ __forceinline__ void store_quad(float* p, int64_t J, int64_t lo, int64_t hi,
                                           const float o[4]) {
    if (J >= lo && J + 4 <= hi) {
        const f4 ov = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(ov, reinterpret_cast<f4*>(p + J));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (J + k >= lo && J + k < hi) p[J + k] = o[k];
    }
}

// Additions each term of a layer's binary64 norm passes through: 16 per
// thread in the workgroup pass, 6 + 3 in its block sum, then in slot_sum 8
// per batch of 2048 slots per thread and 6 + 3 again.
__device__ __forceinline__ int64_t norm_depth(int64_t slots) {
    return 16 + 9 + 8 * ((slots + 2047) / 2048) + 9;
}

// Every value of [q (1 - delta), q (1 + delta)] rounds to the same binary32
// (float conversion is monotone; the slack added to delta by the callers
// covers the rounding of the two products).
__device__ __forceinline__ bool certified(double q, double delta) {
    return (float)(q * (1.0 - delta)) == (float)(q * (1.0 + delta));
}

// ------------------------------------------------------------- exact sums
constexpr int kSqBins = 531;  // squares in units 2^-298: bins 2^0 .. 2^530

// x^2 into per-exponent LDS counters: x = M 2^e (M < 2^24, e >= -149) gives
// M^2 2^(2e), i.e. (M^2 mod 2^24) units at bin 2e + 298 and (M^2 >> 24)
// units at bin 2e + 322.  A workgroup adds at most 2 * 4096 values below
// 2^24 to a counter.  Non-finite values never reach the exact path.
__device__ __forceinline__ void bin_square(unsigned long long* bins, float x) {
    const uint32_t b = __float_as_uint(x) & 0x7FFFFFFFu;
    const uint32_t E = b >> 23;
    if (E == 255u) return;
    const uint64_t M = E ? (uint64_t)((b & 0x7FFFFFu) | 0x800000u) : (uint64_t)(b & 0x7FFFFFu);
    if (M == 0) return;
    const int e2 = 2 * (E ? (int)E - 150 : -149) + 298;
    const uint64_t sq = M * M;
    atomicAdd(&bins[e2], (unsigned long long)(sq & 0xFFFFFFull));
    const uint64_t hi = sq >> 24;
    if (hi) atomicAdd(&bins[e2 + 24], (unsigned long long)hi);
}

// limb[0..LIMBS) += v * 2^shift, v < 2^62 (the sum never leaves LIMBS limbs)
template <int LIMBS>
__device__ void limbs_add_shifted(uint64_t* limb, uint64_t v, int shift) {
    int idx = shift >> 6;
    const int off = shift & 63;
    const uint64_t lo = v << off;
    uint64_t add = off ? (v >> (64 - off)) : 0;  // the part above limb idx
    uint64_t t = limb[idx] + lo;
    add += t < lo;
    limb[idx] = t;
    for (++idx; add && idx < LIMBS; ++idx) {
        t = limb[idx] + add;
        add = t < add;
        limb[idx] = t;
    }
}

// bits [pos, pos + 53) of the integer (pos >= 0)
template <int LIMBS>
__device__ uint64_t limbs_bits53(const uint64_t* limb, int pos) {
    const int idx = pos >> 6;
    const int off = pos & 63;
    uint64_t w = limb[idx] >> off;
    if (off && idx + 1 < LIMBS) w |= limb[idx + 1] << (64 - off);
    return w & ((1ull << 53) - 1);
}

template <int LIMBS>
__device__ bool limbs_bit(const uint64_t* limb, int pos) {
    return (limb[pos >> 6] >> (pos & 63)) & 1ull;
}

template <int LIMBS>
__device__ bool limbs_any_below(const uint64_t* limb, int pos) {
    for (int k = 0; k < (pos >> 6); ++k)
        if (limb[k]) return true;
    const int off = pos & 63;
    return off && (limb[pos >> 6] & ((1ull << off) - 1));
}

// The binary64 nearest to (integer) * 2^unit_exp, ties to even; the results
// formed here are normal numbers.
template <int LIMBS>
__device__ double limbs_to_double(const uint64_t* limb, int unit_exp) {
    int top = LIMBS - 1;
    while (top >= 0 && limb[top] == 0) --top;
    if (top < 0) return 0.0;
    const int p = 64 * top + (64 - __clzll(limb[top]));  // significant bits
    if (p <= 53) return ldexp((double)limb[0], unit_exp);
    const int lo = p - 53;
    uint64_t mnt = limbs_bits53<LIMBS>(limb, lo);
    if (limbs_bit<LIMBS>(limb, lo - 1) &&
        (limbs_any_below<LIMBS>(limb, lo - 1) || (mnt & 1ull)))
        ++mnt;  // 2^53 at most: still exact as a double
    return ldexp((double)mnt, unit_exp + lo);
}

// Exact sum of the layer's per-workgroup integers (slot s of workgroups
// [w0, w1)), rounded once to binary64: thread i < kExactLimbs adds limb i
// of every slot with a 128-bit counter, thread 0 propagates the carries.
// Valid in thread 0; every thread of the block must call it.
__device__ double exact_layer_sum(const uint64_t* __restrict__ slots, int64_t w0, int64_t w1,
                                  int s, uint64_t* lo_s, uint64_t* hi_s) {
    if ((int)threadIdx.x < kExactLimbs) {
        const int i = threadIdx.x;
        uint64_t lo = 0, hi = 0;
        for (int64_t w = w0; w < w1; ++w) {
            const uint64_t v = slots[(w * 2 + s) * kExactLimbs + i];
            lo += v;
            hi += lo < v;
        }
        lo_s[i] = lo;
        hi_s[i] = hi;
    }
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        uint64_t limb[kExactLimbs];
        uint64_t carry = 0;
        for (int i = 0; i < kExactLimbs; ++i) {
            const uint64_t t = lo_s[i] + carry;
            carry = hi_s[i] + (t < carry);
            limb[i] = t;
        }
        r = limbs_to_double<kExactLimbs>(limb, -298);
    }
    __syncthreads();  // lo_s / hi_s are reused
    return r;
}

}  // namespace

// wg_first[l] = number of workgroups of layers 0 .. l-1 (l = 0 .. n_seg), by
// one workgroup: each thread sums a contiguous run of layers, thread 0 scans
// the 256 run totals, then each thread writes its run's prefixes.
__global__ __launch_bounds__(kThreads) void layer_plan_kernel(const int64_t* __restrict__ seg_off,
                                                              int32_t n_seg, int64_t N,
                                                              int64_t* __restrict__ wg_first,
                                                              int32_t* __restrict__ need_any) {
    __shared__ int64_t part[kThreads];
    if (threadIdx.x == 0) *need_any = 0;  // set again by a layer that needs the exact path
    const int per = (n_seg + kThreads - 1) / kThreads;
    const int l0 = threadIdx.x * per;
    const int l1 = l0 + per < n_seg ? l0 + per : n_seg;
    int64_t s = 0;
    int64_t lo, hi;
    for (int l = l0; l < l1; ++l) {
        layer_bounds(seg_off, l, N, lo, hi);
        s += layer_wgs(lo, hi);
    }
    part[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t acc = 0;
        for (int i = 0; i < kThreads; ++i) {
            const int64_t v = part[i];
            part[i] = acc;
            acc += v;
        }
    }
    __syncthreads();
    int64_t acc = part[threadIdx.x];
    for (int l = l0; l < l1; ++l) {
        wg_first[l] = acc;
        layer_bounds(seg_off, l, N, lo, hi);
        acc += layer_wgs(lo, hi);
    }
    if (threadIdx.x == kThreads - 1) wg_first[n_seg] = acc;  // the last run ends at the total
}

__global__ __launch_bounds__(kThreads) void warmup_adam_kernel(float* __restrict__ x,
                                                               float* __restrict__ m,
                                                               float* __restrict__ v,
                                                               const float* __restrict__ g,
                                                               int64_t N, float lr, float eps,
                                                               float b1, float b2) {
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    const int64_t j0 = (int64_t)blockIdx.x * kMaxIters * kTile + 4 * (int64_t)threadIdx.x;
    f4 xv[kMaxIters], mv[kMaxIters], vv[kMaxIters], gv[kMaxIters];
#pragma unroll
    for (int u = 0; u < kMaxIters; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j < N) {
            xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x + j));
            mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + j));
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + j));
            gv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(g + j));
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxIters; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j >= N) break;
        const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        const float ms[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
        const float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        const float gs[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
        float xo[4], mo[4], vo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mo[k] = b1 * ms[k] + omb1 * gs[k];
            vo[k] = b2 * vs[k] + omb2 * (gs[k] * gs[k]);
            const float den = sqrtf(vo[k]) + eps;
            const float upd = mo[k] / den;
            xo[k] = xs[k] - lr * upd;
        }
        __builtin_nontemporal_store(f4{xo[0], xo[1], xo[2], xo[3]}, reinterpret_cast<f4*>(x + j));
        __builtin_nontemporal_store(f4{mo[0], mo[1], mo[2], mo[3]}, reinterpret_cast<f4*>(m + j));
        __builtin_nontemporal_store(f4{vo[0], vo[1], vo[2], vo[3]}, reinterpret_cast<f4*>(v + j));
    }
}

// LAMB warmup pass 1: moments, and the layer's sum x^2 / sum u^2 of this
// workgroup into part[blockIdx.x] = (Sx, Su).
__global__ __launch_bounds__(kThreads) void warmup_lamb_moments_kernel(
    const float* __restrict__ x, float* __restrict__ m, float* __restrict__ v,
    const float* __restrict__ g, const int64_t* __restrict__ seg_off,
    const int64_t* __restrict__ wg_first, int32_t n_seg, int64_t N, double2* __restrict__ part,
    float eps, float b1, float b2) {
    __shared__ double red[kThreads / 64];
    WgRange r;
    if (!wg_range(seg_off, wg_first, n_seg, N, r)) return;  // workgroup-uniform
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    f4 xv[kLambTiles], mv[kLambTiles], vv[kLambTiles], gv[kLambTiles];
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t J = r.base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
        if (J < r.qend) {
            xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x + J));
            mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + J));
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + J));
            gv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(g + J));
        }
    }
    double sx = 0.0, su = 0.0;
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t J = r.base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
        if (J >= r.qend) break;
        const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        const float ms[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
        const float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        const float gs[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
        float mo[4], vo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mo[k] = b1 * ms[k] + omb1 * gs[k];
            vo[k] = b2 * vs[k] + omb2 * (gs[k] * gs[k]);
            const float den = sqrtf(vo[k]) + eps;
            const float uk = mo[k] / den;
            if (J + k >= r.lo && J + k < r.hi) {
                sx += (double)xs[k] * (double)xs[k];
                su += (double)uk * (double)uk;
            }
        }
        store_quad(m, J, r.lo, r.hi, mo);
        store_quad(v, J, r.lo, r.hi, vo);
    }
    const double tx = block_sum_f64(sx, red);
    __syncthreads();  // red is reused
    const double tu = block_sum_f64(su, red);
    if (threadIdx.x == 0) part[blockIdx.x] = make_double2(tx, tu);
}

// One workgroup per layer: the layer's slots in a fixed order, c and the
// moving average, unless c cannot be certified: then the layer is marked for
// the exact path, which writes c and the average instead.
//
// Certification: each binary64 sum is within gamma_D (D = norm_depth) of the
// exact sum, so q = sqrt(Sx) / sqrt(Su) (correctly rounded square roots and
// division) is within (D + 3) u of the exact ratio, and the ratio the exact
// sums rounded to binary64 give is within 4 u of it (u = 2^-53).  The
// interval q (1 -+ (D + 20) u) therefore holds that value.  A zero sum is
// exact (no square of a binary32 value underflows binary64), and infinite
// or NaN sums are what the exact sums give as well.
__global__ __launch_bounds__(kThreads) void warmup_lamb_finalize_kernel(
    const double2* __restrict__ part, const int64_t* __restrict__ wg_first, int32_t n_seg,
    int64_t n_wg, float* __restrict__ c_out, float* __restrict__ c_avg, float b_c,
    int32_t first, int32_t* __restrict__ need) {
    __shared__ double red[kThreads / 64];
    const int l = blockIdx.x;
    if (l >= n_seg) return;
    const int64_t w1 = wg_first[l + 1] < n_wg ? wg_first[l + 1] : n_wg;
    const double2 t = slot_sum(part, wg_first[l], w1, red);
    if (threadIdx.x != 0) return;
    const double sx = t.x, su = t.y;
    float c = 1.0f;
    bool ok = true;
    if (!(sx == 0.0 || su == 0.0)) {
        const double q = sqrt(sx) / sqrt(su);
        c = (float)q;
        if (isfinite(sx) && isfinite(su)) {
            const int64_t d = norm_depth(w1 - wg_first[l]);
            ok = certified(q, (double)(d + 20) * 0x1p-53);
        }
    }
    need[l] = ok ? 0 : 1;
    if (!ok) {
        atomicOr(&need[n_seg], 1);
        return;
    }
    c_out[l] = c;
    c_avg[l] = first ? c : b_c * c_avg[l] + (1.0f - b_c) * c;
}

// Exact pass over the workgroups of the layers marked in need (skipped at
// once when none is: need[n_seg] == 0).  A fixed grid walks the plan's
// workgroups; for each one of a marked layer it bins the squares of its
// elements (LAMB: x and u = m / (sqrtf(v) + eps) from the stored moments, as
// the first pass formed them; else m) and stores their exact sums as
// integers in units 2^-298 in the workgroup's slots.
template <bool LAMB>
__global__ __launch_bounds__(kThreads) void exact_squares_kernel(
    const float* __restrict__ x, const float* __restrict__ m, const float* __restrict__ v,
    const int64_t* __restrict__ seg_off, const int64_t* __restrict__ wg_first, int32_t n_seg,
    int64_t N, float eps, const int32_t* __restrict__ need, uint64_t* __restrict__ slots) {
    constexpr int kSums = LAMB ? 2 : 1;
    __shared__ unsigned long long bins[kSums][kSqBins];
    if (need[n_seg] == 0) return;
    const int64_t total = wg_first[n_seg];
    for (int64_t w = blockIdx.x; w < total; w += gridDim.x) {
        const int l = find_segment(wg_first, n_seg, w);
        if (!need[l]) continue;  // workgroup-uniform
        int64_t lo, hi;
        layer_bounds(seg_off, l, N, lo, hi);
        const int64_t base = (lo & ~(int64_t)3) + (w - wg_first[l]) * kSpan;
        const int64_t qb = (hi + 3) & ~(int64_t)3;
        const int64_t qend = base + kSpan < qb ? base + kSpan : qb;
        for (int k = threadIdx.x; k < kSums * kSqBins; k += kThreads) (&bins[0][0])[k] = 0ull;
        __syncthreads();
        for (int u = 0; u < kLambTiles; ++u) {
            const int64_t J = base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
            if (J >= qend) break;
            const f4 mv = *reinterpret_cast<const f4*>(m + J);
            const float ms[4] = {mv.x, mv.y, mv.z, mv.w};
            if (LAMB) {
                const f4 xv = *reinterpret_cast<const f4*>(x + J);
                const f4 vv = *reinterpret_cast<const f4*>(v + J);
                const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
                const float vs[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (J + k < lo || J + k >= hi) continue;
                    const float den = sqrtf(vs[k]) + eps;
                    bin_square(bins[0], xs[k]);
                    bin_square(bins[kSums - 1], ms[k] / den);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (J + k >= lo && J + k < hi) bin_square(bins[0], ms[k]);
            }
        }
        __syncthreads();
        if ((int)threadIdx.x < kSums) {
            const int sidx = threadIdx.x;
            uint64_t limb[kExactLimbs];
            for (int i = 0; i < kExactLimbs; ++i) limb[i] = 0;
            for (int b = 0; b < kSqBins; ++b)
                if (bins[sidx][b]) limbs_add_shifted<kExactLimbs>(limb, bins[sidx][b], b);
            uint64_t* out = slots + (w * 2 + sidx) * kExactLimbs;
            for (int i = 0; i < kExactLimbs; ++i) out[i] = limb[i];
        }
        __syncthreads();  // bins are cleared for the next workgroup
    }
}

// Exact path of the LAMB coefficient, one workgroup per marked layer: the
// exact sums rounded once to binary64, then c and the average as above.
__global__ __launch_bounds__(kThreads) void warmup_lamb_exact_kernel(
    const uint64_t* __restrict__ slots, const int64_t* __restrict__ wg_first, int32_t n_seg,
    const int32_t* __restrict__ need, float* __restrict__ c_out, float* __restrict__ c_avg,
    float b_c, int32_t first) {
    __shared__ uint64_t lo_s[kExactLimbs], hi_s[kExactLimbs];
    const int l = blockIdx.x;
    if (l >= n_seg || need[n_seg] == 0 || !need[l]) return;  // workgroup-uniform
    const double sx = exact_layer_sum(slots, wg_first[l], wg_first[l + 1], 0, lo_s, hi_s);
    const double su = exact_layer_sum(slots, wg_first[l], wg_first[l + 1], 1, lo_s, hi_s);
    if (threadIdx.x != 0) return;
    const float c = (sx == 0.0 || su == 0.0) ? 1.0f : (float)(sqrt(sx) / sqrt(su));
    c_out[l] = c;
    c_avg[l] = first ? c : b_c * c_avg[l] + (1.0f - b_c) * c;
}

// LAMB warmup pass 2: x -= (lr c_l) (m / (sqrtf(v) + eps)) with the new m, v.
__global__ __launch_bounds__(kThreads) void warmup_lamb_apply_kernel(
    float* __restrict__ x, const float* __restrict__ m, const float* __restrict__ v,
    const int64_t* __restrict__ seg_off, const int64_t* __restrict__ wg_first, int32_t n_seg,
    int64_t N, const float* __restrict__ c, float lr, float eps) {
    WgRange r;
    if (!wg_range(seg_off, wg_first, n_seg, N, r)) return;
    const float step = lr * c[r.layer];
    f4 xv[kLambTiles], mv[kLambTiles], vv[kLambTiles];
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t J = r.base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
        if (J < r.qend) {
            xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x + J));
            mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + J));
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + J));
        }
    }
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t J = r.base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
        if (J >= r.qend) break;
        const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        const float ms[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
        const float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        float xo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float den = sqrtf(vs[k]) + eps;
            const float uk = ms[k] / den;
            xo[k] = xs[k] - step * uk;
        }
        store_quad(x, J, r.lo, r.hi, xo);
    }
}

// Momentum scale, pass 1: sum m^2 of this workgroup's part of its layer.
__global__ __launch_bounds__(kThreads) void momentum_sq_kernel(
    const float* __restrict__ m, const int64_t* __restrict__ seg_off,
    const int64_t* __restrict__ wg_first, int32_t n_seg, int64_t N, double2* __restrict__ part) {
    __shared__ double red[kThreads / 64];
    WgRange r;
    if (!wg_range(seg_off, wg_first, n_seg, N, r)) return;
    f4 mv[kLambTiles];
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t J = r.base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
        if (J < r.qend) mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + J));
    }
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t J = r.base + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
        if (J >= r.qend) break;
        const float ms[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (J + k >= r.lo && J + k < r.hi) s += (double)ms[k] * (double)ms[k];
    }
    const double t = block_sum_f64(s, red);
    if (threadIdx.x == 0) part[blockIdx.x] = make_double2(t, 0.0);
}

// Momentum scale, pass 2: one workgroup per layer, rms[l] = sqrt(sum / d_l).
__global__ __launch_bounds__(kThreads) void momentum_rms_kernel(
    const double2* __restrict__ part, const int64_t* __restrict__ wg_first,
    const int64_t* __restrict__ seg_off, int32_t n_seg, int64_t N, int64_t n_wg,
    double* __restrict__ rms) {
    __shared__ double red[kThreads / 64];
    const int l = blockIdx.x;
    if (l >= n_seg) return;
    const int64_t w1 = wg_first[l + 1] < n_wg ? wg_first[l + 1] : n_wg;
    const double s = slot_sum(part, wg_first[l], w1, red).x;
    if (threadIdx.x != 0) return;
    int64_t lo, hi;
    layer_bounds(seg_off, l, N, lo, hi);
    const int64_t d = hi - lo;
    rms[l] = d > 0 ? sqrt(s / (double)d) : 0.0;
}

// Momentum scale, pass 3 (one workgroup): the mean over layers with a_l > 0,
// then k_l, written only if every layer's k_l is certified; otherwise every
// layer is marked for the exact path (the mean needs all of them).
//
// Certification: with D_l = norm_depth of layer l, the binary64 RMS is
// within (D_l / 2 + 2) u of the exact RMS, the fixed-order mean within
// (max D / 2 + 2 + D_S + 1) u of the exact mean (D_S additions over the
// layers), and k_l within the sum of both plus u; the value the exact sums
// give is within 7 u.  The slack (max D + D_S + 32) u covers all of it.
// Infinite or NaN norms are what the exact sums give as well.
__global__ __launch_bounds__(kThreads) void momentum_scale_kernel(
    const double* __restrict__ rms, const int64_t* __restrict__ wg_first, int32_t n_seg,
    float* __restrict__ k, int32_t* __restrict__ need) {
    __shared__ double red[kThreads / 64];
    __shared__ double bc[2];
    __shared__ unsigned long long dmax;
    if (threadIdx.x == 0) dmax = 0;
    double s = 0.0, cnt = 0.0;
    int64_t slots_max = 0;
    for (int l = threadIdx.x; l < n_seg; l += kThreads) {
        const double a = rms[l];
        if (a > 0.0) {
            s += a;
            cnt += 1.0;
        }
        const int64_t sl = wg_first[l + 1] - wg_first[l];
        slots_max = sl > slots_max ? sl : slots_max;
    }
    const double ts = block_sum_f64(s, red);
    __syncthreads();
    const double tc = block_sum_f64(cnt, red);
    atomicMax(&dmax, (unsigned long long)slots_max);
    if (threadIdx.x == 0) {
        bc[0] = ts;
        bc[1] = tc;
    }
    __syncthreads();
    const double mean = bc[1] > 0.0 ? bc[0] / bc[1] : 0.0;
    const int64_t d_s = (n_seg + kThreads - 1) / kThreads + 9;
    const double delta = (double)(norm_depth((int64_t)dmax) + d_s + 32) * 0x1p-53;
    bool ok = true;
    for (int l = threadIdx.x; l < n_seg; l += kThreads) {
        const double a = rms[l];
        if (a > 0.0 && isfinite(a) && isfinite(mean)) ok = ok && certified(mean / a, delta);
    }
    const int all_ok = __syncthreads_and(ok ? 1 : 0);
    for (int l = threadIdx.x; l < n_seg; l += kThreads) {
        need[l] = all_ok ? 0 : 1;
        if (all_ok) {
            const double a = rms[l];
            k[l] = a > 0.0 ? (float)(mean / a) : 1.0f;
        }
    }
    if (threadIdx.x == 0) need[n_seg] = all_ok ? 0 : 1;
}

// Exact path of k_l, per layer: rms_exact[l] = sqrt(exact sum / d_l).
__global__ __launch_bounds__(kThreads) void momentum_exact_rms_kernel(
    const uint64_t* __restrict__ slots, const int64_t* __restrict__ wg_first,
    const int64_t* __restrict__ seg_off, int32_t n_seg, int64_t N, const int32_t* __restrict__ need,
    double* __restrict__ rms_exact) {
    __shared__ uint64_t lo_s[kExactLimbs], hi_s[kExactLimbs];
    const int l = blockIdx.x;
    if (l >= n_seg || need[n_seg] == 0) return;  // all layers are marked together
    const double sq = exact_layer_sum(slots, wg_first[l], wg_first[l + 1], 0, lo_s, hi_s);
    if (threadIdx.x != 0) return;
    int64_t lo, hi;
    layer_bounds(seg_off, l, N, lo, hi);
    rms_exact[l] = hi > lo ? sqrt(sq / (double)(hi - lo)) : 0.0;
}

// Exact path of k_l, one workgroup: the exact sum of the RMS values over
// layers with a_l > 0 (units 2^-1074, 34 limbs: 2^31 binary64 terms), rounded
// once to binary64 and divided by their count, then k_l = mean / a_l.
__global__ __launch_bounds__(kThreads) void momentum_exact_scale_kernel(
    const double* __restrict__ rms_exact, int32_t n_seg, const int32_t* __restrict__ need,
    float* __restrict__ k) {
    constexpr int kWideLimbs = 34;
    __shared__ double mean_s;
    if (need[n_seg] == 0) return;
    if (threadIdx.x == 0) {
        uint64_t wide[kWideLimbs];
        for (int i = 0; i < kWideLimbs; ++i) wide[i] = 0;
        int64_t cnt = 0;
        for (int l = 0; l < n_seg; ++l) {
            const double a = rms_exact[l];
            if (!(a > 0.0)) continue;
            ++cnt;
            const uint64_t b = (uint64_t)__double_as_longlong(a);
            const int E = (int)((b >> 52) & 0x7FF);
            const uint64_t M = (b & ((1ull << 52) - 1)) | (E ? (1ull << 52) : 0ull);
            limbs_add_shifted<kWideLimbs>(wide, M, E ? E - 1 : 0);
        }
        mean_s = cnt ? limbs_to_double<kWideLimbs>(wide, -1074) / (double)cnt : 0.0;
    }
    __syncthreads();
    const double mean = mean_s;
    for (int l = threadIdx.x; l < n_seg; l += kThreads) {
        const double a = rms_exact[l];
        k[l] = a > 0.0 ? (float)(mean / a) : 1.0f;
    }
}

// ---------------------------------------------------------------- launchers

int64_t layer_grid(int64_t N, int32_t n_seg) {
    return (N + kSpan - 1) / kSpan + 2 * (int64_t)n_seg + 1;
}

hipError_t launch_warmup_adam(float* x, float* m, float* v, const float* g, int64_t N, float lr,
                              float eps, float b1, float b2, hipStream_t st) {
    const int64_t per_wg = (int64_t)kMaxIters * kTile;
    hipLaunchKernelGGL(warmup_adam_kernel, dim3((unsigned)((N + per_wg - 1) / per_wg)),
                       dim3(kThreads), 0, st, x, m, v, g, N, lr, eps, b1, b2);
    return hipGetLastError();
}

// workgroups of the exact pass: a fixed grid that walks the plan (it returns
// at once when no layer is marked)
constexpr int kExactGrid = 1024;

hipError_t launch_warmup_lamb(const WarmupLambArgs& a, const WarmupWs& ws, hipStream_t st) {
    const int64_t n_wg = layer_grid(a.N, a.n_seg);
    const dim3 grid((unsigned)n_wg);
    hipLaunchKernelGGL(layer_plan_kernel, dim3(1), dim3(kThreads), 0, st, a.seg_off, a.n_seg, a.N,
                       ws.wg_first, ws.need + a.n_seg);
    hipLaunchKernelGGL(warmup_lamb_moments_kernel, grid, dim3(kThreads), 0, st, a.x, a.m, a.v, a.g,
                       a.seg_off, ws.wg_first, a.n_seg, a.N, ws.part, a.eps, a.beta1, a.beta2);
    hipLaunchKernelGGL(warmup_lamb_finalize_kernel, dim3(a.n_seg), dim3(kThreads), 0, st, ws.part,
                       ws.wg_first, a.n_seg, n_wg, a.c, a.c_avg, a.beta_c, a.first, ws.need);
    hipLaunchKernelGGL(exact_squares_kernel<true>, dim3(kExactGrid), dim3(kThreads), 0, st, a.x,
                       a.m, a.v, a.seg_off, ws.wg_first, a.n_seg, a.N, a.eps, ws.need, ws.slots);
    hipLaunchKernelGGL(warmup_lamb_exact_kernel, dim3(a.n_seg), dim3(kThreads), 0, st, ws.slots,
                       ws.wg_first, a.n_seg, ws.need, a.c, a.c_avg, a.beta_c, a.first);
    hipLaunchKernelGGL(warmup_lamb_apply_kernel, grid, dim3(kThreads), 0, st, a.x, a.m, a.v,
                       a.seg_off, ws.wg_first, a.n_seg, a.N, a.c, a.lr, a.eps);
    return hipGetLastError();
}

hipError_t launch_momentum_scale(const float* m, int64_t N, const int64_t* seg_off, int32_t n_seg,
                                 float* k, const WarmupWs& ws, hipStream_t st) {
    const int64_t n_wg = layer_grid(N, n_seg);
    hipLaunchKernelGGL(layer_plan_kernel, dim3(1), dim3(kThreads), 0, st, seg_off, n_seg, N,
                       ws.wg_first, ws.need + n_seg);
    hipLaunchKernelGGL(momentum_sq_kernel, dim3((unsigned)n_wg), dim3(kThreads), 0, st, m, seg_off,
                       ws.wg_first, n_seg, N, ws.part);
    hipLaunchKernelGGL(momentum_rms_kernel, dim3(n_seg), dim3(kThreads), 0, st, ws.part, ws.wg_first,
                       seg_off, n_seg, N, n_wg, ws.rms);
    hipLaunchKernelGGL(momentum_scale_kernel, dim3(1), dim3(kThreads), 0, st, ws.rms, ws.wg_first,
                       n_seg, k, ws.need);
    hipLaunchKernelGGL(exact_squares_kernel<false>, dim3(kExactGrid), dim3(kThreads), 0, st,
                       nullptr, m, nullptr, seg_off, ws.wg_first, n_seg, N, 0.0f, ws.need,
                       ws.slots);
    hipLaunchKernelGGL(momentum_exact_rms_kernel, dim3(n_seg), dim3(kThreads), 0, st, ws.slots,
                       ws.wg_first, seg_off, n_seg, N, ws.need, ws.rms_exact);
    hipLaunchKernelGGL(momentum_exact_scale_kernel, dim3(1), dim3(kThreads), 0, st, ws.rms_exact,
                       n_seg, ws.need, k);
    return hipGetLastError();
}

}  // namespace onebit
