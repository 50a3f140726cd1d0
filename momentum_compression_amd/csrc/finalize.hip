// Chunk-mean finalize: turns the per-workgroup fp64 partial sums of |x| into
// the binary32 value nearest to the exact mean (ties to even).
//
// Fast path.  The fp64 sum of non-negative terms, each passing through at
// most d additions, is within gamma_d = d u / (1 - d u) (u = 2^-53) of the
// exact sum relative to itself; with the final division the mean is within
// gamma_{d+1} <= (d + 1) u (1 + 3e-12) for d <= kMaxSumDepth = 12288.  The
// launch passes the relative slack (d + 4) u for the plan's own depth d,
// which also covers the rounding of mu_hat -+ slack in the comparison.  If
// mu_hat (1 -+ slack) lies strictly between the two binary32 rounding
// boundaries around (float)mu_hat, the exact mean rounds to the same value
// and the result is certified.
//
// Exact path (taken when certification fails, e.g. at an exact tie).  The
// same workgroup re-reads the chunk's stored values and accumulates the
// 24-bit significands per binary exponent in 64-bit LDS counters; thread 0
// assembles the exact sum as a 320-bit integer in units of 2^-149, divides by
// L and rounds to nearest even.
#include "common.h"

namespace onebit {

namespace {

constexpr int kLimbs = 10;  // 320 bits: sum < 2^32 * 2^24 * 2^253

__device__ void big_add_shifted(uint32_t* limb, uint64_t v, int sh) {
    int idx = sh >> 5;
    const int off = sh & 31;
    // v << off spans at most 3 limbs (v < 2^56)
    const uint64_t lo = v << off;
    const uint64_t hi = off ? (v >> (64 - off)) : 0;
    uint32_t parts[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi};
    uint64_t carry = 0;
    for (int k = 0; k < 3 || carry; ++k, ++idx) {
        if (idx >= kLimbs) break;
        uint64_t t = (uint64_t)limb[idx] + (k < 3 ? parts[k] : 0u) + carry;
        limb[idx] = (uint32_t)t;
        carry = t >> 32;
    }
}

__device__ uint32_t big_bits(const uint32_t* limb, int pos, int count) {
    // bits [pos, pos+count) (count <= 32) of the big integer
    const int idx = pos >> 5;
    const int off = pos & 31;
    uint64_t w = (uint64_t)limb[idx];
    if (idx + 1 < kLimbs) w |= (uint64_t)limb[idx + 1] << 32;
    w >>= off;
    return count == 32 ? (uint32_t)w : (uint32_t)(w & ((1ull << count) - 1));
}

__device__ bool big_any_below(const uint32_t* limb, int pos) {
    // any set bit strictly below bit `pos`
    const int idx = pos >> 5;
    for (int k = 0; k < idx; ++k)
        if (limb[k]) return true;
    const int off = pos & 31;
    return off && (limb[idx] & ((1u << off) - 1u));
}

// binary32 nearest to (sum over e of bins[e] * 2^(e-1)) * 2^-149 / L
__device__ float exact_mean_from_bins(const unsigned long long* bins, uint64_t L) {
    uint32_t limb[kLimbs];
    for (int k = 0; k < kLimbs; ++k) limb[k] = 0;
    for (int e = 1; e < 255; ++e)
        if (bins[e]) big_add_shifted(limb, bins[e], e - 1);
    uint64_t rem = 0;
    for (int k = kLimbs - 1; k >= 0; --k) {
        const uint64_t cur = (rem << 32) | limb[k];
        limb[k] = (uint32_t)(cur / L);
        rem = cur % L;
    }
    int top = kLimbs - 1;
    while (top >= 0 && limb[top] == 0) --top;
    if (top < 0) {  // quotient 0: below one unit of 2^-149
        return __uint_as_float((2 * rem > L) ? 1u : 0u);
    }
    const int bl = 32 * top + (32 - __clz(limb[top]));
    if (bl <= 24) {  // subnormal or the first normal binade: units of 2^-149
        uint32_t q = limb[0];
        if (2 * rem > L || (2 * rem == L && (q & 1u))) ++q;
        return __uint_as_float(q);  // q <= 2^24: the bit pattern equals q
    }
    int b = bl - 24;
    uint32_t m24 = big_bits(limb, b, 24);
    const uint32_t half = big_bits(limb, b - 1, 1);
    const bool sticky = big_any_below(limb, b - 1) || rem != 0;
    if (half && (sticky || (m24 & 1u))) ++m24;
    if (m24 == (1u << 24)) {
        m24 = 1u << 23;
        ++b;
    }
    if (b + 1 >= 255) return __uint_as_float(0x7F800000u);
    return __uint_as_float(((uint32_t)b << 23) + m24);
}

// Sum over the kFinThreads threads of the finalize workgroup: wave
// butterflies (6 levels), then a pairwise tree over the 16 wave sums (4
// levels); valid in thread 0.
__device__ __forceinline__ double fin_block_sum(double v, double* red) {
    v = wave_sum(v);
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        double t[kFinThreads / 64];
#pragma unroll
        for (int w = 0; w < kFinThreads / 64; ++w) t[w] = red[w];
#pragma unroll
        for (int width = kFinThreads / 128; width >= 1; width >>= 1)
#pragma unroll
            for (int w = 0; w < width; ++w) t[w] = t[2 * w] + t[2 * w + 1];
        r = t[0];
    }
    return r;
}

}  // namespace

// prev (or null): receives out[pair] as found on entry, before it is
// overwritten (the server's scales of the previous step)
__global__ __launch_bounds__(kFinThreads) void mean_finalize_kernel(
    const double* __restrict__ partials, int64_t bpc, int64_t L, const float* __restrict__ data,
    int64_t row_stride, int32_t chunks, float* __restrict__ out, int32_t unit,
    float* __restrict__ prev, double slack_rel) {
    __shared__ double red[kFinThreads / 64];
    __shared__ unsigned long long bins[256];
    __shared__ int exact;
    const int64_t pair = blockIdx.x;
    // thread 0 is the only writer of out[pair], and it copies it first
    if (prev && threadIdx.x == 0) prev[pair] = out[pair];
    if (unit) {  // the unscaled sign: every scale is 1
        if (threadIdx.x == 0) out[pair] = 1.0f;
        return;
    }
    const double* p = partials + pair * bpc;
    // thread t adds partials t, t + T, t + 2T, ... (T = kFinThreads) in that
    // order; the loads of 8 of them are issued before the additions
    constexpr int kBatch = 8;
    double acc = 0.0;
    for (int64_t k0 = threadIdx.x; k0 < bpc; k0 += (int64_t)kFinThreads * kBatch) {
        double v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t k = k0 + (int64_t)q * kFinThreads;
            v[q] = k < bpc ? p[k] : 0.0;
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) acc += v[q];
    }
    const double tot = fin_block_sum(acc, red);
    if (threadIdx.x == 0) {
        const double mu = tot / (double)L;
        const float r = (float)mu;
        int need_exact = 1;
        if (!(mu == mu) || isinf(mu) || tot == 0.0) {
            need_exact = 0;  // NaN, Inf (present in the data) or all zeros: exact as is
        } else if (!isinf(r)) {
            // neighbours of r >= 0 (the mean of absolute values is not negative)
            const uint32_t rb = __float_as_uint(r);
            const float rd = rb ? __uint_as_float(rb - 1u) : -__uint_as_float(1u);
            const float ru = __uint_as_float(rb + 1u);
            const double mlo = ((double)rd + (double)r) * 0.5;
            const double mhi = ((double)r + (double)ru) * 0.5;
            const double slack = mu * slack_rel;
            if (mu - slack > mlo && mu + slack < mhi) need_exact = 0;
        }
        exact = need_exact;
        if (!need_exact) out[pair] = r;
    }
    __syncthreads();
    if (!exact) return;

    // exact path: per-exponent significand sums of the stored chunk values
    for (int k = threadIdx.x; k < 256; k += kFinThreads) bins[k] = 0;
    __syncthreads();
    const int64_t row = pair / chunks;
    const int64_t c = pair - row * chunks;
    const float* x = data + row * row_stride + c * L;
    for (int64_t j = threadIdx.x; j < L; j += kFinThreads) {
        const uint32_t a = __float_as_uint(x[j]) & 0x7FFFFFFFu;
        uint32_t e = a >> 23;
        uint32_t mant = a & 0x7FFFFFu;
        if (e) mant |= 0x800000u; else e = 1;
        if (mant) atomicAdd(&bins[e], (unsigned long long)mant);
    }
    __syncthreads();
    if (threadIdx.x == 0) out[pair] = exact_mean_from_bins(bins, (uint64_t)L);
}

hipError_t launch_mean_finalize_keep(const double* partials, const ChunkPlan& plan,
                                     int64_t pairs, MeanTarget tgt, float* prev, hipStream_t st) {
    // relative slack of the certification for this plan's summation depth
    const double slack_rel = (double)(sum_depth(plan) + 4) * 0x1p-53;
    hipLaunchKernelGGL(mean_finalize_kernel, dim3((unsigned)pairs), dim3(kFinThreads), 0, st,
                       partials, plan.bpc, plan.L, tgt.data, tgt.row_stride, tgt.chunks, tgt.out,
                       tgt.unit ? 1 : 0, prev, slack_rel);
    return hipGetLastError();
}

hipError_t launch_mean_finalize(const double* partials, const ChunkPlan& plan, int64_t pairs,
                                MeanTarget tgt, hipStream_t st) {
    return launch_mean_finalize_keep(partials, plan, pairs, tgt, nullptr, st);
}

// ---------------------------------------------------------------- plan
ChunkPlan make_plan(int64_t L, int64_t chunks, int32_t max_iters, int32_t min_iters) {
    ChunkPlan p;
    p.L = L;
    const int64_t tiles = (L + kTile - 1) / kTile;
    // aim for at least ~8 workgroups per CU (256 CUs) over all chunks
    int64_t iters = max_iters;
    while (iters > min_iters && ((tiles + iters - 1) / iters) * chunks < 2048) iters >>= 1;
    if (iters < min_iters) iters = min_iters;
    p.iters = (int32_t)iters;
    p.bpc = (tiles + iters - 1) / iters;
    return p;
}

int64_t sum_depth(const ChunkPlan& p) {
    // producer workgroup: per thread 4 * iters sequential adds, 6 butterfly
    // levels, 2 LDS levels; finalize: ceil(bpc / kFinThreads) sequential adds,
    // 6 butterfly levels, 4 tree levels over the 16 waves; 1 division
    return 4 * (int64_t)p.iters + 6 + 2 + (p.bpc + kFinThreads - 1) / kFinThreads + 6 + 4 + 1;
}

}  // namespace onebit
