// Block-wise INT8 stochastic rounding with error feedback
// (gradient-quantisation tutorial, "FP32 -> INT8": max/127 scale per block,
// floor plus a Bernoulli(fraction) draw, clamp to [-127, 127], dequantise;
// error feedback from its 1-bit section).
//
// Each lane owns 4 consecutive elements (one float4, one Philox4x32-10 call
// whose 4 output words are the 4 uniforms, one 32-bit store of 4 codes).  A
// quantisation block of B elements spans B/4 lanes; its max |g'| is a
// butterfly over those lanes (B <= 256) or, for B = 512 / 1024, combined
// across waves through LDS.
//
// Philox4x32-10 is the SC'11 construction: per round two 32x32->64
// multiplies of counter words 0 and 2, xor of the high halves with the other
// words and the round key; key bumped by the two Weyl constants.
#include "common.h"

namespace onebit {

namespace {

__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3, uint32_t k0, uint32_t k1) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
}

__device__ __forceinline__ void philox10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                         uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        philox_round(c0, c1, c2, c3, k0, k1);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

template <int B>
__device__ __forceinline__ float group_max(float v, float* lds) {
    constexpr int lanes = B / 4;  // lanes per quantisation block
    constexpr int wl = lanes < 64 ? lanes : 64;
#pragma unroll
    for (int off = 1; off < wl; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if constexpr (lanes > 64) {
        constexpr int waves = lanes / 64;  // waves per block (2 or 4)
        const int w = threadIdx.x >> 6;
        if (lane_id() == 0) lds[w] = v;
        __syncthreads();
        const int g0 = (w / waves) * waves;
        float r = lds[g0];
#pragma unroll
        for (int q = 1; q < waves; ++q) r = fmaxf(r, lds[g0 + q]);
        __syncthreads();
        v = r;
    }
    return v;
}

}  // namespace

// B = 0: one scale for the whole tensor, from the maximum a previous kernel
// left in *tensor_max (bit pattern of a non-negative float).
// NEAREST: round to the nearest integer, halves away from zero, instead of
// the stochastic draw.
template <int B, bool EF, bool DEQ, bool NEAREST>
__global__ __launch_bounds__(kThreads) void int8_kernel(const float* __restrict__ g,
                                                       float* __restrict__ err,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       float* __restrict__ deq, int64_t N,
                                                       int32_t iters, uint32_t k0, uint32_t k1,
                                                       uint32_t step,
                                                       const uint32_t* __restrict__ tensor_max) {
    __shared__ float lds[kThreads / 64];
    constexpr int lanes = B == 0 ? 64 : B / 4;
    const float Mt = B == 0 ? __uint_as_float(*tensor_max) : 0.0f;
    const int64_t base = (int64_t)blockIdx.x * iters * kTile;
    // loads of all tiles first (memory-level parallelism), then the blocks
    f4 gv[kInt8Tiles], ev[kInt8Tiles];
#pragma unroll
    for (int it = 0; it < kInt8Tiles; ++it) {
        const int64_t J = base + (int64_t)it * kTile + 4 * (int64_t)threadIdx.x;
        gv[it] = f4{0.f, 0.f, 0.f, 0.f};
        ev[it] = f4{0.f, 0.f, 0.f, 0.f};
        if (it < iters && J < N) {
            gv[it] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(g + J));
            if (EF) ev[it] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(err + J));
        }
    }
#pragma unroll
    for (int it = 0; it < kInt8Tiles; ++it) {
        if (it >= iters || base + (int64_t)it * kTile >= N) break;  // workgroup-uniform
        const int64_t J = base + (int64_t)it * kTile + 4 * (int64_t)threadIdx.x;
        const bool active = J < N;
        float x[4] = {gv[it].x, gv[it].y, gv[it].z, gv[it].w};
        if (EF) {
            x[0] = x[0] + ev[it].x;
            x[1] = x[1] + ev[it].y;
            x[2] = x[2] + ev[it].z;
            x[3] = x[3] + ev[it].w;
        }
        float M = Mt;
        if constexpr (B != 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) M = fmaxf(M, fabsf(x[k]));
            M = group_max<B>(M, lds);
        }
        const float scale = M / 127.0f;

        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if constexpr (!NEAREST) {
            uint32_t c0 = (uint32_t)((uint64_t)J >> 2), c1 = (uint32_t)((uint64_t)J >> 34),
                     c2 = step, c3 = 0;
            philox10(c0, c1, c2, c3, k0, k1);
            w[0] = c0;
            w[1] = c1;
            w[2] = c2;
            w[3] = c3;
        }

        float q[4], d[4], e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (scale == 0.0f) {
                q[k] = 0.0f;
                d[k] = 0.0f;
            } else {
                const float xs = x[k] / scale;
                float qq;
                if constexpr (NEAREST) {
                    qq = roundf(xs);
                } else {
                    const float f = floorf(xs);
                    const float p = xs - f;
                    const float u = (float)(w[k] >> 8) * 0x1p-24f;
                    qq = f + (u < p ? 1.0f : 0.0f);
                }
                qq = fminf(fmaxf(qq, -127.0f), 127.0f);
                q[k] = qq;
                d[k] = qq * scale;
            }
            e[k] = x[k] - d[k];
        }
        if (active) {
            const uint32_t packed = ((uint32_t)(uint8_t)(int8_t)(int)q[0]) |
                                    ((uint32_t)(uint8_t)(int8_t)(int)q[1] << 8) |
                                    ((uint32_t)(uint8_t)(int8_t)(int)q[2] << 16) |
                                    ((uint32_t)(uint8_t)(int8_t)(int)q[3] << 24);
            // nontemporal: measured 7 % faster than normal stores for codes and error
            __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(codes + J));
            if (EF) {
                const f4 eo = {e[0], e[1], e[2], e[3]};
                __builtin_nontemporal_store(eo, reinterpret_cast<f4*>(err + J));
            }
            if (DEQ) {
                const f4 dq = {d[0], d[1], d[2], d[3]};
                __builtin_nontemporal_store(dq, reinterpret_cast<f4*>(deq + J));
            }
            if constexpr (B == 0) {
                if (J == 0) scales[0] = scale;
            } else if ((threadIdx.x % lanes) == 0) {
                scales[J / B] = scale;
            }
        }
    }
}

// max over the tensor of |g (+ err)| (NaN skipped) as the bit pattern of a
// non-negative float.  A fixed grid strides over the tensor, four tiles per
// pass with all loads issued before the maxima, and each workgroup ends with
// one atomicMax, so the single accumulator sees a few thousand atomics rather
// than one per tile.
template <bool EF>
__global__ __launch_bounds__(kThreads) void tensor_absmax_kernel(const float* __restrict__ g,
                                                                const float* __restrict__ err,
                                                                int64_t N,
                                                                uint32_t* __restrict__ out) {
    __shared__ uint32_t red[kThreads / 64];
    constexpr int64_t span = (int64_t)kMaxIters * kTile;
    const int64_t stride = (int64_t)gridDim.x * span;
    float M = 0.0f;
    for (int64_t base = (int64_t)blockIdx.x * span; base < N; base += stride) {
        f4 gv[kMaxIters], ev[kMaxIters];
#pragma unroll
        for (int it = 0; it < kMaxIters; ++it) {
            const int64_t J = base + (int64_t)it * kTile + 4 * (int64_t)threadIdx.x;
            gv[it] = f4{0.f, 0.f, 0.f, 0.f};
            ev[it] = f4{0.f, 0.f, 0.f, 0.f};
            if (J < N) {
                gv[it] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(g + J));
                if (EF) ev[it] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(err + J));
            }
        }
#pragma unroll
        for (int it = 0; it < kMaxIters; ++it) {
            f4 x = gv[it];
            if (EF) x = f4{x.x + ev[it].x, x.y + ev[it].y, x.z + ev[it].z, x.w + ev[it].w};
            M = fmaxf(M, fabsf(x.x));
            M = fmaxf(M, fabsf(x.y));
            M = fmaxf(M, fabsf(x.z));
            M = fmaxf(M, fabsf(x.w));
        }
    }
    uint32_t u = __float_as_uint(M);  // non-negative: integer order is value order
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)u, off, 64);
        u = o > u ? o : u;
    }
    if (lane_id() == 0) red[threadIdx.x >> 6] = u;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = red[0];
        for (int w = 1; w < kThreads / 64; ++w) b = red[w] > b ? red[w] : b;
        atomicMax(out, b);
    }
}

constexpr int64_t kAbsmaxBlocks = 2048;

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

template <int B, bool NEAREST>
static void launch_b(dim3 grid, hipStream_t st, const float* g, float* err, int8_t* codes,
                     float* scales, float* deq, int64_t N, int32_t iters, uint32_t k0, uint32_t k1,
                     uint32_t step, const uint32_t* tmax) {
    if (err && deq)
        hipLaunchKernelGGL((int8_kernel<B, true, true, NEAREST>), grid, dim3(kThreads), 0, st, g,
                           err, codes, scales, deq, N, iters, k0, k1, step, tmax);
    else if (err)
        hipLaunchKernelGGL((int8_kernel<B, true, false, NEAREST>), grid, dim3(kThreads), 0, st, g,
                           err, codes, scales, deq, N, iters, k0, k1, step, tmax);
    else if (deq)
        hipLaunchKernelGGL((int8_kernel<B, false, true, NEAREST>), grid, dim3(kThreads), 0, st, g,
                           err, codes, scales, deq, N, iters, k0, k1, step, tmax);
    else
        hipLaunchKernelGGL((int8_kernel<B, false, false, NEAREST>), grid, dim3(kThreads), 0, st, g,
                           err, codes, scales, deq, N, iters, k0, k1, step, tmax);
}

template <bool NEAREST>
static hipError_t launch_r(dim3 grid, hipStream_t st, const float* g, float* err, int8_t* codes,
                           float* scales, float* deq, int64_t N, int32_t block, int32_t iters,
                           uint32_t k0, uint32_t k1, uint32_t step, uint32_t* tmax) {
    switch (block) {
        case 0:
            hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, st, tmax);
            {
                // 8 workgroups per CU; fewer when the tensor is small
                const int64_t spans = (N + (int64_t)kMaxIters * kTile - 1) / ((int64_t)kMaxIters * kTile);
                const dim3 mgrid((unsigned)(spans < kAbsmaxBlocks ? spans : kAbsmaxBlocks));
                if (err)
                    hipLaunchKernelGGL(tensor_absmax_kernel<true>, mgrid, dim3(kThreads), 0, st, g,
                                       err, N, tmax);
                else
                    hipLaunchKernelGGL(tensor_absmax_kernel<false>, mgrid, dim3(kThreads), 0, st, g,
                                       err, N, tmax);
            }
            launch_b<0, NEAREST>(grid, st, g, err, codes, scales, deq, N, iters, k0, k1, step, tmax);
            break;
        case 64: launch_b<64, NEAREST>(grid, st, g, err, codes, scales, deq, N, iters, k0, k1, step, tmax); break;
        case 128: launch_b<128, NEAREST>(grid, st, g, err, codes, scales, deq, N, iters, k0, k1, step, tmax); break;
        case 256: launch_b<256, NEAREST>(grid, st, g, err, codes, scales, deq, N, iters, k0, k1, step, tmax); break;
        case 512: launch_b<512, NEAREST>(grid, st, g, err, codes, scales, deq, N, iters, k0, k1, step, tmax); break;
        case 1024: launch_b<1024, NEAREST>(grid, st, g, err, codes, scales, deq, N, iters, k0, k1, step, tmax); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_int8(const float* g, float* err, int8_t* codes, float* scales, float* deq,
                       int64_t N, int32_t block, uint64_t seed, uint32_t step, bool nearest,
                       uint32_t* tensor_max, hipStream_t st) {
    const int32_t iters = kInt8Tiles;
    const int64_t tiles = (N + kTile - 1) / kTile;
    const dim3 grid((unsigned)((tiles + iters - 1) / iters));
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (nearest)
        return launch_r<true>(grid, st, g, err, codes, scales, deq, N, block, iters, k0, k1, step,
                              tensor_max);
    return launch_r<false>(grid, st, g, err, codes, scales, deq, N, block, iters, k0, k1, step,
                           tensor_max);
}

}  // namespace onebit
