// Worker-side compression kernel (one pass over m and the error state).
//
// Per element (1-bit Adam article, section 2.1, on the momentum; scaled sign
// of the gradient-quantisation tutorial; reset and clamp of section 4.1):
//   e  = reset ? 0 : ef_prev -/+ s_prev      (lazy error, same fp32 op)
//   g' = k_l * m + e, clamped;  ef = g';  bit = g' >= 0
// and the chunk's sum of |g'| in fp64 as one partial per workgroup, which the
// finalize kernel turns into the exactly rounded mean.
//
// Layout: workgroup w of chunk (i, c) streams tiles of 1024 consecutive
// elements (float4 per lane, fully coalesced) of worker row i, chunk c.  The
// 4 sign bits of a lane are merged over 8 lanes with DPP into one 32-bit
// word, stored by the first lane of each group.
#include "common.h"

namespace onebit {

template <bool SEG, bool CLAMP, bool RESET>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const float* __restrict__ m, float* __restrict__ ef, const float* __restrict__ s_prev,
    uint32_t* __restrict__ bits, double* __restrict__ partials, int64_t N, int32_t n,
    int64_t L, int32_t iters, int64_t bpc, float clip, const int64_t* __restrict__ seg_off,
    const float* __restrict__ seg_k, int32_t n_seg) {
    __shared__ double red[kThreads / 64];
    const int64_t pair = blockIdx.x / bpc;
    const int64_t wg = blockIdx.x - pair * bpc;
    const int32_t i = (int32_t)(pair / n);
    const int32_t c = (int32_t)(pair - (int64_t)i * n);
    const int64_t row = (int64_t)i * N;
    const int64_t cbase = (int64_t)c * L;           // chunk start within the row
    const int64_t start = wg * (int64_t)iters * kTile;
    int64_t end = start + (int64_t)iters * kTile;
    if (end > L) end = L;
    const float s = RESET ? 0.0f : s_prev[pair];
    const int lane8 = lane_id() & 7;

    // segment tracking (per thread, monotone in j)
    int seg = 0;
    int64_t seg_hi = 0;
    float kv = 1.0f;
    if (SEG) {
        const int64_t J0 = cbase + start + 4 * (int64_t)threadIdx.x;
        seg = find_segment(seg_off, n_seg, J0 < N ? J0 : N - 1);
        seg_hi = seg_off[seg + 1];
        kv = seg_k[seg];
    }

    double acc = 0.0;
    for (int it0 = 0; it0 < iters; it0 += kUnroll) {
        // issue the loads of kUnroll tiles before any use (memory-level parallelism)
        f4 mv[kUnroll], pv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = start + (int64_t)(it0 + u) * kTile + 4 * (int64_t)threadIdx.x;
            mv[u] = f4{0.f, 0.f, 0.f, 0.f};
            pv[u] = f4{0.f, 0.f, 0.f, 0.f};
            if (it0 + u < iters && j < end) {
                mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + row + cbase + j));
                if (!RESET)
                    pv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(ef + row + cbase + j));
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = start + (int64_t)(it0 + u) * kTile + 4 * (int64_t)threadIdx.x;
            const bool active = it0 + u < iters && j < end;
            const int64_t idx = row + cbase + j;
            float g[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
            const float p[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (SEG) {
                    const int64_t J = cbase + j + k;
                    while (active && J >= seg_hi && seg + 1 < n_seg) {
                        ++seg;
                        seg_hi = seg_off[seg + 1];
                        kv = seg_k[seg];
                    }
                    g[k] = kv * g[k];
                }
                const float e = RESET ? 0.0f : ef_error(p[k], s);
                float v = g[k] + e;
                if (CLAMP) v = fminf(fmaxf(v, -clip), clip);
                g[k] = v;
            }
            const uint32_t word = or8(sign_nibble(g[0], g[1], g[2], g[3]) << (4 * lane8));
            if (active) {
                const f4 out = {g[0], g[1], g[2], g[3]};
                __builtin_nontemporal_store(out, reinterpret_cast<f4*>(ef + idx));
                acc += (double)fabsf(g[0]);
                acc += (double)fabsf(g[1]);
                acc += (double)fabsf(g[2]);
                acc += (double)fabsf(g[3]);
                if (lane8 == 0) bits[(row >> 5) + ((cbase + j) >> 5)] = word;
            }
        }
    }
    const double tot = block_sum(acc, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = tot;
}

template <bool SEG, bool CLAMP, bool RESET>
static void launch_t(dim3 grid, hipStream_t st, const float* m, float* ef, const float* s_prev,
                     uint32_t* bits, double* partials, int64_t N, int32_t n, const ChunkPlan& p,
                     float clip, const int64_t* seg_off, const float* seg_k, int32_t n_seg) {
    hipLaunchKernelGGL((compress_kernel<SEG, CLAMP, RESET>), grid, dim3(kThreads), 0, st, m, ef,
                       s_prev, bits, partials, N, n, p.L, p.iters, p.bpc, clip, seg_off, seg_k,
                       n_seg);
}

hipError_t launch_compress(const float* m, float* ef, const float* s_prev, uint32_t* bits,
                           double* partials, int64_t N, int32_t n, const ChunkPlan& plan,
                           float clip, bool clamp_on, bool reset, const int64_t* seg_off,
                           const float* seg_k, int32_t n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(plan.bpc * (int64_t)n * n));
    const bool seg = seg_off != nullptr;
    const int sel = (seg ? 4 : 0) | (clamp_on ? 2 : 0) | (reset ? 1 : 0);
#define ONEBIT_CASE(S, C, R)                                                                    \
    case (S ? 4 : 0) | (C ? 2 : 0) | (R ? 1 : 0):                                               \
        launch_t<S, C, R>(grid, st, m, ef, s_prev, bits, partials, N, n, plan, clip, seg_off,  \
                          seg_k, n_seg);                                                        \
        break;
    switch (sel) {
        ONEBIT_CASE(false, false, false)
        ONEBIT_CASE(false, false, true)
        ONEBIT_CASE(false, true, false)
        ONEBIT_CASE(false, true, true)
        ONEBIT_CASE(true, false, false)
        ONEBIT_CASE(true, false, true)
        ONEBIT_CASE(true, true, false)
        ONEBIT_CASE(true, true, true)
    }
#undef ONEBIT_CASE
    return hipGetLastError();
}

}  // namespace onebit
