// Worker-side compression kernel (one pass over m and the error state).
//
// Per element (1-bit Adam article, section 2.1, on the momentum; scaled sign
// of the gradient-quantisation tutorial; reset and clamp of section 4.1):
//   e  = reset ? 0 : ef_prev -/+ s_prev      (lazy error, same fp32 op)
//   g' = k_l * m + e, clamped;  ef = g';  bit = g' >= 0
// and the chunk's sum of |g'| in fp64 as one partial per workgroup, which the
// finalize kernel turns into the exactly rounded mean.
//
// With MOM the input is the worker's gradient instead of its momentum: the
// local momentum m = beta1 mbar + (1 - beta1) g is formed on the fly from the
// previous step's packed global momentum (server sign words and chunk
// scales, divided by k_l in LAMB mode), so m is never written to memory
// (1-bit Adam article, section 2.1, momentum recursion).
//
// Layout: the grid is (workgroups per chunk, n * n); workgroup (w, i n + c)
// streams kCompressIters tiles of 1024 consecutive elements (float4 per
// lane, fully coalesced) of worker row i, chunk c.  One tile per workgroup
// measured fastest: millions of short workgroups keep every CU's memory
// pipeline full.  The 4 sign bits of a lane are merged over 8 lanes with DPP
// into one 32-bit word, stored by the first lane of each group.
#include "common.h"

namespace onebit {

template <bool SEG, bool CLAMP, bool RESET, bool MOM, bool ERS>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const float* __restrict__ m, float* __restrict__ ef, const float* __restrict__ s_prev,
    uint32_t* __restrict__ bits, double* __restrict__ partials, int64_t N, int32_t n,
    int64_t L, int32_t iters, int64_t bpc, float clip, const int64_t* __restrict__ seg_off,
    const float* __restrict__ seg_k, int32_t n_seg, const uint32_t* __restrict__ mb_bits,
    const float* __restrict__ mb_scales, float beta1, const float* __restrict__ seg_r) {
    __shared__ double red[kThreads / 64];
    // grid (bpc, n * n): x = workgroup within the chunk, y = (worker, chunk);
    // a 1-D grid of all of them could exceed 2^32 work-items
    const int64_t pair = blockIdx.y;
    const int64_t wg = blockIdx.x;
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
    float rv = 1.0f;  // ERS: step-ratio factor of the carried error in this layer
    if (SEG) {
        // one (scalar) search for the workgroup's first element, then each
        // thread walks to the layer of its own first element
        const int64_t W0 = cbase + start;
        seg = find_segment(seg_off, n_seg, W0);
        seg_hi = seg_off[seg + 1];
        const int64_t J0 = W0 + 4 * (int64_t)threadIdx.x;
        while (J0 >= seg_hi && seg + 1 < n_seg) {
            ++seg;
            seg_hi = seg_off[seg + 1];
        }
        kv = seg_k[seg];
        if (ERS) rv = seg_r[seg];
    }

    // MOM: value of a set bit of the previous global momentum in this chunk
    // (S[c], or S[c] / k_l in LAMB mode), recomputed when the layer changes
    const float omb1 = 1.0f - beta1;
    const float mS = MOM ? mb_scales[c] : 0.0f;
    float mq = (MOM && SEG) ? mS / kv : mS;

    double acc = 0.0;
    for (int it0 = 0; it0 < iters; it0 += kCompressUnroll) {
        // issue the loads of kCompressUnroll tiles before any use
        f4 mv[kCompressUnroll], pv[kCompressUnroll];
        uint32_t mw[kCompressUnroll];
#pragma unroll
        for (int u = 0; u < kCompressUnroll; ++u) {
            const int64_t j = start + (int64_t)(it0 + u) * kTile + 4 * (int64_t)threadIdx.x;
            mv[u] = f4{0.f, 0.f, 0.f, 0.f};
            pv[u] = f4{0.f, 0.f, 0.f, 0.f};
            mw[u] = 0u;
            if (it0 + u < iters && j < end) {
                mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + row + cbase + j));
                if (!RESET)
                    pv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(ef + row + cbase + j));
                if (MOM) mw[u] = mb_bits[(cbase + j) >> 5];
            }
        }
#pragma unroll
        for (int u = 0; u < kCompressUnroll; ++u) {
            const int64_t j = start + (int64_t)(it0 + u) * kTile + 4 * (int64_t)threadIdx.x;
            const bool active = it0 + u < iters && j < end;
            const int64_t idx = row + cbase + j;
            float g[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
            const float p[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
            const uint32_t mword = mw[u] >> ((cbase + j) & 31);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (SEG) {
                    const int64_t J = cbase + j + k;
                    if (active && J >= seg_hi && seg + 1 < n_seg) {
                        while (J >= seg_hi && seg + 1 < n_seg) {
                            ++seg;
                            seg_hi = seg_off[seg + 1];
                            kv = seg_k[seg];
                            if (ERS) rv = seg_r[seg];
                        }
                        if (MOM) mq = mS / kv;
                    }
                }
                if (MOM) {
                    const float mbar = ((mword >> k) & 1u) ? mq : -mq;
                    const float a = beta1 * mbar;
                    const float b = omb1 * g[k];
                    g[k] = a + b;
                }
                if (SEG) g[k] = kv * g[k];
                float e = RESET ? 0.0f : ef_error(p[k], s);
                if (ERS) e = rv * e;
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
    if (threadIdx.x == 0) partials[pair * bpc + wg] = tot;
}

template <bool SEG, bool CLAMP, bool RESET, bool MOM, bool ERS>
static void launch_t(dim3 grid, hipStream_t st, const CompressArgs& a, const ChunkPlan& p) {
    hipLaunchKernelGGL((compress_kernel<SEG, CLAMP, RESET, MOM, ERS>), grid, dim3(kThreads), 0, st,
                       a.m, a.ef, a.s_prev, a.bits, a.partials, a.N, a.n, p.L, p.iters, p.bpc,
                       a.clip, a.seg_off, a.seg_k, a.n_seg, a.mb_bits, a.mb_scales, a.beta1,
                       a.seg_r);
}

template <bool SEG, bool CLAMP, bool RESET>
static void launch_m(dim3 grid, hipStream_t st, const CompressArgs& a, const ChunkPlan& p) {
    // the step-ratio factor needs a layer table and a carried error
    constexpr bool kErsPossible = SEG && !RESET;
    const bool ers = kErsPossible && a.seg_r != nullptr;
    if (a.mb_bits) {
        if (ers) launch_t<SEG, CLAMP, RESET, true, kErsPossible>(grid, st, a, p);
        else launch_t<SEG, CLAMP, RESET, true, false>(grid, st, a, p);
    } else {
        if (ers) launch_t<SEG, CLAMP, RESET, false, kErsPossible>(grid, st, a, p);
        else launch_t<SEG, CLAMP, RESET, false, false>(grid, st, a, p);
    }
}

hipError_t launch_compress(const CompressArgs& a, const ChunkPlan& plan, hipStream_t st) {
    const dim3 grid((unsigned)plan.bpc, (unsigned)((int64_t)a.n * a.n));
    const int sel = (a.seg_off ? 4 : 0) | (a.clamp_on ? 2 : 0) | (a.reset ? 1 : 0);
    switch (sel) {
        case 0: launch_m<false, false, false>(grid, st, a, plan); break;
        case 1: launch_m<false, false, true>(grid, st, a, plan); break;
        case 2: launch_m<false, true, false>(grid, st, a, plan); break;
        case 3: launch_m<false, true, true>(grid, st, a, plan); break;
        case 4: launch_m<true, false, false>(grid, st, a, plan); break;
        case 5: launch_m<true, false, true>(grid, st, a, plan); break;
        case 6: launch_m<true, true, false>(grid, st, a, plan); break;
        default: launch_m<true, true, true>(grid, st, a, plan); break;
    }
    return hipGetLastError();
}

}  // namespace onebit
