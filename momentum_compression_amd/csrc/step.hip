// Frozen-variance parameter steps.
//
// Adam (1-bit Adam article, sections 2.1 and 6; frozen denominator from the
// 1-bit LAMB page, algorithm paragraph):  x = x - lr * (m / (sqrtf(v) + eps)).
//
// LAMB (1-bit LAMB page, algorithm and analysis paragraphs), one streaming
// pass:  g = (m - beta1 m_prev) / (1 - beta1);  v_f = beta2 v_f + (1-beta2) g^2;
// per-layer max of v / v_f (order-preserving uint keys, NaN skipped; one slot
// per workgroup inside a layer, LDS-merged atomics for the workgroups across
// layer boundaries);  x -= (lr c_{t-1,l}) m / (sqrtf(v)+eps).  A per-layer
// kernel then reduces the slots and forms r_t and c_t.  With use_c_t the x
// update moves to a second pass after r_t / c_t are known.
#include "common.h"

namespace onebit {

__global__ __launch_bounds__(kThreads) void adam_kernel(float* __restrict__ x,
                                                        const float* __restrict__ m,
                                                        const float* __restrict__ v, int64_t N,
                                                        float lr, float eps) {
    const int64_t j0 = (int64_t)blockIdx.x * kMaxIters * kTile + 4 * (int64_t)threadIdx.x;
    f4 xv[kMaxIters], mv[kMaxIters], vv[kMaxIters];
#pragma unroll
    for (int u = 0; u < kMaxIters; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j < N) {
            xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x + j));
            mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + j));
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + j));
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxIters; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j >= N) break;
        const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        const float ms[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
        const float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        float o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float den = sqrtf(vs[k]) + eps;
            const float upd = ms[k] / den;
            o[k] = xs[k] - lr * upd;
        }
        const f4 ov = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(ov, reinterpret_cast<f4*>(x + j));
    }
}

hipError_t launch_adam(float* x, const float* m, const float* v, int64_t N, float lr, float eps,
                       hipStream_t st) {
    const int64_t per_wg = (int64_t)kMaxIters * kTile;
    hipLaunchKernelGGL(adam_kernel, dim3((unsigned)((N + per_wg - 1) / per_wg)), dim3(kThreads), 0,
                       st, x, m, v, N, lr, eps);
    return hipGetLastError();
}

// Adam with the global momentum read packed: sign words and chunk scales of
// the server (the decompression every worker performs, fused into the step).
// OUT: the decompressed momentum is stored as well (nontemporal).
template <bool OUT>
__global__ __launch_bounds__(kThreads) void adam_packed_kernel(
    float* __restrict__ x, const uint32_t* __restrict__ mbits, const float* __restrict__ mscales,
    const float* __restrict__ v, float* __restrict__ m_out, int64_t N, int64_t L, float lr,
    float eps) {
    const int64_t j0 = (int64_t)blockIdx.x * kMaxIters * kTile + 4 * (int64_t)threadIdx.x;
    f4 xv[kMaxIters], vv[kMaxIters];
    uint32_t w[kMaxIters];
#pragma unroll
    for (int u = 0; u < kMaxIters; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j < N) {
            xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x + j));
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + j));
            w[u] = mbits[j >> 5];
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxIters; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j >= N) break;
        const float S = mscales[j / L];  // L is a multiple of 64: the 4 elements share a chunk
        const uint32_t word = w[u] >> (j & 31);
        const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        const float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        float o[4], mb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mb[k] = ((word >> k) & 1u) ? S : -S;
            const float den = sqrtf(vs[k]) + eps;
            const float upd = mb[k] / den;
            o[k] = xs[k] - lr * upd;
        }
        const f4 ov = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(ov, reinterpret_cast<f4*>(x + j));
        if (OUT) {
            const f4 mv = {mb[0], mb[1], mb[2], mb[3]};
            __builtin_nontemporal_store(mv, reinterpret_cast<f4*>(m_out + j));
        }
    }
}

hipError_t launch_adam_packed(float* x, const uint32_t* mbits, const float* mscales,
                              const float* v, float* m_out, int64_t N, int32_t chunks, float lr,
                              float eps, hipStream_t st) {
    const int64_t per_wg = (int64_t)kMaxIters * kTile;
    const dim3 grid((unsigned)((N + per_wg - 1) / per_wg));
    if (m_out)
        hipLaunchKernelGGL(adam_packed_kernel<true>, grid, dim3(kThreads), 0, st, x, mbits,
                           mscales, v, m_out, N, N / chunks, lr, eps);
    else
        hipLaunchKernelGGL(adam_packed_kernel<false>, grid, dim3(kThreads), 0, st, x, mbits,
                           mscales, v, m_out, N, N / chunks, lr, eps);
    return hipGetLastError();
}

// ---------------------------------------------------------------- LAMB

__global__ void fill_u32_kernel(uint32_t* p, int32_t n, uint32_t val) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = val;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// The global momentum m_t arrives decompressed (m), or PACKED: the server's
// sign words and chunk scales with the layer coefficients, decoded here as
// (bit ? S_c : -S_c) / k_l exactly as the decompression computes it, and
// stored to m_out when that is given. With PREV_PACKED the previous step's
// momentum m_{t-1} is decoded the same way from that step's words and scales
// instead of being read as floats (1/8 byte per element instead of 4).
struct PackedMomentum {
    const uint32_t* bits;   // [N/32]
    const float* scales;    // [chunks]
    const float* seg_k;     // [n_seg]
    float* out;             // [N] or null
    int64_t L;              // chunk length
    const uint32_t* pbits;  // [N/32] previous step's words (PREV_PACKED)
    const float* pscales;   // [chunks] previous step's scales (PREV_PACKED)
};

template <bool UPDATE_X, bool PACKED, bool PREV_PACKED>
__global__ __launch_bounds__(kThreads) void lamb_kernel(
    float* __restrict__ x, const float* __restrict__ m, const float* __restrict__ mp,
    float* __restrict__ vf, const float* __restrict__ v, const int64_t* __restrict__ seg_off,
    int32_t n_seg, const float* __restrict__ c_prev, uint32_t* __restrict__ keys,
    uint32_t* __restrict__ wg_max, int64_t N, float c_lr, float c_eps, float c_beta1,
    float c_beta2, PackedMomentum pk) {
    __shared__ uint32_t red[kThreads / 64];
    // workgroups across layer boundaries: maxima of layers seg0 .. seg0 + 255,
    // merged in LDS so that each layer takes one global atomic per workgroup
    __shared__ uint32_t win[kThreads];
    const float c_omb1 = 1.0f - c_beta1;
    const float c_omb2 = 1.0f - c_beta2;
    const int64_t wstart = (int64_t)blockIdx.x * kLambTiles * kTile;
    int64_t wend = wstart + (int64_t)kLambTiles * kTile;
    if (wend > N) wend = N;
    // workgroup-uniform segment test
    const int seg0 = find_segment(seg_off, n_seg, wstart);
    const bool uniform = seg_off[seg0 + 1] >= wend;

    const int64_t j0 = wstart + 4 * (int64_t)threadIdx.x;
    int seg = uniform ? seg0 : find_segment(seg_off, n_seg, j0 < N ? j0 : N - 1);
    int64_t hi = seg_off[seg + 1];
    float step = c_lr * c_prev[seg];
    uint32_t kmax = 0;
    if (!uniform) {  // workgroup-uniform branch
        win[threadIdx.x] = 0u;
        __syncthreads();
    }
    auto flush = [&](int sg, uint32_t km) {
        const int d = sg - seg0;  // >= 0: a thread's layers start at or after seg0
        if (d < kThreads) atomicMax(&win[d], km);
        else atomicMax(&keys[sg], km);
    };
    f4 mv[kLambTiles], pv[kLambTiles], fv[kLambTiles], vv[kLambTiles], xv[kLambTiles];
    uint32_t mw[kLambTiles], pw[kLambTiles];
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j < wend) {
            if (PACKED) mw[u] = pk.bits[j >> 5];
            else mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(m + j));
            if (PREV_PACKED) pw[u] = pk.pbits[j >> 5];
            else pv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(mp + j));
            fv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(vf + j));
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + j));
            if (UPDATE_X) xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x + j));
        }
    }
    // PACKED: value of a set bit for the current (chunk, layer), and
    // (PREV_PACKED) of the previous step's set bit
    int64_t q_c = -1;
    int q_seg = -1;
    float q = 0.0f, qp = 0.0f;
#pragma unroll
    for (int u = 0; u < kLambTiles; ++u) {
        const int64_t j = j0 + (int64_t)u * kTile;
        if (j >= wend) break;
        float ms[4];
        if (!PACKED) {
            ms[0] = mv[u].x;
            ms[1] = mv[u].y;
            ms[2] = mv[u].z;
            ms[3] = mv[u].w;
        }
        const int64_t c = PACKED ? j / pk.L : 0;  // L is a multiple of 64: one chunk per quad
        const uint32_t word = PACKED ? mw[u] >> (j & 31) : 0u;
        const uint32_t pword = PREV_PACKED ? pw[u] >> (j & 31) : 0u;
        float ps[4];
        if (!PREV_PACKED) {
            ps[0] = pv[u].x;
            ps[1] = pv[u].y;
            ps[2] = pv[u].z;
            ps[3] = pv[u].w;
        }
        const float fs[4] = {fv[u].x, fv[u].y, fv[u].z, fv[u].w};
        const float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        float xs[4] = {0.f, 0.f, 0.f, 0.f};
        if (UPDATE_X) {
            xs[0] = xv[u].x;
            xs[1] = xv[u].y;
            xs[2] = xv[u].z;
            xs[3] = xv[u].w;
        }
        float nf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!uniform) {
                while (j + k >= hi && seg + 1 < n_seg) {
                    if (kmax) flush(seg, kmax);
                    kmax = 0;
                    ++seg;
                    hi = seg_off[seg + 1];
                    step = c_lr * c_prev[seg];
                }
            }
            if (PACKED) {
                if (c != q_c || seg != q_seg) {
                    q_c = c;
                    q_seg = seg;
                    q = pk.scales[c] / pk.seg_k[seg];
                    if (PREV_PACKED) qp = pk.pscales[c] / pk.seg_k[seg];
                }
                ms[k] = ((word >> k) & 1u) ? q : -q;  // -S / k is exactly -(S / k)
                if (PREV_PACKED) ps[k] = ((pword >> k) & 1u) ? qp : -qp;
            }
            const float g = (ms[k] - c_beta1 * ps[k]) / c_omb1;
            const float vn = c_beta2 * fs[k] + c_omb2 * (g * g);
            nf[k] = vn;
            const float ratio = vs[k] / vn;
            if (ratio == ratio) {
                const uint32_t key = float_key(ratio);
                kmax = key > kmax ? key : kmax;
            }
            if (UPDATE_X) {
                const float den = sqrtf(vs[k]) + c_eps;
                const float upd = ms[k] / den;
                xs[k] = xs[k] - step * upd;
            }
        }
        const f4 nv = {nf[0], nf[1], nf[2], nf[3]};
        __builtin_nontemporal_store(nv, reinterpret_cast<f4*>(vf + j));
        if (PACKED && pk.out) {
            const f4 mo = {ms[0], ms[1], ms[2], ms[3]};
            __builtin_nontemporal_store(mo, reinterpret_cast<f4*>(pk.out + j));
        }
        if (UPDATE_X) {
            const f4 xo = {xs[0], xs[1], xs[2], xs[3]};
            __builtin_nontemporal_store(xo, reinterpret_cast<f4*>(x + j));
        }
    }
    // A workgroup inside one layer leaves its maximum in its own slot (the
    // finalize reduces a layer's slots): one atomic per workgroup on the
    // layer's key would serialise thousands of workgroups on one address.
    // Workgroups across a layer boundary (at most one per boundary) raise
    // the keys of their layers atomically and leave 0 (no ratio) in their
    // slot.
    if (uniform) {
        const uint32_t wm = wave_max_u32(kmax);
        if (lane_id() == 0) red[threadIdx.x >> 6] = wm;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t b = red[0];
            for (int w = 1; w < kThreads / 64; ++w) b = red[w] > b ? red[w] : b;
            wg_max[blockIdx.x] = b;
        }
    } else {
        if (kmax) flush(seg, kmax);
        __syncthreads();
        if (threadIdx.x == 0) wg_max[blockIdx.x] = 0u;
        const uint32_t w = win[threadIdx.x];
        if (w) atomicMax(&keys[seg0 + threadIdx.x], w);
    }
}

// One wave per layer: the maximum over the slots of the workgroups that
// overlap the layer (those inside it hold their maximum, the others 0),
// combined with the key the boundary workgroups raised atomically.
__global__ __launch_bounds__(kThreads) void lamb_finalize_kernel(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ wg_max,
    const int64_t* __restrict__ seg_off, int64_t n_wg, int32_t n_seg,
    const float* __restrict__ c_avg, float* __restrict__ r_prev, float* __restrict__ c_prev,
    float* __restrict__ ratio_max, float* __restrict__ err_ratio, float thr, float r_min,
    float r_max) {
    __shared__ uint32_t red[kThreads / 64];
    const int l = blockIdx.x;
    if (l >= n_seg) return;
    constexpr int64_t span = (int64_t)kLambTiles * kTile;
    constexpr int kBatch = 8;  // slot loads in flight per thread
    const int64_t a = seg_off[l], b = seg_off[l + 1];
    uint32_t km = 0;
    if (b > a) {
        const int64_t w0 = a > 0 ? a / span : 0;
        int64_t w1 = (b - 1) / span;
        if (w1 > n_wg - 1) w1 = n_wg - 1;
        for (int64_t wb = w0; wb <= w1; wb += (int64_t)kThreads * kBatch) {
            uint32_t v[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int64_t w = wb + (int64_t)q * kThreads + threadIdx.x;
                v[q] = w <= w1 ? wg_max[w] : 0u;
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) km = v[q] > km ? v[q] : km;
        }
    }
    km = wave_max_u32(km);
    if (lane_id() == 0) red[threadIdx.x >> 6] = km;
    __syncthreads();
    if (threadIdx.x != 0) return;
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) km = red[w] > km ? red[w] : km;
    km = red[0] > km ? red[0] : km;
    const uint32_t k0 = keys[l];
    const uint32_t key = k0 > km ? k0 : km;
    const float R = key ? key_float(key) : __uint_as_float(0x7FC00000u);
    const float rp = r_prev[l];
    const float Rv = (R == R) ? R : rp;
    const float lo = (1.0f - thr) * rp;
    const float hi = (1.0f + thr) * rp;
    float r = fminf(fmaxf(Rv, lo), hi);
    r = fminf(fmaxf(r, r_min), r_max);
    const float c = c_avg[l] * r;
    if (err_ratio) err_ratio[l] = c_prev[l] / c;  // c_{t-1} / c_t for the next error feedback
    r_prev[l] = r;
    c_prev[l] = c;
    if (ratio_max) ratio_max[l] = R;
}

__global__ __launch_bounds__(kThreads) void lamb_apply_kernel(
    float* __restrict__ x, const float* __restrict__ m, const float* __restrict__ v,
    const int64_t* __restrict__ seg_off, int32_t n_seg, const float* __restrict__ c, int64_t N,
    int32_t iters, float lr, float eps) {
    const int64_t j0 = (int64_t)blockIdx.x * iters * kTile + 4 * (int64_t)threadIdx.x;
    if (j0 >= N) return;
    int seg = find_segment(seg_off, n_seg, j0);
    int64_t hi = seg_off[seg + 1];
    float step = lr * c[seg];
    for (int it = 0; it < iters; ++it) {
        const int64_t j = j0 + (int64_t)it * kTile;
        if (j >= N) break;
        const f4 xv = *reinterpret_cast<const f4*>(x + j);
        const f4 mv = *reinterpret_cast<const f4*>(m + j);
        const f4 vv = *reinterpret_cast<const f4*>(v + j);
        float xs[4] = {xv.x, xv.y, xv.z, xv.w};
        const float ms[4] = {mv.x, mv.y, mv.z, mv.w};
        const float vs[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            while (j + k >= hi && seg + 1 < n_seg) {
                ++seg;
                hi = seg_off[seg + 1];
                step = lr * c[seg];
            }
            const float den = sqrtf(vs[k]) + eps;
            const float upd = ms[k] / den;
            xs[k] = xs[k] - step * upd;
        }
        const f4 xo = {xs[0], xs[1], xs[2], xs[3]};
        *reinterpret_cast<f4*>(x + j) = xo;
    }
}

hipError_t launch_lamb(const onebit_frozen_v_args& a, uint32_t* keys, uint32_t* wg_max,
                       hipStream_t st) {
    const int64_t n_wg = lamb_workgroups(a.N);
    const dim3 grid((unsigned)n_wg);
    hipLaunchKernelGGL(fill_u32_kernel, dim3((a.n_seg + 255) / 256), dim3(256), 0, st, keys,
                       a.n_seg, 0u);
    const bool packed = a.mode == 3;
    const bool prev_packed = packed && a.mp_bits != nullptr;
    PackedMomentum pk{a.m_bits, a.m_scales, a.m_seg_k, a.m_out,
                      packed ? a.N / a.m_chunks : (int64_t)1, a.mp_bits, a.mp_scales};
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st, a.x, a.m, a.m_prev, a.v_fresh, a.v,
                           a.seg_off, a.n_seg, a.c_prev, keys, wg_max, a.N, a.lr, a.eps, a.beta1,
                           a.beta2, pk);
    };
    if (a.use_c_t) {
        if (prev_packed) launch(lamb_kernel<false, true, true>);
        else if (packed) launch(lamb_kernel<false, true, false>);
        else launch(lamb_kernel<false, false, false>);
    } else {
        if (prev_packed) launch(lamb_kernel<true, true, true>);
        else if (packed) launch(lamb_kernel<true, true, false>);
        else launch(lamb_kernel<true, false, false>);
    }
    hipLaunchKernelGGL(lamb_finalize_kernel, dim3(a.n_seg), dim3(kThreads), 0, st, keys, wg_max,
                       a.seg_off, n_wg, a.n_seg, a.c_avg, a.r_prev, a.c_prev, a.ratio_max,
                       a.err_ratio, a.r_threshold, a.r_min, a.r_max);
    // second pass with c_t; a packed momentum was decompressed into m_out
    if (a.use_c_t)
        hipLaunchKernelGGL(lamb_apply_kernel, grid, dim3(kThreads), 0, st, a.x,
                           packed ? a.m_out : a.m, a.v, a.seg_off, a.n_seg, a.c_prev, a.N,
                           (int32_t)kLambTiles, a.lr, a.eps);
    return hipGetLastError();
}

}  // namespace onebit
