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

}  // namespace

// wg_first[l] = number of workgroups of layers 0 .. l-1 (l = 0 .. n_seg), by
// one workgroup: each thread sums a contiguous run of layers, thread 0 scans
// the 256 run totals, then each thread writes its run's prefixes.
__global__ __launch_bounds__(kThreads) void layer_plan_kernel(const int64_t* __restrict__ seg_off,
                                                              int32_t n_seg, int64_t N,
                                                              int64_t* __restrict__ wg_first) {
    __shared__ int64_t part[kThreads];
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
// moving average.
__global__ __launch_bounds__(kThreads) void warmup_lamb_finalize_kernel(
    const double2* __restrict__ part, const int64_t* __restrict__ wg_first, int32_t n_seg,
    int64_t n_wg, float* __restrict__ c_out, float* __restrict__ c_avg, float b_c,
    int32_t first) {
    __shared__ double red[kThreads / 64];
    const int l = blockIdx.x;
    if (l >= n_seg) return;
    const int64_t w1 = wg_first[l + 1] < n_wg ? wg_first[l + 1] : n_wg;
    const double2 t = slot_sum(part, wg_first[l], w1, red);
    if (threadIdx.x != 0) return;
    const double sx = t.x, su = t.y;
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
// then k_l.
__global__ __launch_bounds__(kThreads) void momentum_scale_kernel(const double* __restrict__ rms,
                                                                  int32_t n_seg,
                                                                  float* __restrict__ k) {
    __shared__ double red[kThreads / 64];
    __shared__ double bc[2];
    double s = 0.0, cnt = 0.0;
    for (int l = threadIdx.x; l < n_seg; l += kThreads) {
        const double a = rms[l];
        if (a > 0.0) {
            s += a;
            cnt += 1.0;
        }
    }
    const double ts = block_sum_f64(s, red);
    __syncthreads();
    const double tc = block_sum_f64(cnt, red);
    if (threadIdx.x == 0) {
        bc[0] = ts;
        bc[1] = tc;
    }
    __syncthreads();
    const double mean = bc[1] > 0.0 ? bc[0] / bc[1] : 0.0;
    for (int l = threadIdx.x; l < n_seg; l += kThreads) {
        const double a = rms[l];
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

hipError_t launch_warmup_lamb(const WarmupLambArgs& a, const WarmupWs& ws, hipStream_t st) {
    const int64_t n_wg = layer_grid(a.N, a.n_seg);
    const dim3 grid((unsigned)n_wg);
    hipLaunchKernelGGL(layer_plan_kernel, dim3(1), dim3(kThreads), 0, st, a.seg_off, a.n_seg, a.N,
                       ws.wg_first);
    hipLaunchKernelGGL(warmup_lamb_moments_kernel, grid, dim3(kThreads), 0, st, a.x, a.m, a.v, a.g,
                       a.seg_off, ws.wg_first, a.n_seg, a.N, ws.part, a.eps, a.beta1, a.beta2);
    hipLaunchKernelGGL(warmup_lamb_finalize_kernel, dim3(a.n_seg), dim3(kThreads), 0, st, ws.part,
                       ws.wg_first, a.n_seg, n_wg, a.c, a.c_avg, a.beta_c, a.first);
    hipLaunchKernelGGL(warmup_lamb_apply_kernel, grid, dim3(kThreads), 0, st, a.x, a.m, a.v,
                       a.seg_off, ws.wg_first, a.n_seg, a.N, a.c, a.lr, a.eps);
    return hipGetLastError();
}

hipError_t launch_momentum_scale(const float* m, int64_t N, const int64_t* seg_off, int32_t n_seg,
                                 float* k, const WarmupWs& ws, hipStream_t st) {
    const int64_t n_wg = layer_grid(N, n_seg);
    hipLaunchKernelGGL(layer_plan_kernel, dim3(1), dim3(kThreads), 0, st, seg_off, n_seg, N,
                       ws.wg_first);
    hipLaunchKernelGGL(momentum_sq_kernel, dim3((unsigned)n_wg), dim3(kThreads), 0, st, m, seg_off,
                       ws.wg_first, n_seg, N, ws.part);
    hipLaunchKernelGGL(momentum_rms_kernel, dim3(n_seg), dim3(kThreads), 0, st, ws.part, ws.wg_first,
                       seg_off, n_seg, N, n_wg, ws.rms);
    hipLaunchKernelGGL(momentum_scale_kernel, dim3(1), dim3(kThreads), 0, st, ws.rms, n_seg, k);
    return hipGetLastError();
}

}  // namespace onebit
