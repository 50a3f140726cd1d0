// Segment-wise layer scaling (1-bit LAMB page, layer-scaling paragraph) and
// materialisation of the error held by a lazy error-feedback state.
#include "common.h"

namespace onebit {

// Each workgroup covers `iters` consecutive tiles of one row; every thread
// walks the segment table forward from its first element.
template <bool DIV>
__global__ __launch_bounds__(kThreads) void layer_scale_kernel(
    float* __restrict__ buf, int64_t N, int32_t iters,
    const int64_t* __restrict__ seg_off, const float* __restrict__ seg_k, int32_t n_seg) {
    const int64_t row = blockIdx.y;  // grid (workgroups per row, batch)
    const int64_t wg = blockIdx.x;
    float* b = buf + row * N;
    const int64_t j0 = wg * (int64_t)iters * kTile + 4 * (int64_t)threadIdx.x;
    if (j0 >= N) return;
    int seg = find_segment(seg_off, n_seg, j0);
    int64_t hi = seg_off[seg + 1];
    float k = seg_k[seg];
    for (int it = 0; it < iters; ++it) {
        const int64_t j = j0 + (int64_t)it * kTile;
        if (j >= N) break;
        f4 v = *reinterpret_cast<const f4*>(b + j);
        float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            while (j + q >= hi && seg + 1 < n_seg) {
                ++seg;
                hi = seg_off[seg + 1];
                k = seg_k[seg];
            }
            x[q] = DIV ? x[q] / k : x[q] * k;
        }
        const f4 o = {x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f4*>(b + j) = o;
    }
}

hipError_t launch_layer_scale(float* buf, int64_t N, int32_t batch, const int64_t* seg_off,
                              const float* seg_k, int32_t n_seg, bool divide, hipStream_t st) {
    const int64_t tiles = (N + kTile - 1) / kTile;
    const int32_t iters = 8;
    const dim3 grid((unsigned)((tiles + iters - 1) / iters), (unsigned)batch);
    if (divide)
        hipLaunchKernelGGL(layer_scale_kernel<true>, grid, dim3(kThreads), 0, st, buf, N, iters,
                           seg_off, seg_k, n_seg);
    else
        hipLaunchKernelGGL(layer_scale_kernel<false>, grid, dim3(kThreads), 0, st, buf, N, iters,
                           seg_off, seg_k, n_seg);
    return hipGetLastError();
}

// e = ef >= 0 ? ef - s : ef + s with s the scale of the element's chunk.
__global__ __launch_bounds__(kThreads) void materialize_kernel(
    const float* __restrict__ ef, const float* __restrict__ scales, float* __restrict__ e,
    int64_t N, int32_t n, int64_t L) {
    const int64_t row = blockIdx.y;  // grid (ceil(N / 1024), rows)
    const int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (j >= N) return;
    const int64_t idx = row * N + j;
    const int64_t c = j / L;
    const float s = scales[row * n + c];
    const f4 v = *reinterpret_cast<const f4*>(ef + idx);
    const f4 o = {ef_error(v.x, s), ef_error(v.y, s), ef_error(v.z, s), ef_error(v.w, s)};
    *reinterpret_cast<f4*>(e + idx) = o;
}

hipError_t launch_materialize(const float* ef, const float* scales, float* e_out, int64_t N,
                              int32_t rows, int32_t n, hipStream_t st) {
    const dim3 grid((unsigned)((N / 4 + kThreads - 1) / kThreads), (unsigned)rows);
    hipLaunchKernelGGL(materialize_kernel, grid, dim3(kThreads), 0, st, ef, scales, e_out, N, n,
                       N / n);
    return hipGetLastError();
}

}  // namespace onebit
