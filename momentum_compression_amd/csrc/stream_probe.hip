// Stream probes shaped like the worker compression, built into a separate
// library (libonebit_probe.so) that only the benchmark loads: they give the
// ceiling of the compression's memory pattern on this GPU, not a step of the
// method.
//
// Same geometry as the compression: n rows of N floats, chunks of L = N / n,
// grid (workgroups per chunk, n * n), one 1024-element tile per 256-thread
// workgroup, nontemporal float4 loads and stores.  Every mode reads a and b
// and writes b = a + b (in place, like the error state); the mode's bits add
// the compression's other outputs:
//   1: one sign word per 8 lanes, at the compression's word address;
//   2: the workgroup's sum of |b| in binary64 (wave butterfly, LDS, barrier)
//      and one partial per workgroup.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

using f4 = float __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t or8(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    return v;
}

template <bool BITS, bool SUM>
__global__ __launch_bounds__(256) void stream_probe_kernel(const float* __restrict__ a,
                                                           float* __restrict__ b,
                                                           uint32_t* __restrict__ bits,
                                                           double* __restrict__ part, int64_t N,
                                                           int32_t n, int64_t L, int64_t bpc) {
    __shared__ double red[4];
    const int64_t pair = blockIdx.y;
    const int64_t i = pair / n, c = pair - i * n;
    const int64_t j = (int64_t)blockIdx.x * 1024 + 4 * (int64_t)threadIdx.x;
    const bool active = j < L;
    const int64_t idx = i * N + c * L + j;
    f4 g = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(a + idx));
        const f4 y = __builtin_nontemporal_load(reinterpret_cast<const f4*>(b + idx));
        g = x + y;
        __builtin_nontemporal_store(g, reinterpret_cast<f4*>(b + idx));
    }
    if (BITS) {
        const int lane8 = threadIdx.x & 7;
        const uint32_t nib = (g.x >= 0.f ? 1u : 0u) | (g.y >= 0.f ? 2u : 0u) |
                             (g.z >= 0.f ? 4u : 0u) | (g.w >= 0.f ? 8u : 0u);
        const uint32_t word = or8(nib << (4 * lane8));
        if (active && lane8 == 0) bits[idx >> 5] = word;
    }
    if (SUM) {
        double acc = (double)fabsf(g.x);
        acc += (double)fabsf(g.y);
        acc += (double)fabsf(g.z);
        acc += (double)fabsf(g.w);
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) part[pair * bpc + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

}  // namespace

extern "C" {

// Runs one probe launch on `stream`.  a, b: n rows of N floats (device,
// 16-byte aligned; b is overwritten); bits: n rows of N / 32 words; part:
// n * n * ceil(N / n / 1024) doubles.  N must be a multiple of 64 n, and
// N / n / 1024 * 256 below 2^32.  Returns 0, -2 for invalid sizes or mode,
// -6 for a HIP launch error.
int onebit_probe_stream(const float* a, float* b, uint32_t* bits, double* part, int64_t N,
                        int32_t n, int32_t mode, hipStream_t stream) {
    if (n < 1 || n > 64 || N <= 0 || N % (64 * (int64_t)n) || mode < 0 || mode > 3) return -2;
    const int64_t L = N / n;
    const int64_t bpc = (L + 1023) / 1024;
    if (bpc * 256 >= ((int64_t)1 << 32)) return -2;
    const dim3 grid((unsigned)bpc, (unsigned)((int64_t)n * n));
    switch (mode) {
        case 0:
            hipLaunchKernelGGL((stream_probe_kernel<false, false>), grid, dim3(256), 0, stream, a,
                               b, bits, part, N, n, L, bpc);
            break;
        case 1:
            hipLaunchKernelGGL((stream_probe_kernel<true, false>), grid, dim3(256), 0, stream, a, b,
                               bits, part, N, n, L, bpc);
            break;
        case 2:
            hipLaunchKernelGGL((stream_probe_kernel<false, true>), grid, dim3(256), 0, stream, a, b,
                               bits, part, N, n, L, bpc);
            break;
        default:
            hipLaunchKernelGGL((stream_probe_kernel<true, true>), grid, dim3(256), 0, stream, a, b,
                               bits, part, N, n, L, bpc);
            break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
