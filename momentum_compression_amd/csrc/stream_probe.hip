// Stream probes shaped like the worker compression, the server and the INT8
// quantiser, and plain read, write and copy streams, built into a separate
// library (libonebit_probe.so) that only the benchmark loads: they give the
// ceiling of each kernel's memory pattern on this GPU, not a step of the
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

// The server's memory operations without its arithmetic: two 1024-element
// tiles of chunk c per 256-thread workgroup (grid (workgroups per chunk, n)),
// every worker's 64 sign words of the group staged through LDS by coalesced
// wave loads exactly as the server does, the carried state read and written
// in place (nontemporal), one server sign word per 8 lanes and the binary64
// block sum.  Each lane folds its n staged words with XOR (so every word is
// read) instead of decoding and adding the workers.
// NW: the worker count when known at compile time (16), else 0 (any n).
template <int NW>
__global__ __launch_bounds__(256) void server_probe_kernel(const uint32_t* __restrict__ bits,
                                                           float* __restrict__ ef,
                                                           uint32_t* __restrict__ sv_bits,
                                                           double* __restrict__ part, int32_t n,
                                                           int64_t L, int64_t bpc, int64_t wrow) {
    __shared__ double red[4];
    extern __shared__ uint32_t stage[];  // [n][64]
    const int64_t c = blockIdx.y;
    const int64_t wg = blockIdx.x;
    const int64_t cbase = c * L;
    const int64_t g0 = wg * 2048;
    int64_t end = g0 + 2048;
    if (end > L) end = L;
    const int64_t gw = (cbase + g0) >> 5;
    const int64_t gwords = (end - g0 + 31) >> 5;
    const int nn = NW > 0 ? NW : n;
    f4 pv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t j = g0 + u * 1024 + 4 * (int64_t)threadIdx.x;
        pv[u] = f4{0.f, 0.f, 0.f, 0.f};
        if (j < end) pv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(ef + cbase + j));
    }
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int lane = threadIdx.x & 63;
        const bool okw = lane < gwords;
        for (int r0 = 0; r0 < nn; r0 += 16) {
            uint32_t v[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int i = r0 + 4 * b + wave;
                v[b] = 0u;
                if (i < nn) v[b] = bits[(int64_t)i * wrow + gw + (okw ? lane : 0)];
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int i = r0 + 4 * b + wave;
                if (i < nn) stage[i * 64 + lane] = okw ? ~v[b] : ~0u;
            }
        }
    }
    __syncthreads();
    double acc = 0.0;
    const int lane8 = threadIdx.x & 7;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t j = g0 + u * 1024 + 4 * (int64_t)threadIdx.x;
        const bool active = j < end;
        const int wl = u * 32 + (threadIdx.x >> 3);
        uint32_t x = 0;
#pragma unroll 16
        for (int i = 0; i < nn; ++i) x ^= stage[i * 64 + wl];
        const float d = (float)(x & 1u);
        const f4 g = pv[u] + f4{d, d, d, d};
        const uint32_t nib = (g.x >= 0.f ? 1u : 0u) | (g.y >= 0.f ? 2u : 0u) |
                             (g.z >= 0.f ? 4u : 0u) | (g.w >= 0.f ? 8u : 0u);
        const uint32_t word = or8(nib << (4 * lane8));
        if (active) {
            __builtin_nontemporal_store(g, reinterpret_cast<f4*>(ef + cbase + j));
            acc += (double)fabsf(g.x);
            acc += (double)fabsf(g.y);
            acc += (double)fabsf(g.z);
            acc += (double)fabsf(g.w);
            if (lane8 == 0) sv_bits[(cbase + j) >> 5] = word;
        }
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) part[c * bpc + wg] = (red[0] + red[1]) + (red[2] + red[3]);
}

// The block INT8 quantiser's memory operations without its arithmetic: two
// 1024-element tiles per 256-thread workgroup, g and the error read
// (nontemporal float4), the packed codes (4 bytes per lane), the error and
// the dequantised values written (nontemporal), and one block scale per 256
// elements (one lane in 64), as the quantiser with block 256, error
// feedback and dequantised output does.
__global__ __launch_bounds__(256) void int8_probe_kernel(const float* __restrict__ g,
                                                         float* __restrict__ err,
                                                         int8_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         float* __restrict__ deq, int64_t N) {
    const int64_t base = (int64_t)blockIdx.x * 2048;
    f4 gv[2], ev[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int64_t J = base + it * 1024 + 4 * (int64_t)threadIdx.x;
        gv[it] = f4{0.f, 0.f, 0.f, 0.f};
        ev[it] = f4{0.f, 0.f, 0.f, 0.f};
        if (J < N) {
            gv[it] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(g + J));
            ev[it] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(err + J));
        }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int64_t J = base + it * 1024 + 4 * (int64_t)threadIdx.x;
        if (J >= N) continue;
        const f4 x = gv[it] + ev[it];
        const uint32_t packed = __float_as_uint(x.x) ^ __float_as_uint(x.w);
        __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(codes + J));
        __builtin_nontemporal_store(x, reinterpret_cast<f4*>(err + J));
        __builtin_nontemporal_store(x * 0.5f, reinterpret_cast<f4*>(deq + J));
        if ((threadIdx.x & 63) == 0) scales[J / 256] = x.y;
    }
}

// Plain streams over N floats with the library's access shape (one float4
// per lane, 256-thread workgroups, nontemporal loads and stores): the
// practical HBM ceilings of reading, writing, copying, and reading two
// streams while writing one back in place (the compression's mix).
// MODE 0: read a; 1: write b; 2: b = a; 3: b = a + b.  The read-only form
// stores one value only if it sees a sentinel no benchmark input holds, so
// its loads are kept.
template <int MODE>
__global__ __launch_bounds__(256) void basic_probe_kernel(const float* __restrict__ a,
                                                          float* __restrict__ b) {
    const int64_t j = (int64_t)blockIdx.x * 1024 + 4 * (int64_t)threadIdx.x;
    if (MODE == 1) {
        __builtin_nontemporal_store(f4{1.f, 2.f, 3.f, 4.f}, reinterpret_cast<f4*>(b + j));
        return;
    }
    const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(a + j));
    if (MODE == 0) {
        if (x.x == -1234.5f && x.y == 1234.5f) b[j] = x.z;
        return;
    }
    if (MODE == 2) {
        __builtin_nontemporal_store(x, reinterpret_cast<f4*>(b + j));
        return;
    }
    const f4 y = __builtin_nontemporal_load(reinterpret_cast<const f4*>(b + j));
    __builtin_nontemporal_store(x + y, reinterpret_cast<f4*>(b + j));
}

// Streams with the read/write mixes of the parameter passes: R buffers read,
// the first W of them written back in place (3 and 2: the LAMB pass with
// both momenta packed, x, v_f and v_Tw read, x and v_f written; 4 and 3:
// the Adam warm-up step).  Same access shape as above.
template <int R, int W>
__global__ __launch_bounds__(256) void mix_probe_kernel(float* __restrict__ a,
                                                        float* __restrict__ b,
                                                        float* __restrict__ c,
                                                        float* __restrict__ d) {
    static_assert(R >= 1 && R <= 4 && W >= 1 && W <= R, "mix");
    const int64_t j = (int64_t)blockIdx.x * 1024 + 4 * (int64_t)threadIdx.x;
    float* const p[4] = {a, b, c, d};
    f4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p[r] + j));
    f4 sum = v[0];
#pragma unroll
    for (int r = 1; r < R; ++r) sum = sum + v[r];
#pragma unroll
    for (int w = 0; w < W; ++w)
        __builtin_nontemporal_store(v[w] * 0.5f + sum, reinterpret_cast<f4*>(p[w] + j));
}

}  // namespace

extern "C" {

// Runs one read/write mix probe launch on `stream`: a, b, c, d N floats each
// (device, 16-byte aligned; d may be NULL when reads is 3), the first
// `reads` of them read and the first `writes` written back in place.
// (reads, writes) must be (3, 2) or (4, 3); N a positive multiple of 1024
// with N / 4 below 2^32.  Returns 0, -2 for an invalid size or mix, -6 for a
// HIP launch error.
int onebit_probe_mix(float* a, float* b, float* c, float* d, int64_t N, int32_t reads,
                     int32_t writes, hipStream_t stream) {
    if (N <= 0 || N % 1024 || N / 4 >= ((int64_t)1 << 32)) return -2;
    const bool m32 = reads == 3 && writes == 2, m43 = reads == 4 && writes == 3;
    if (!m32 && !m43) return -2;
    (void)hipGetLastError();  // drop an error an earlier call left behind
    const dim3 grid((unsigned)(N / 1024));
    if (m32) hipLaunchKernelGGL((mix_probe_kernel<3, 2>), grid, dim3(256), 0, stream, a, b, c, d);
    else hipLaunchKernelGGL((mix_probe_kernel<4, 3>), grid, dim3(256), 0, stream, a, b, c, d);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Runs one plain stream probe launch on `stream`: a and b N floats each
// (device, 16-byte aligned; b is overwritten by modes 1 to 3), mode 0 read
// a, 1 write b, 2 copy a to b, 3 b = a + b.  N must be a positive multiple
// of 1024 with N / 4 below 2^32.  Returns 0, -2 for an invalid size or
// mode, -6 for a HIP launch error.
int onebit_probe_basic(const float* a, float* b, int64_t N, int32_t mode, hipStream_t stream) {
    if (N <= 0 || N % 1024 || mode < 0 || mode > 3) return -2;
    if (N / 4 >= ((int64_t)1 << 32)) return -2;
    (void)hipGetLastError();  // drop an error an earlier call left behind
    const dim3 grid((unsigned)(N / 1024));
    switch (mode) {
        case 0: hipLaunchKernelGGL(basic_probe_kernel<0>, grid, dim3(256), 0, stream, a, b); break;
        case 1: hipLaunchKernelGGL(basic_probe_kernel<1>, grid, dim3(256), 0, stream, a, b); break;
        case 2: hipLaunchKernelGGL(basic_probe_kernel<2>, grid, dim3(256), 0, stream, a, b); break;
        default: hipLaunchKernelGGL(basic_probe_kernel<3>, grid, dim3(256), 0, stream, a, b); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

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
    (void)hipGetLastError();  // drop an error an earlier call left behind
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

// Runs one server probe launch on `stream`: bits n rows of `pitch` words
// each holding a worker's N / 32 sign words (pitch 0 means N / 32, the
// library's layout), ef N floats (the server state, 16-byte aligned,
// overwritten), sv_bits N / 32 words, part n * ceil(N / n / 2048) doubles.
// N must be a multiple of 64 n and pitch 0 or at least N / 32.  Returns 0,
// -2 for invalid sizes, -6 for a HIP launch error.
int onebit_probe_server(const uint32_t* bits, float* ef, uint32_t* sv_bits, double* part,
                        int64_t N, int32_t n, int64_t pitch, hipStream_t stream) {
    if (n < 1 || n > 64 || N <= 0 || N % (64 * (int64_t)n)) return -2;
    if (pitch == 0) pitch = N >> 5;
    if (pitch < (N >> 5)) return -2;
    const int64_t L = N / n;
    const int64_t bpc = (L + 2047) / 2048;
    if (bpc * 256 >= ((int64_t)1 << 32)) return -2;
    const dim3 grid((unsigned)bpc, (unsigned)n);
    (void)hipGetLastError();  // drop an error an earlier call left behind
    const size_t lds = (size_t)n * 64 * sizeof(uint32_t);
    if (n == 16)
        hipLaunchKernelGGL(server_probe_kernel<16>, grid, dim3(256), lds, stream, bits, ef, sv_bits,
                           part, n, L, bpc, pitch);
    else
        hipLaunchKernelGGL(server_probe_kernel<0>, grid, dim3(256), lds, stream, bits, ef, sv_bits,
                           part, n, L, bpc, pitch);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Runs one INT8 probe launch on `stream`: g, err, deq N floats, codes N
// bytes, scales N / 256 floats (device; err and deq 16-byte aligned and
// overwritten).  N must be a positive multiple of 256.  Returns 0, -2 for an
// invalid size, -6 for a HIP launch error.
int onebit_probe_int8(const float* g, float* err, int8_t* codes, float* scales, float* deq,
                      int64_t N, hipStream_t stream) {
    if (N <= 0 || N % 256) return -2;
    const int64_t wgs = (N + 2047) / 2048;
    if (wgs * 256 >= ((int64_t)1 << 32)) return -2;
    (void)hipGetLastError();  // drop an error an earlier call left behind
    hipLaunchKernelGGL(int8_probe_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, g, err, codes,
                       scales, deq, N);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
