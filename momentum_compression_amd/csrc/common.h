// Internal helpers shared by the gfx950 kernels of libonebit (device side)
// and the launch code (host side).  Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "onebit.h"

namespace onebit {

using f4 = float __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;           // threads per workgroup (4 waves)
constexpr int kTile = kThreads * 4;     // elements per workgroup iteration (float4 / lane)
constexpr int kMaxIters = 4;            // tiles per workgroup: Adam (both forms), warmup Adam,
                                        // the INT8 tensor maximum pass
// Tiles per workgroup of the kernels whose best shape differs (measured on
// the full-size workloads): many one-tile workgroups for the worker
// compression, two tiles for the server and the INT8 pass.
constexpr int kCompressIters = 1;
constexpr int kCompressUnroll = 1;
constexpr int kServerIters = 2;
constexpr int kServerUnroll = 2;
constexpr int kInt8Tiles = 2;
constexpr int kDecompressTiles = 4;
constexpr int kLambTiles = 4;           // tiles per workgroup in the LAMB pass (5 streams in flight)
constexpr int kFinThreads = 1024;       // threads of a chunk-mean finalize workgroup (16 waves)

// workgroups of the LAMB pass over N elements
inline int64_t lamb_workgroups(int64_t N) {
    const int64_t span = (int64_t)kLambTiles * kTile;
    return (N + span - 1) / span;
}

// ---------------------------------------------------------------- launch plan
// One plan for the chunked kernels (worker compress, server reduce): the
// workgroups of one chunk cover consecutive tiles, `iters` tiles each.
struct ChunkPlan {
    int64_t L;        // chunk length (elements)
    int32_t iters;    // tiles per workgroup
    int64_t bpc;      // workgroups per chunk
};

// min_iters: the tiles one workgroup always covers (the server's group of
// kServerUnroll tiles), so that 4 * iters bounds every thread's additions.
ChunkPlan make_plan(int64_t L, int64_t chunks, int32_t max_iters, int32_t min_iters = 1);

// The server's plan for n workers with chunks of L elements (the workspace
// size and the launch take it from here).
inline ChunkPlan server_plan(int64_t L, int32_t n) {
    return make_plan(L, n, kServerIters, kServerUnroll);
}

// Upper bound on the number of floating-point additions any one term passes
// through in the fp64 chunk sum (per-thread sequence, wave butterfly, LDS
// tree, finalize sequence, finalize tree, division).
int64_t sum_depth(const ChunkPlan& p);
constexpr int64_t kMaxSumDepth = 12288;  // bound the finalize's certification assumes

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// OR of a value over each aligned group of 8 lanes, broadcast to all 8 lanes
// (quad swaps, then half-row mirror).  Pure register crosslane moves (DPP).
__device__ __forceinline__ uint32_t or8(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true); // row_half_mirror
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over a workgroup of kThreads threads; result valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* lds /* [kThreads/64] */) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if (lane_id() == 0) lds[w] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        r = (lds[0] + lds[1]) + (lds[2] + lds[3]);
    }
    return r;
}

// Nibble of 4 sign bits (bit k = (x_k >= 0)).
__device__ __forceinline__ uint32_t sign_nibble(float a, float b, float c, float d) {
    return (a >= 0.0f ? 1u : 0u) | (b >= 0.0f ? 2u : 0u) | (c >= 0.0f ? 4u : 0u) |
           (d >= 0.0f ? 8u : 0u);
}

// e = g' - s for g' >= 0, g' + s otherwise (NaN takes the second branch).
__device__ __forceinline__ float ef_error(float gp, float s) {
    return gp >= 0.0f ? gp - s : gp + s;
}

// Index of the segment that contains element J: largest l with off[l] <= J.
__device__ __forceinline__ int find_segment(const int64_t* off, int n_seg, int64_t J) {
    int lo = 0, hi = n_seg - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= J) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Order-preserving map of a non-NaN float to uint32 (0 is below every key).
__device__ __forceinline__ uint32_t float_key(float x) {
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace onebit

// ---------------------------------------------------------------- launchers
// Host-side entry points into each kernel file (validation happens in api.hip).
namespace onebit {

struct MeanTarget {
    const float* data;   // base of the stored values (ef)
    int64_t row_stride;  // elements between rows
    int32_t chunks;      // chunks per row (n)
    float* out;          // [rows * chunks] scales
    bool unit;           // write 1 (the unscaled sign) instead of the mean
};

hipError_t launch_mean_finalize(const double* partials, const ChunkPlan& plan, int64_t pairs,
                                MeanTarget tgt, hipStream_t st);

struct CompressArgs {
    const float* m;          // momentum [n][N], or the gradient when mb_bits != nullptr
    float* ef;               // error state [n][N]
    const float* s_prev;     // [n][n] scales: read as the previous ones, rewritten later
    uint32_t* bits;          // [n][N/32]
    double* partials;        // workspace
    int64_t N;
    int32_t n;
    float clip;
    bool clamp_on;
    bool reset;
    const int64_t* seg_off;  // layer table or nullptr
    const float* seg_k;
    int32_t n_seg;
    const uint32_t* mb_bits; // previous global momentum (server words) or nullptr
    const float* mb_scales;  // its chunk scales [n]
    float beta1;
    const float* seg_r;      // per-layer factor of the carried error, or nullptr
};

hipError_t launch_compress(const CompressArgs& a, const ChunkPlan& plan, hipStream_t st);

hipError_t launch_server(const uint32_t* bits, const float* scales, float* ef, const float* S_prev,
                         uint32_t* sv_bits, double* partials, int64_t N, int32_t n,
                         const ChunkPlan& plan, bool reset, const int64_t* seg_off,
                         const float* seg_r, int32_t n_seg, hipStream_t st);

hipError_t launch_decompress(const uint32_t* sv_bits, const float* S, float* m_out,
                             const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                             int64_t N, int32_t n, hipStream_t st);

hipError_t launch_materialize(const float* ef, const float* scales, float* e_out, int64_t N,
                              int32_t rows, int32_t n, hipStream_t st);

hipError_t launch_layer_scale(float* buf, int64_t N, int32_t batch, const int64_t* seg_off,
                              const float* seg_k, int32_t n_seg, bool divide, hipStream_t st);

hipError_t launch_adam(float* x, const float* m, const float* v, int64_t N, float lr, float eps,
                       hipStream_t st);

hipError_t launch_adam_packed(float* x, const uint32_t* mbits, const float* mscales,
                              const float* v, float* m_out, int64_t N, int32_t chunks, float lr,
                              float eps, hipStream_t st);

hipError_t launch_lamb(const onebit_frozen_v_args& a, uint32_t* keys, uint32_t* wg_max,
                       hipStream_t st);

hipError_t launch_int8(const float* g, float* err, int8_t* codes, float* scales, float* deq,
                       int64_t N, int32_t block, uint64_t seed, uint32_t step, bool nearest,
                       uint32_t* tensor_max, hipStream_t st);

// Warmup phase: layer passes with one workgroup range inside one layer.
struct WarmupLambArgs {
    float* x;
    float* m;
    float* v;
    const float* g;
    const int64_t* seg_off;
    int32_t n_seg;
    int64_t N;
    float lr, eps, beta1, beta2, beta_c;
    int32_t first;
    float* c;      // [n_seg] this step's coefficients
    float* c_avg;  // [n_seg] moving average, in/out
};

struct WarmupWs {
    int64_t* wg_first;  // [n_seg + 1] first workgroup of each layer
    double2* part;      // [layer_grid] per-workgroup binary64 sums
    double* rms;        // [n_seg]
    // exact fallback of the squared norms (taken only where the binary64
    // sums cannot certify the binary32 result)
    int32_t* need;      // [n_seg + 1] 1: the layer's sums are recomputed exactly;
                        // need[n_seg]: any layer does
    double* rms_exact;  // [n_seg]
    uint64_t* slots;    // [layer_grid][2][kExactLimbs] per-workgroup exact sums
};

// Limbs (64-bit) of an exact sum of squares of binary32 values in units of
// 2^-298: a square is below 2^554 units, so 2^31 of them stay below 2^640.
constexpr int kExactLimbs = 10;

// Upper bound on the workgroups of a layer pass (launch grid and slot count).
int64_t layer_grid(int64_t N, int32_t n_seg);

hipError_t launch_warmup_adam(float* x, float* m, float* v, const float* g, int64_t N, float lr,
                              float eps, float b1, float b2, hipStream_t st);

hipError_t launch_warmup_lamb(const WarmupLambArgs& a, const WarmupWs& ws, hipStream_t st);

hipError_t launch_momentum_scale(const float* m, int64_t N, const int64_t* seg_off, int32_t n_seg,
                                 float* k, const WarmupWs& ws, hipStream_t st);

}  // namespace onebit
