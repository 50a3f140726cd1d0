// Server-side reduction and the decompression every worker performs.
//
// Server c owns chunk c (1-bit LAMB page, experiments paragraph: the
// all-to-all phase delivers chunk c of every worker to server c; the
// all-gather phase returns the server chunks to every worker).  On one GPU the
// n workers are rows of one buffer, so both phases are addressing: the server
// workgroups read chunk c's words of every row directly.
//
// Per element: the n decoded values +-s[i][c] are accumulated in ascending
// worker order in binary32 from +0 and divided by n (a multiplication by 1/n
// when n is a power of two, which is the same correctly rounded result);
// the lazy server error is added, the sign packed, the state stored and |g''|
// summed in fp64 for the exact chunk mean.
#include "common.h"

namespace onebit {

// Words of the kServerUnroll tiles a workgroup processes together, for every
// worker, are staged through LDS with coalesced loads (32 consecutive words
// per worker and tile); each lane then reads its word per worker from LDS.
//
// Within one chunk every worker's scale is fixed, so the binary32 sum over
// the first m = min(n, 8) workers, taken in order from +0, depends only on
// their m sign bits: a 2^m-entry LDS table, built once per workgroup in the
// same order, gives it exactly.  A lane forms the 4 table indices of its 4
// elements at once: worker i's nibble (the 4 bits at the lane's offset) is
// spread to bit i of bytes 0..3 by a multiplication with 0x204081 and the
// mask 0x01010101 (the copies at shifts 0, 7, 14, 21 do not overlap, and of
// the copy at shift 7k only bit k reaches a masked position, bit 8k).
// Workers m .. n-1 are then added one by one as before.
// NW: the worker count when known at compile time (8, 16), else 0 (any n).
// RESET: the carried server error is dropped (not read).
// ERS: the step-ratio form asks the compiler for 8 waves per SIMD (64 VGPRs,
// no spills): left to itself it takes 68 at n = 16, 7 workgroups per CU in
// place of 8, and the kernel ran 3 % slower.  The other forms fit anyway and
// take the compiler's default (a minimum of 1 wave is no constraint).
template <bool ERS, int NW, bool RESET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ERS ? 8 : 1)))
void server_kernel(
    const uint32_t* __restrict__ bits, const float* __restrict__ scales, float* __restrict__ ef,
    const float* __restrict__ S_prev, uint32_t* __restrict__ sv_bits, double* __restrict__ partials,
    int64_t N, int32_t n, int64_t L, int32_t iters, int64_t bpc, int32_t pow2, float inv_n,
    const int64_t* __restrict__ seg_off, const float* __restrict__ seg_r, int32_t n_seg) {
    constexpr int kWordsPerTile = kTile / 32;              // 32
    constexpr int kGroupWords = kWordsPerTile * kServerUnroll;  // words per worker per group
    static_assert(kGroupWords == 64, "staging maps one wave to one worker's words");
    __shared__ double red[kThreads / 64];
    __shared__ float sc[64];
    __shared__ float lut[256];
    extern __shared__ uint32_t stage[];                    // [n][kGroupWords]
    const int64_t c = blockIdx.y;  // grid (bpc, n)
    const int64_t wg = blockIdx.x;
    const int64_t cbase = c * L;
    const int64_t start = wg * (int64_t)iters * kTile;
    int64_t end = start + (int64_t)iters * kTile;
    if (end > L) end = L;
    if ((int)threadIdx.x < n) sc[threadIdx.x] = scales[(int64_t)threadIdx.x * n + c];
    const int nn = NW > 0 ? NW : n;
    const int m8 = nn < 8 ? nn : 8;  // n >= 1
    __syncthreads();
    if ((int)threadIdx.x < (1 << m8)) {
        // entry b: bit i set = worker i's (inverted) sign bit set = -s[i][c]
        float a = 0.0f;
        for (int i = 0; i < m8; ++i) {
            const uint32_t b = (threadIdx.x >> i) & 1u;
            a = a + __uint_as_float((b << 31) | __float_as_uint(sc[i]));
        }
        lut[threadIdx.x] = a;
    }
    // (the first group's __syncthreads orders the table before its use)
    const float S = RESET ? 0.0f : S_prev[c];
    // a lane's 4 elements start at bit (4 tid) & 31 of their word in every
    // tile: chunk starts are multiples of 64 and workgroup starts of kTile
    const int sh = (4 * (int)threadIdx.x) & 31;
    const bool p2 = NW > 0 ? (NW & (NW - 1)) == 0 : pow2 != 0;
    const float nf = (float)n;
    const int64_t wrow = N >> 5;  // words per worker row
    const int lane8 = lane_id() & 7;
    // ERS: step-ratio factor of the carried error, per layer (segment walk)
    // (a workgroup inside one layer takes the layer's factor once)
    int seg = 0;
    int64_t seg_hi = 0;
    float rv = 1.0f;
    bool seg_uniform = true;
    if (ERS) {
        const int64_t j0 = cbase + start + 4 * (int64_t)threadIdx.x;
        seg = find_segment(seg_off, n_seg, cbase + start);
        seg_hi = seg_off[seg + 1];
        seg_uniform = seg_hi >= cbase + end;  // workgroup-uniform
        while (j0 >= seg_hi && seg + 1 < n_seg) {
            ++seg;
            seg_hi = seg_off[seg + 1];
        }
        rv = seg_r[seg];
    }

    double acc = 0.0;
    for (int it0 = 0; it0 < iters; it0 += kServerUnroll) {
        const int64_t g0 = start + (int64_t)it0 * kTile;   // first element of this group
        const int64_t gw = (cbase + g0) >> 5;             // its first word in a row
        const int64_t gwords = (end - g0 + 31) >> 5;      // words of this group inside the chunk
        __syncthreads();                                  // previous group done with `stage`
        f4 pv[kServerUnroll];
#pragma unroll
        for (int u = 0; u < kServerUnroll; ++u) {
            const int64_t j = g0 + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
            pv[u] = f4{0.f, 0.f, 0.f, 0.f};
            if (!RESET && it0 + u < iters && j < end)
                pv[u] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(ef + cbase + j));
        }
        // Staging: a group holds 64 words per worker, so wave w stages workers
        // w, w + 4, w + 8, ... with one coalesced 256-byte load each (lane l
        // takes word l); the worker, hence the row pointer, is wave-uniform.
        // The words are inverted so that a clear bit (negative value) becomes
        // the set sign bit in the decode below.  A lane past the chunk's end
        // reads the group's first word and stores all-ones (discarded later).
        {
            const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
            const int lane = lane_id();
            const bool okw = lane < gwords;
            constexpr int kBatch = 4;  // workers per wave whose loads are in flight together
            for (int r0 = 0; r0 < nn; r0 += 4 * kBatch) {
                uint32_t v[kBatch];
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    const int i = r0 + 4 * b + wave;  // wave-uniform
                    v[b] = 0u;
                    if (i < nn) v[b] = bits[(int64_t)i * wrow + gw + (okw ? lane : 0)];
                }
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    const int i = r0 + 4 * b + wave;
                    if (i < nn) stage[i * kGroupWords + lane] = okw ? ~v[b] : ~0u;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kServerUnroll; ++u) {
            const int64_t j = g0 + (int64_t)u * kTile + 4 * (int64_t)threadIdx.x;
            const bool active = it0 + u < iters && j < end;
            const int64_t J = cbase + j;
            const int wl = u * kWordsPerTile + (threadIdx.x >> 3);  // this lane's word in the group
            // first m workers: table indices, one byte per element
            uint32_t idx = 0;
#pragma unroll 8
            for (int i = 0; i < m8; ++i) {
                // rotate the lane's nibble to bits i..i+3 (so that the 24-bit
                // multiplier stays 0x204081), spread, mask to bit i of each byte
                const uint32_t w = stage[i * kGroupWords + wl];
                const uint32_t nib = __builtin_amdgcn_alignbit(w, w, (uint32_t)(sh - i) & 31u) &
                                     (0xFu << i);
                idx |= __umul24(nib, 0x204081u) & (0x01010101u << i);
            }
            float a[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] = lut[(idx >> (8 * k)) & 0xFFu];
#pragma unroll 8
            for (int i = m8; i < nn; ++i) {
                // inverted bit of element k becomes the sign of +s[i][c]
                // (one bit-field extract, one shift-or, one add)
                const uint32_t w = stage[i * kGroupWords + wl];
                const uint32_t sb = __float_as_uint(sc[i]);  // scales are >= 0
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t b = (w >> (sh + k)) & 1u;
                    a[k] = a[k] + __uint_as_float((b << 31) | sb);
                }
            }
            const float p[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
            float g[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float avg = p2 ? a[k] * inv_n : a[k] / nf;
                float e = RESET ? 0.0f : ef_error(p[k], S);
                if (ERS) {
                    if (!seg_uniform && active && J + k >= seg_hi && seg + 1 < n_seg) {
                        while (J + k >= seg_hi && seg + 1 < n_seg) {
                            ++seg;
                            seg_hi = seg_off[seg + 1];
                        }
                        rv = seg_r[seg];
                    }
                    e = rv * e;
                }
                g[k] = avg + e;
            }
            const uint32_t word = or8(sign_nibble(g[0], g[1], g[2], g[3]) << (4 * lane8));
            if (active) {
                const f4 out = {g[0], g[1], g[2], g[3]};
                __builtin_nontemporal_store(out, reinterpret_cast<f4*>(ef + J));
                acc += (double)fabsf(g[0]);
                acc += (double)fabsf(g[1]);
                acc += (double)fabsf(g[2]);
                acc += (double)fabsf(g[3]);
                if (lane8 == 0) sv_bits[J >> 5] = word;
            }
        }
    }
    const double tot = block_sum(acc, red);
    if (threadIdx.x == 0) partials[c * bpc + wg] = tot;
}

hipError_t launch_server(const uint32_t* bits, const float* scales, float* ef, const float* S_prev,
                         uint32_t* sv_bits, double* partials, int64_t N, int32_t n,
                         const ChunkPlan& plan, bool reset, const int64_t* seg_off,
                         const float* seg_r, int32_t n_seg, hipStream_t st) {
    const bool pow2 = (n & (n - 1)) == 0;
    const float inv_n = 1.0f / (float)n;  // exact for powers of two
    const size_t lds = (size_t)n * (kTile / 32) * kServerUnroll * sizeof(uint32_t);
    const dim3 grid((unsigned)plan.bpc, (unsigned)n);
    const bool ers = seg_r && seg_off && !reset;
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, bits, scales, ef, S_prev, sv_bits,
                           partials, N, n, plan.L, plan.iters, plan.bpc, pow2 ? 1 : 0, inv_n,
                           seg_off, seg_r, n_seg);
    };
    if (ers) {
        if (n == 8) launch(server_kernel<true, 8, false>);
        else if (n == 16) launch(server_kernel<true, 16, false>);
        else launch(server_kernel<true, 0, false>);
    } else if (reset) {
        if (n == 8) launch(server_kernel<false, 8, true>);
        else if (n == 16) launch(server_kernel<false, 16, true>);
        else launch(server_kernel<false, 0, true>);
    } else {
        if (n == 8) launch(server_kernel<false, 8, false>);
        else if (n == 16) launch(server_kernel<false, 16, false>);
        else launch(server_kernel<false, 0, false>);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- decompress
// Workgroups cover kDecompressTiles consecutive tiles; each lane writes 4 elements
// per tile (nontemporal: the output is consumed by a later kernel).
template <bool SEG>
__global__ __launch_bounds__(kThreads) void decompress_kernel(
    const uint32_t* __restrict__ sv_bits, const float* __restrict__ S, float* __restrict__ out,
    const int64_t* __restrict__ seg_off, const float* __restrict__ seg_k, int32_t n_seg, int64_t N,
    int64_t L) {
    const int64_t wstart = (int64_t)blockIdx.x * kDecompressTiles * kTile;
    const int64_t j0 = wstart + 4 * (int64_t)threadIdx.x;
    if (j0 >= N) return;
    uint32_t words[kDecompressTiles];
#pragma unroll
    for (int u = 0; u < kDecompressTiles; ++u) {
        const int64_t J = j0 + (int64_t)u * kTile;
        words[u] = J < N ? sv_bits[J >> 5] : 0u;
    }
    int seg = 0;
    int64_t hi = 0;
    float kv = 1.0f;
    if (SEG) {
        // workgroup-uniform search, then a short walk to this thread's start
        seg = find_segment(seg_off, n_seg, wstart);
        hi = seg_off[seg + 1];
        while (j0 >= hi && seg + 1 < n_seg) {
            ++seg;
            hi = seg_off[seg + 1];
        }
        kv = seg_k[seg];
    }
    // value of a set bit: S[c], or S[c] / k_l for the current (chunk, layer);
    // a clear bit gives its negation (the quotient of -S is exactly -(S / k))
    int64_t cur_c = -1;
    float q = 0.0f;
#pragma unroll
    for (int u = 0; u < kDecompressTiles; ++u) {
        const int64_t J = j0 + (int64_t)u * kTile;
        if (J >= N) break;
        const int64_t c = J / L;  // L is a multiple of 64, so the 4 elements share a chunk
        if (c != cur_c) {
            cur_c = c;
            q = SEG ? S[c] / kv : S[c];
        }
        const uint32_t word = words[u] >> (J & 31);
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (SEG) {
                if (J + k >= hi && seg + 1 < n_seg) {
                    while (J + k >= hi && seg + 1 < n_seg) {
                        ++seg;
                        hi = seg_off[seg + 1];
                        kv = seg_k[seg];
                    }
                    q = S[c] / kv;
                }
            }
            v[k] = ((word >> k) & 1u) ? q : -q;
        }
        const f4 o = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f4*>(out + J));
    }
}

hipError_t launch_decompress(const uint32_t* sv_bits, const float* S, float* m_out,
                             const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                             int64_t N, int32_t n, hipStream_t st) {
    const int64_t per_wg = (int64_t)kDecompressTiles * kTile;
    const dim3 grid((unsigned)((N + per_wg - 1) / per_wg));
    const int64_t L = N / n;
    if (seg_off)
        hipLaunchKernelGGL(decompress_kernel<true>, grid, dim3(kThreads), 0, st, sv_bits, S, m_out,
                           seg_off, seg_k, n_seg, N, L);
    else
        hipLaunchKernelGGL(decompress_kernel<false>, grid, dim3(kThreads), 0, st, sv_bits, S,
                           m_out, seg_off, seg_k, n_seg, N, L);
    return hipGetLastError();
}

}  // namespace onebit
