// C ABI of libonebit: host-side validation, workspace carving, launches.
// Every check runs before the first HIP call, so invalid calls touch nothing.
#include <math.h>

#include <mutex>

#include "common.h"

using namespace onebit;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int32_t kMaxWorkers = 64;

int check_rows(int64_t N, int32_t n) {
    if (n < 1 || n > kMaxWorkers) return ONEBIT_E_SIZE;
    if (N < 0) return ONEBIT_E_SIZE;
    if (N % (64 * (int64_t)n)) return ONEBIT_E_SIZE;
    // chunk length below 2^31: keeps the fp64 sums' addition depth (about
    // L / 2^18 + 21) within the finalize's certified bound
    if (N / n >= (int64_t)1 << 31) return ONEBIT_E_SIZE;
    return ONEBIT_OK;
}

// Segment tables live in device memory; the host can check only what it sees.
int check_segments(const int64_t* seg_off, const float* seg_k, int32_t n_seg, bool need_k) {
    if (seg_off == nullptr && seg_k == nullptr && n_seg == 0) return ONEBIT_OK;
    if (seg_off == nullptr || (need_k && seg_k == nullptr)) return ONEBIT_E_NULL;
    if (n_seg < 1) return ONEBIT_E_ARG;
    if (!aligned(seg_off, 8) || (seg_k && !aligned(seg_k, 4))) return ONEBIT_E_ALIGN;
    return ONEBIT_OK;
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A dispatch counts its grid in work-items with 32 bits: a launch takes at
// most 2^32 - 1 work-items along x, i.e. 16,777,215 workgroups of 256.
// Larger requests would be cut short without an error, so they are refused.
bool groups_ok(int64_t groups) { return groups <= (int64_t)(0xFFFFFFFFu / kThreads); }

// LAMB step: the layer keys, then one slot per workgroup of the pass
size_t lamb_ws_bytes(int64_t N, int32_t n_seg) {
    return round_up((size_t)n_seg * sizeof(uint32_t)) +
           round_up((size_t)lamb_workgroups(N) * sizeof(uint32_t));
}

// Warmup layer passes: plan table, per-workgroup binary64 pairs, layer RMS.
WarmupWs split_warmup_ws(void* ws, int64_t N, int32_t n_seg) {
    char* p = static_cast<char*>(ws);
    WarmupWs w;
    w.wg_first = reinterpret_cast<int64_t*>(p);
    p += round_up((size_t)(n_seg + 1) * sizeof(int64_t));
    w.part = reinterpret_cast<double2*>(p);
    p += round_up((size_t)layer_grid(N, n_seg) * 2 * sizeof(double));
    w.rms = reinterpret_cast<double*>(p);
    p += round_up((size_t)n_seg * sizeof(double));
    w.need = reinterpret_cast<int32_t*>(p);
    p += round_up((size_t)(n_seg + 1) * sizeof(int32_t));
    w.rms_exact = reinterpret_cast<double*>(p);
    p += round_up((size_t)n_seg * sizeof(double));
    w.slots = reinterpret_cast<uint64_t*>(p);
    return w;
}

size_t partial_bytes(int64_t N, int32_t n) {
    const int64_t L = N / n;
    const ChunkPlan pw = make_plan(L, (int64_t)n * n, kCompressIters);
    const ChunkPlan ps = server_plan(L, n);
    const int64_t w = pw.bpc * n * n;
    const int64_t s = ps.bpc * n;
    return round_up((size_t)(w > s ? w : s) * sizeof(double));
}

int hip_status(hipError_t e) { return e == hipSuccess ? ONEBIT_OK : ONEBIT_E_HIP; }

// The launch helpers return hipGetLastError after their launches, which
// reports the last error of any HIP call on this thread.  An entry point
// therefore drops an error an earlier call left behind (a caller's stream
// or event query that returned hipErrorNotReady, say) before its first
// launch, so that its status reflects only its own launches.
void drop_stale_error() { (void)hipGetLastError(); }

// Scratch of onebit_server_reduce_noalloc: the fp64 partial sums of the
// server's chunk means (one per workgroup), in a file-scope device array.
// Every device the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocDoubles = (size_t)1 << 20;  // 8 MiB
__device__ __align__(256) double scratch[kNoAllocDoubles];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch[kMaxDevices];  // device address of `scratch`, per device

int scratch_of_current_device(double** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ONEBIT_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ONEBIT_E_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return ONEBIT_E_HIP;
        g_scratch[dev] = static_cast<double*>(p);
    }
    *out = g_scratch[dev];
    return ONEBIT_OK;
}

}  // namespace

namespace onebit {
// the chunk-mean finalize that first copies each scale it will overwrite to
// prev (finalize.hip); ONEBIT_KEEP_PREV passes the second half of sv_scales
hipError_t launch_mean_finalize_keep(const double* partials, const ChunkPlan& plan,
                                     int64_t pairs, MeanTarget tgt, float* prev, hipStream_t st);
}  // namespace onebit

extern "C" {

const char* onebit_strerror(int status) {
    switch (status) {
        case ONEBIT_OK: return "ok";
        case ONEBIT_E_NULL: return "required pointer is NULL";
        case ONEBIT_E_SIZE: return "invalid size (N must be a multiple of 64*n, 1 <= n <= 64, N/n < 2^31; block and N must agree; grids within 2^32 work-items)";
        case ONEBIT_E_ALIGN: return "pointer misaligned (streamed float buffers need 16 bytes)";
        case ONEBIT_E_WORKSPACE: return "workspace missing or smaller than onebit_workspace_bytes()";
        case ONEBIT_E_ARG: return "invalid argument";
        case ONEBIT_E_HIP: return "HIP runtime error on launch";
        default: return "unknown status";
    }
}

size_t onebit_workspace_bytes(int64_t N, int32_t n, int32_t n_seg) {
    if (check_rows(N, n) != ONEBIT_OK || n_seg < 0) return 0;
    if (N == 0) return 256;
    return partial_bytes(N, n) + round_up((size_t)(n_seg > 0 ? n_seg : 1) * sizeof(uint32_t));
}

size_t frozen_v_workspace_bytes(int64_t N, int32_t n_seg) {
    if (N < 0 || (N % 4) || n_seg < 1) return 0;
    return lamb_ws_bytes(N, n_seg);
}

int onebit_compress_ex(const float* m, const uint32_t* mb_bits, const float* mb_scales, float beta1,
                       float* ef, float* scales, uint32_t* bits, int64_t N, int32_t n, float clip,
                       int32_t reset, const int64_t* seg_off, const float* seg_k,
                       const float* seg_err_ratio, int32_t n_seg, uint32_t flags, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    int st = check_rows(N, n);
    if (st) return st;
    if (!m || !ef || !scales || !bits) return ONEBIT_E_NULL;
    if ((mb_bits == nullptr) != (mb_scales == nullptr)) return ONEBIT_E_NULL;
    if ((st = check_segments(seg_off, seg_k, n_seg, true))) return st;
    if (seg_err_ratio && !seg_off) return ONEBIT_E_ARG;
    if (!aligned(m, 16) || !aligned(ef, 16) || !aligned(scales, 4) || !aligned(bits, 4) ||
        (mb_bits && !aligned(mb_bits, 4)) || (mb_scales && !aligned(mb_scales, 4)) ||
        (seg_err_ratio && !aligned(seg_err_ratio, 4)))
        return ONEBIT_E_ALIGN;
    if (clip != clip || beta1 != beta1 || (flags & ~ONEBIT_UNIT_SCALE)) return ONEBIT_E_ARG;
    if (N == 0) return ONEBIT_OK;
    const size_t need = onebit_workspace_bytes(N, n, n_seg);
    if (!ws || ws_bytes < need) return ONEBIT_E_WORKSPACE;
    if (!aligned(ws, 256)) return ONEBIT_E_ALIGN;

    const ChunkPlan plan = make_plan(N / n, (int64_t)n * n, kCompressIters);
    if (sum_depth(plan) > kMaxSumDepth || !groups_ok(plan.bpc)) return ONEBIT_E_SIZE;
    const bool clamp_on = clip > 0.0f && !isinf(clip);
    double* partials = static_cast<double*>(ws);
    CompressArgs a{m, ef, scales, bits, partials, N, n, clip, clamp_on, reset != 0,
                   seg_off, seg_k, n_seg, mb_bits, mb_scales, beta1, seg_err_ratio};
    drop_stale_error();
    hipError_t e = launch_compress(a, plan, stream);
    if (e != hipSuccess) return ONEBIT_E_HIP;
    MeanTarget tgt{ef, N, n, scales, (flags & ONEBIT_UNIT_SCALE) != 0};
    return hip_status(launch_mean_finalize(partials, plan, (int64_t)n * n, tgt, stream));
}

int onebit_compress(const float* m, float* ef, float* scales, uint32_t* bits, int64_t N, int32_t n,
                    float clip, int32_t reset, const int64_t* seg_off, const float* seg_k,
                    int32_t n_seg, void* ws, size_t ws_bytes, hipStream_t stream) {
    return onebit_compress_ex(m, nullptr, nullptr, 0.0f, ef, scales, bits, N, n, clip, reset,
                              seg_off, seg_k, nullptr, n_seg, 0u, ws, ws_bytes, stream);
}

int onebit_compress_grad(const float* g, const uint32_t* mb_bits, const float* mb_scales,
                         float beta1, float* ef, float* scales, uint32_t* bits, int64_t N,
                         int32_t n, float clip, int32_t reset, const int64_t* seg_off,
                         const float* seg_k, int32_t n_seg, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    if (!mb_bits || !mb_scales) return ONEBIT_E_NULL;
    return onebit_compress_ex(g, mb_bits, mb_scales, beta1, ef, scales, bits, N, n, clip, reset,
                              seg_off, seg_k, nullptr, n_seg, 0u, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Argument checks of the server calls (everything but the scratch).
int check_server(const uint32_t* bits, const float* scales, float* ef, float* sv_scales,
                 uint32_t* sv_bits, float* m_out, const int64_t* seg_off, const float* seg_k,
                 const float* seg_err_ratio, int32_t n_seg, int64_t N, int32_t n,
                 uint32_t flags) {
    int st = check_rows(N, n);
    if (st) return st;
    if (!bits || !scales || !ef || !sv_scales || !sv_bits) return ONEBIT_E_NULL;
    if ((st = check_segments(seg_off, seg_k, n_seg, true))) return st;
    if (seg_err_ratio && !seg_off) return ONEBIT_E_ARG;
    if (!aligned(bits, 4) || !aligned(scales, 4) || !aligned(ef, 16) || !aligned(sv_scales, 4) ||
        !aligned(sv_bits, 4) || (m_out && !aligned(m_out, 16)) ||
        (seg_err_ratio && !aligned(seg_err_ratio, 4)))
        return ONEBIT_E_ALIGN;
    if (flags & ~(ONEBIT_UNIT_SCALE | ONEBIT_KEEP_PREV)) return ONEBIT_E_ARG;
    if (N == 0) return ONEBIT_OK;
    const ChunkPlan plan = server_plan(N / n, n);
    if (sum_depth(plan) > kMaxSumDepth || !groups_ok(plan.bpc)) return ONEBIT_E_SIZE;
    if (m_out && !groups_ok(ceil_div(N, (int64_t)kDecompressTiles * kTile))) return ONEBIT_E_SIZE;
    return ONEBIT_OK;
}

// The server's launches on validated arguments, with the partial sums in
// `partials` (server_plan(N / n, n).bpc * n doubles).
int server_launch(const uint32_t* bits, const float* scales, float* ef, float* sv_scales,
                  uint32_t* sv_bits, float* m_out, const int64_t* seg_off, const float* seg_k,
                  const float* seg_err_ratio, int32_t n_seg, int64_t N, int32_t n,
                  int32_t reset, uint32_t flags, double* partials, hipStream_t stream) {
    const ChunkPlan plan = server_plan(N / n, n);
    drop_stale_error();
    hipError_t e = launch_server(bits, scales, ef, sv_scales, sv_bits, partials, N, n, plan,
                                 reset != 0, seg_off, seg_err_ratio, n_seg, stream);
    if (e != hipSuccess) return ONEBIT_E_HIP;
    MeanTarget tgt{ef, N, n, sv_scales, (flags & ONEBIT_UNIT_SCALE) != 0};
    // ONEBIT_KEEP_PREV: the finalize copies the scales it replaces to [n, 2n)
    e = launch_mean_finalize_keep(partials, plan, n, tgt,
                                  (flags & ONEBIT_KEEP_PREV) ? sv_scales + n : nullptr, stream);
    if (e != hipSuccess) return ONEBIT_E_HIP;
    if (m_out)
        return hip_status(
            launch_decompress(sv_bits, sv_scales, m_out, seg_off, seg_k, n_seg, N, n, stream));
    return ONEBIT_OK;
}

}  // namespace

extern "C" {

int onebit_server_reduce_ex(const uint32_t* bits, const float* scales, float* ef,
                            float* sv_scales, uint32_t* sv_bits, float* m_out,
                            const int64_t* seg_off, const float* seg_k,
                            const float* seg_err_ratio, int32_t n_seg, int64_t N, int32_t n,
                            int32_t reset, uint32_t flags, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    int st = check_server(bits, scales, ef, sv_scales, sv_bits, m_out, seg_off, seg_k,
                          seg_err_ratio, n_seg, N, n, flags);
    if (st || N == 0) return st;
    const size_t need = onebit_workspace_bytes(N, n, n_seg);
    if (!ws || ws_bytes < need) return ONEBIT_E_WORKSPACE;
    if (!aligned(ws, 256)) return ONEBIT_E_ALIGN;
    return server_launch(bits, scales, ef, sv_scales, sv_bits, m_out, seg_off, seg_k,
                         seg_err_ratio, n_seg, N, n, reset, flags, static_cast<double*>(ws),
                         stream);
}

int onebit_server_reduce_noalloc(const uint32_t* bits, const float* scales, float* ef,
                                 float* sv_scales, uint32_t* sv_bits, float* m_out,
                                 const int64_t* seg_off, const float* seg_k,
                                 const float* seg_err_ratio, int32_t n_seg, int64_t N, int32_t n,
                                 int32_t reset, uint32_t flags, hipStream_t stream) {
    int st = check_server(bits, scales, ef, sv_scales, sv_bits, m_out, seg_off, seg_k,
                          seg_err_ratio, n_seg, N, n, flags);
    if (st || N == 0) return st;
    const ChunkPlan plan = server_plan(N / n, n);
    if ((size_t)(plan.bpc * n) > kNoAllocDoubles) return ONEBIT_E_WORKSPACE;
    double* partials = nullptr;
    if ((st = scratch_of_current_device(&partials))) return st;
    // every partial the finalize reads is written by this call's server
    // kernel first, so the scratch needs no clearing
    return server_launch(bits, scales, ef, sv_scales, sv_bits, m_out, seg_off, seg_k,
                         seg_err_ratio, n_seg, N, n, reset, flags, partials, stream);
}

int onebit_server_reduce(const uint32_t* bits, const float* scales, float* ef, float* sv_scales,
                         uint32_t* sv_bits, float* m_out, const int64_t* seg_off,
                         const float* seg_k, int32_t n_seg, int64_t N, int32_t n, int32_t reset,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
    return onebit_server_reduce_ex(bits, scales, ef, sv_scales, sv_bits, m_out, seg_off, seg_k,
                                   nullptr, n_seg, N, n, reset, 0u, ws, ws_bytes, stream);
}

int onebit_decompress(const uint32_t* sv_bits, const float* sv_scales, float* m_out,
                      const int64_t* seg_off, const float* seg_k, int32_t n_seg, int64_t N,
                      int32_t n, hipStream_t stream) {
    int st = check_rows(N, n);
    if (st) return st;
    if (!sv_bits || !sv_scales || !m_out) return ONEBIT_E_NULL;
    if ((st = check_segments(seg_off, seg_k, n_seg, true))) return st;
    if (!aligned(sv_bits, 4) || !aligned(sv_scales, 4) || !aligned(m_out, 16)) return ONEBIT_E_ALIGN;
    if (N == 0) return ONEBIT_OK;
    if (!groups_ok(ceil_div(N, (int64_t)kDecompressTiles * kTile))) return ONEBIT_E_SIZE;
    drop_stale_error();
    return hip_status(
        launch_decompress(sv_bits, sv_scales, m_out, seg_off, seg_k, n_seg, N, n, stream));
}

int onebit_error_materialize(const float* ef, const float* scales, float* e_out, int64_t N,
                             int32_t rows, int32_t n, hipStream_t stream) {
    int st = check_rows(N, n);
    if (st) return st;
    if (rows < 1 || rows > kMaxWorkers) return ONEBIT_E_SIZE;
    if (!ef || !scales || !e_out) return ONEBIT_E_NULL;
    if (!aligned(ef, 16) || !aligned(e_out, 16) || !aligned(scales, 4)) return ONEBIT_E_ALIGN;
    if (N == 0) return ONEBIT_OK;
    if (!groups_ok(ceil_div(N, kTile))) return ONEBIT_E_SIZE;
    drop_stale_error();
    return hip_status(launch_materialize(ef, scales, e_out, N, rows, n, stream));
}

int lamb_layer_scale(float* buf, int64_t N, int32_t batch, const int64_t* seg_off,
                     const float* seg_k, int32_t n_seg, int32_t divide, hipStream_t stream) {
    if (N < 0 || (N % 4) || batch < 1) return ONEBIT_E_SIZE;
    if (!buf || !seg_off || !seg_k) return ONEBIT_E_NULL;
    if (n_seg < 1) return ONEBIT_E_ARG;
    if (!aligned(buf, 16) || !aligned(seg_off, 8) || !aligned(seg_k, 4)) return ONEBIT_E_ALIGN;
    if (N == 0) return ONEBIT_OK;
    if (batch > 65535 || !groups_ok(ceil_div(ceil_div(N, kTile), 8))) return ONEBIT_E_SIZE;
    drop_stale_error();
    return hip_status(launch_layer_scale(buf, N, batch, seg_off, seg_k, n_seg, divide != 0, stream));
}

int frozen_v_step(const onebit_frozen_v_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!a) return ONEBIT_E_NULL;
    if (a->N < 0 || (a->N % 4)) return ONEBIT_E_SIZE;
    if (!groups_ok(ceil_div(a->N, (int64_t)kMaxIters * kTile)) || !groups_ok(lamb_workgroups(a->N)))
        return ONEBIT_E_SIZE;
    const bool packed_m = a->mode == 2 || a->mode == 3;  // momentum given as sign words
    if (!a->x || (!a->m && !packed_m) || !a->v) return ONEBIT_E_NULL;
    if (!aligned(a->x, 16) || !aligned(a->m, 16) || !aligned(a->v, 16)) return ONEBIT_E_ALIGN;
    if (a->mode == 0) {
        if (a->N == 0) return ONEBIT_OK;
        drop_stale_error();
        return hip_status(launch_adam(a->x, a->m, a->v, a->N, a->lr, a->eps, stream));
    }
    if (a->mode == 2) {
        if (!a->m_bits || !a->m_scales) return ONEBIT_E_NULL;
        if (a->m_chunks < 1 || a->m_chunks > kMaxWorkers || (a->N % (64 * (int64_t)a->m_chunks)))
            return ONEBIT_E_SIZE;
        if (!aligned(a->m_bits, 4) || !aligned(a->m_scales, 4) || !aligned(a->m_out, 16))
            return ONEBIT_E_ALIGN;
        if (a->N == 0) return ONEBIT_OK;
        drop_stale_error();
        return hip_status(launch_adam_packed(a->x, a->m_bits, a->m_scales, a->v, a->m_out, a->N,
                                             a->m_chunks, a->lr, a->eps, stream));
    }
    if (a->mode != 1 && a->mode != 3) return ONEBIT_E_ARG;
    // mode 3 may take the previous momentum packed instead of m_prev
    const bool prev_packed = a->mode == 3 && a->mp_bits != nullptr;
    if ((!a->m_prev && !prev_packed) || !a->v_fresh || !a->seg_off || !a->c_avg || !a->r_prev ||
        !a->c_prev)
        return ONEBIT_E_NULL;
    if (a->mode == 3) {
        if (!a->m_bits || !a->m_scales || !a->m_seg_k || (a->use_c_t && !a->m_out))
            return ONEBIT_E_NULL;
        if ((a->mp_bits == nullptr) != (a->mp_scales == nullptr)) return ONEBIT_E_NULL;
        if (a->m_chunks < 1 || a->m_chunks > kMaxWorkers || (a->N % (64 * (int64_t)a->m_chunks)))
            return ONEBIT_E_SIZE;
        if (!aligned(a->m_bits, 4) || !aligned(a->m_scales, 4) || !aligned(a->m_seg_k, 4) ||
            !aligned(a->m_out, 16) || !aligned(a->mp_bits, 4) || !aligned(a->mp_scales, 4))
            return ONEBIT_E_ALIGN;
        if (a->m_out && !prev_packed) {  // m_out must not overlap m_prev, which is read
            const uintptr_t o = (uintptr_t)a->m_out, p = (uintptr_t)a->m_prev;
            const uintptr_t bytes = (uintptr_t)a->N * sizeof(float);
            if (o < p + bytes && p < o + bytes) return ONEBIT_E_ARG;
        }
    }
    if (a->n_seg < 1) return ONEBIT_E_ARG;
    if (!groups_ok(a->n_seg)) return ONEBIT_E_SIZE;
    if (!aligned(a->m_prev, 16) || !aligned(a->v_fresh, 16) || !aligned(a->seg_off, 8) ||
        !aligned(a->c_avg, 4) || !aligned(a->r_prev, 4) || !aligned(a->c_prev, 4) ||
        (a->ratio_max && !aligned(a->ratio_max, 4)) || (a->err_ratio && !aligned(a->err_ratio, 4)))
        return ONEBIT_E_ALIGN;
    if (a->N == 0) return ONEBIT_OK;
    const size_t need = lamb_ws_bytes(a->N, a->n_seg);
    if (!ws || ws_bytes < need) return ONEBIT_E_WORKSPACE;
    if (!aligned(ws, 256)) return ONEBIT_E_ALIGN;
    uint32_t* keys = static_cast<uint32_t*>(ws);
    uint32_t* wg_max = keys + round_up((size_t)a->n_seg * sizeof(uint32_t)) / sizeof(uint32_t);
    drop_stale_error();
    return hip_status(launch_lamb(*a, keys, wg_max, stream));
}

int int8_quantize(const float* g, float* err, int8_t* codes, float* block_scales, float* deq,
                  int64_t N, int32_t block, int32_t rounding, uint64_t seed, uint32_t step,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
    if (block != 0 && block != 64 && block != 128 && block != 256 && block != 512 && block != 1024)
        return ONEBIT_E_SIZE;
    if (N < 0 || (N % 4) || (block && (N % block))) return ONEBIT_E_SIZE;
    if (!groups_ok(ceil_div(N, (int64_t)kInt8Tiles * kTile))) return ONEBIT_E_SIZE;
    if (rounding != 0 && rounding != 1) return ONEBIT_E_ARG;
    if (!g || !codes || !block_scales) return ONEBIT_E_NULL;
    if (!aligned(g, 16) || (err && !aligned(err, 16)) || !aligned(codes, 4) ||
        !aligned(block_scales, 4) || (deq && !aligned(deq, 16)))
        return ONEBIT_E_ALIGN;
    if (N == 0) return ONEBIT_OK;
    if (block == 0) {
        if (!ws || ws_bytes < 256) return ONEBIT_E_WORKSPACE;
        if (!aligned(ws, 256)) return ONEBIT_E_ALIGN;
    }
    drop_stale_error();
    return hip_status(launch_int8(g, err, codes, block_scales, deq, N, block, seed, step,
                                  rounding == 1, static_cast<uint32_t*>(ws), stream));
}

int int8_sr_quantize(const float* g, float* err, int8_t* codes, float* block_scales, float* deq,
                     int64_t N, int32_t block, uint64_t seed, uint32_t step, hipStream_t stream) {
    if (block == 0) return ONEBIT_E_SIZE;  // the per-tensor variant needs a workspace
    return int8_quantize(g, err, codes, block_scales, deq, N, block, 0, seed, step, nullptr, 0,
                         stream);
}

// ---------------------------------------------------------------- warmup

size_t warmup_workspace_bytes(int64_t N, int32_t n_seg) {
    if (N < 0 || (N % 4) || n_seg < 1) return 0;
    return round_up((size_t)(n_seg + 1) * sizeof(int64_t)) +
           round_up((size_t)layer_grid(N, n_seg) * 2 * sizeof(double)) +
           round_up((size_t)n_seg * sizeof(double)) +
           round_up((size_t)(n_seg + 1) * sizeof(int32_t)) +
           round_up((size_t)n_seg * sizeof(double)) +
           round_up((size_t)layer_grid(N, n_seg) * 2 * kExactLimbs * sizeof(uint64_t));
}

int warmup_adam_step(float* x, float* m, float* v, const float* g, int64_t N, float lr, float eps,
                     float beta1, float beta2, hipStream_t stream) {
    if (N < 0 || (N % 4) || !groups_ok(ceil_div(N, (int64_t)kMaxIters * kTile)))
        return ONEBIT_E_SIZE;
    if (N == 0) return ONEBIT_OK;
    if (!x || !m || !v || !g) return ONEBIT_E_NULL;
    if (!aligned(x, 16) || !aligned(m, 16) || !aligned(v, 16) || !aligned(g, 16))
        return ONEBIT_E_ALIGN;
    drop_stale_error();
    return hip_status(launch_warmup_adam(x, m, v, g, N, lr, eps, beta1, beta2, stream));
}

int warmup_lamb_step(float* x, float* m, float* v, const float* g, int64_t N,
                     const int64_t* seg_off, int32_t n_seg, float lr, float eps, float beta1,
                     float beta2, float beta_c, int32_t first, float* c, float* c_avg, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
    if (N < 0 || (N % 4)) return ONEBIT_E_SIZE;
    if ((N > 0 && (!x || !m || !v || !g)) || !seg_off || !c || !c_avg) return ONEBIT_E_NULL;
    if (n_seg < 1 || (first != 0 && first != 1)) return ONEBIT_E_ARG;
    if (!groups_ok(layer_grid(N, n_seg)) || !groups_ok(n_seg)) return ONEBIT_E_SIZE;
    if (!aligned(x, 16) || !aligned(m, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(seg_off, 8) || !aligned(c, 4) || !aligned(c_avg, 4))
        return ONEBIT_E_ALIGN;
    if (!ws || ws_bytes < warmup_workspace_bytes(N, n_seg)) return ONEBIT_E_WORKSPACE;
    if (!aligned(ws, 256)) return ONEBIT_E_ALIGN;
    WarmupLambArgs a;
    a.x = x;
    a.m = m;
    a.v = v;
    a.g = g;
    a.seg_off = seg_off;
    a.n_seg = n_seg;
    a.N = N;
    a.lr = lr;
    a.eps = eps;
    a.beta1 = beta1;
    a.beta2 = beta2;
    a.beta_c = beta_c;
    a.first = first;
    a.c = c;
    a.c_avg = c_avg;
    // N == 0: every layer is empty, c = 1 (the coefficient of a zero norm)
    drop_stale_error();
    return hip_status(launch_warmup_lamb(a, split_warmup_ws(ws, N, n_seg), stream));
}

int lamb_momentum_scale(const float* m, int64_t N, const int64_t* seg_off, int32_t n_seg,
                        float* k, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (N < 0 || (N % 4)) return ONEBIT_E_SIZE;
    if ((N > 0 && !m) || !seg_off || !k) return ONEBIT_E_NULL;
    if (n_seg < 1) return ONEBIT_E_ARG;
    if (!groups_ok(layer_grid(N, n_seg)) || !groups_ok(n_seg)) return ONEBIT_E_SIZE;
    if (!aligned(m, 16) || !aligned(seg_off, 8) || !aligned(k, 4)) return ONEBIT_E_ALIGN;
    if (!ws || ws_bytes < warmup_workspace_bytes(N, n_seg)) return ONEBIT_E_WORKSPACE;
    if (!aligned(ws, 256)) return ONEBIT_E_ALIGN;
    drop_stale_error();
    return hip_status(
        launch_momentum_scale(m, N, seg_off, n_seg, k, split_warmup_ws(ws, N, n_seg), stream));
}

}  // extern "C"
