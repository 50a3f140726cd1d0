/*
 * onebit.h -- C ABI of libonebit.so, the error-compensated 1-bit (and INT8)
 * compression stage of 1-bit Adam / 1-bit LAMB on AMD Instinct MI355X
 * (gfx950).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller, except
 *   the argument struct of frozen_v_step (host memory, read during the call).
 *   The library never allocates, frees or synchronises; it validates
 *   arguments on the host (before any HIP call) and enqueues kernels on
 *   `stream` only.  Results are ready when the stream reaches them.
 * - The library keeps no global state apart from the scratch array of
 *   onebit_server_reduce_noalloc (one per device, shared by every call of
 *   that entry point on the device): other calls on different streams or
 *   host threads are safe when their buffers (workspace included) are
 *   disjoint; calls that share a buffer must be ordered by the caller.
 *   Results do not depend on the stream or on the launch geometry.
 * - Return value: ONEBIT_OK (0) or a negative onebit_status.  Validation
 *   failures leave every buffer untouched.  ONEBIT_E_HIP reports a launch
 *   error from the HIP runtime.  An error that an earlier HIP call left as
 *   the calling thread's last error is cleared before the first launch, so
 *   it is neither reported nor kept.
 * - Floating point is IEEE binary32 throughout: round to nearest even, no
 *   fused multiply-add contraction, correctly rounded division and square
 *   root, subnormals kept.  NaN and Inf in the data are not errors; they
 *   propagate by IEEE rules.
 * - n simulated workers each hold a flat buffer of N elements ("row").  A row
 *   is split into n chunks of L = N / n consecutive elements; chunk c of
 *   every worker is reduced by server c.  N must be a multiple of 64 * n (the
 *   caller zero-pads).  1 <= n <= 64, L < 2^31.  N == 0 is a no-op.
 * - Sign convention: bit = 1 when x >= 0 (both zeros encode +1), 0 when
 *   x < 0 or NaN.  Packed words: element j of a row is bit (j & 31) of
 *   uint32 word (j >> 5) of that row (least significant bit first).
 * - Chunk scales are the exact mean of |x| over the chunk, rounded once to
 *   binary32 (ties to even): independent of launch geometry and bit-exact.
 * - Alignment: float buffers that are streamed (m, ef, e_out, m_out, x, v,
 *   g, err, deq, buf) must be 16-byte aligned; all others 4-byte (8 for
 *   int64 tables).
 *
 * Error-feedback state ("lazy" error)
 * -----------------------------------
 * The error of error compensation (1-bit Adam article, section 2.1:
 * e_t = g'_t - q_t) is not stored as e.  The state is the pair
 * (ef, scales): ef holds the last compensated value g' and scales its chunk
 * scale s, and e = g' - s (g' >= 0) or g' + s (g' < 0), the same single
 * binary32 operation evaluated when the next call needs it.  This halves the
 * memory passes of a step.  A zero-filled state means e = 0.
 * onebit_error_materialize() writes e out explicitly.
 */
#ifndef ONEBIT_H
#define ONEBIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ONEBIT_OK = 0,
    ONEBIT_E_NULL = -1,      /* a required pointer is NULL               */
    ONEBIT_E_SIZE = -2,      /* N, n, block or a size relation invalid,  */
                             /* or a launch beyond the device's 2^32     */
                             /* work-items along x: per row about 1.7e10 */
                             /* elements for onebit_error_materialize,   */
                             /* 3.4e10 for the INT8 entry points, 6.9e10 */
                             /* for the other per-element passes        */
    ONEBIT_E_ALIGN = -3,     /* pointer misaligned                       */
    ONEBIT_E_WORKSPACE = -4, /* workspace NULL or smaller than required  */
    ONEBIT_E_ARG = -5,       /* other invalid argument (mode, segments)  */
    ONEBIT_E_HIP = -6        /* HIP runtime reported an error on launch  */
} onebit_status;

/*
 * Worker side: reset, compensate, clamp, layer scale, chunk scale, sign pack.
 *
 * Source: 1-bit Adam article, section 2.1 (g' = g + e_prev; q = sign(g');
 * e = g' - q), applied to the momentum as in 1-bit LAMB (layer-scaling
 * paragraph); scaled sign mean(|g'|) * sign(g') from the gradient-quantisation
 * tutorial ("1-bit gradient quantisation"), per chunk; periodic reset and
 * clamp of the compensated value from the article's section 4.1 code example.
 *
 * For every worker i and element j:
 *   e      = reset ? 0 : (ef >= 0 ? ef - s_prev[i][c] : ef + s_prev[i][c])
 *   g'     = (seg ? k_l * m : m) + e
 *   g'     = clip_on ? fminf(fmaxf(g', -clip), clip) : g'
 *   ef     = g'                                   (new state)
 *   bit    = g' >= 0                              -> bits
 *   s[i][c]= mean over chunk c of |g'|            -> scales (exact, rounded)
 *
 * m       [n][N] float   momentum of each worker (read)
 * ef      [n][N] float   error state, in/out
 * scales  [n][n] float   in: previous scales (the error state's second half);
 *                        out: this call's scales, s[i][c] at i * n + c
 * bits    [n][N/32] u32  out: packed signs of g'
 * clip    clamp bound; clip <= 0 or +inf disables the clamp
 * reset   nonzero: treat the carried error as zero (first compressed step,
 *         periodic reset)
 * seg_off [n_seg+1] int64, seg_k [n_seg] float: optional (both NULL and
 *         n_seg == 0 to disable) per-layer coefficients over the N elements
 *         of a row; seg_off ascending, seg_off[0] = 0, seg_off[n_seg] = N
 *         (1-bit LAMB page, layer-scaling paragraph: x k before compression)
 * ws, ws_bytes  device workspace of at least onebit_workspace_bytes(N, n,
 *         n_seg) bytes; contents need no initialisation and are scratch
 */
int onebit_compress(const float* m, float* ef, float* scales, uint32_t* bits,
                    int64_t N, int32_t n, float clip, int32_t reset,
                    const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Server side: unpack and average n workers, compensate, chunk scale, pack;
 * optionally decompress the global momentum.
 *
 * Source: 1-bit LAMB page, experiments paragraph (compressed all-to-all /
 * all-gather backend: server c receives chunk c of every worker, averages,
 * error-compensates and re-compresses; every worker decompresses all server
 * chunks) and layer-scaling paragraph (divide by k_l after communication).
 *
 * For every chunk c and element j of it:
 *   acc = +0; for i = 0..n-1: acc = acc + (bit_i ? s[i][c] : -s[i][c])
 *   avg = acc / n
 *   E   = reset ? 0 : (ef >= 0 ? ef - S_prev[c] : ef + S_prev[c])
 *   g'' = avg + E;   ef = g'';   B = g'' >= 0;   S[c] = mean |g''| (exact)
 *   m_out = (B ? S[c] : -S[c]) [/ k_l]      (only when m_out != NULL)
 *
 * bits    [n][N/32] u32, scales [n][n] float: the worker outputs
 * ef      [N] float  server error state, in/out
 * sv_scales [n] float  in: previous server scales; out: S
 * sv_bits [N/32] u32   out
 * m_out   [N] float or NULL: decompressed global momentum
 * seg_off, seg_k, n_seg  as onebit_compress (applied as / k_l to m_out)
 * ws, ws_bytes  as onebit_compress (onebit_workspace_bytes serves both)
 */
int onebit_server_reduce(const uint32_t* bits, const float* scales, float* ef,
                         float* sv_scales, uint32_t* sv_bits, float* m_out,
                         const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                         int64_t N, int32_t n, int32_t reset,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Worker side fed with gradients: the local momentum update fused into
 * onebit_compress (1-bit Adam article, section 2.1: m_t = beta1 m_{t-1} +
 * (1 - beta1) g_t, where m_{t-1} is the global momentum every worker
 * decompressed in the previous step).  The previous global momentum is read
 * packed, as the server left it: sign words mb_bits [N/32] and chunk scales
 * mb_scales [n] (divided by k_l when a layer table is given).  Per element
 *   mbar = (bit ? S[c] : -S[c]) [/ k_l]
 *   m    = beta1 * mbar + (1 - beta1) * g        (1 - beta1 rounded once)
 * and then exactly onebit_compress on m.  m is never written to memory.
 * Pass the server's sv_bits / sv_scales of step t-1 before calling
 * onebit_server_reduce for step t (a zero-filled pair means mbar = 0).
 */
int onebit_compress_grad(const float* g, const uint32_t* mb_bits, const float* mb_scales,
                         float beta1, float* ef, float* scales, uint32_t* bits,
                         int64_t N, int32_t n, float clip, int32_t reset,
                         const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Options of the extended calls.
 * ONEBIT_UNIT_SCALE: the unscaled 1-bit sign of the 1-bit Adam article,
 * section 2.1 (q = sign(g'), i.e. every chunk scale is 1; e = g' -+ 1), at
 * the worker and, in onebit_server_reduce_ex, at the server.
 * ONEBIT_KEEP_PREV (onebit_server_reduce_ex only): sv_scales holds 2n floats.
 * [0, n) are the scales as without the flag (the previous step's on entry,
 * part of the server's error state; this step's on return), and [n, 2n)
 * receives the values [0, n) held on entry, so the previous step's scales
 * stay available next to its sign words (frozen_v_step mode 3, mp_scales).
 * The sign words need no such copy: they are output only, so a caller can
 * alternate two sv_bits buffers.
 */
#define ONEBIT_UNIT_SCALE 1u
#define ONEBIT_KEEP_PREV 2u

/*
 * onebit_compress and onebit_compress_grad in one call, plus the variants.
 *   m         momentum [n][N], or the gradient when mb_bits != NULL
 *             (mb_bits, mb_scales, beta1: as onebit_compress_grad)
 *   seg_err_ratio [n_seg] or NULL: step-ratio-scaled error feedback of the
 *             1-bit LAMB page (analysis paragraph): the carried error of an
 *             element of layer l is multiplied by seg_err_ratio[l]
 *             (c_{t-2} / c_{t-1}, as frozen_v_step's err_ratio writes it)
 *             before it is added; needs seg_off / seg_k
 *   flags     0 or ONEBIT_UNIT_SCALE
 */
int onebit_compress_ex(const float* m, const uint32_t* mb_bits, const float* mb_scales,
                       float beta1, float* ef, float* scales, uint32_t* bits,
                       int64_t N, int32_t n, float clip, int32_t reset,
                       const int64_t* seg_off, const float* seg_k, const float* seg_err_ratio,
                       int32_t n_seg, uint32_t flags, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * onebit_server_reduce with the variants of onebit_compress_ex: the server
 * error E is multiplied by seg_err_ratio[l] of its element's layer before it
 * is added (NULL: no factor), ONEBIT_UNIT_SCALE makes every S[c] = 1, and
 * ONEBIT_KEEP_PREV keeps the scales found on entry in sv_scales[n .. 2n).
 */
int onebit_server_reduce_ex(const uint32_t* bits, const float* scales, float* ef,
                            float* sv_scales, uint32_t* sv_bits, float* m_out,
                            const int64_t* seg_off, const float* seg_k,
                            const float* seg_err_ratio, int32_t n_seg, int64_t N, int32_t n,
                            int32_t reset, uint32_t flags, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * onebit_server_reduce_ex for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: the per-workgroup partial sums of the
 * chunk means go to a fixed scratch array of 8 MiB (2^20 doubles) that the
 * library holds, one copy per device, until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the scratch's device address is looked up on the first call on a device.
 * Arguments, layouts and results are exactly those of
 * onebit_server_reduce_ex (bit-identical outputs), on the current device
 * (the stream must belong to it).
 * Limit: the server needs one double per workgroup of 2048 elements of a
 * chunk, n * ceil(N / n / 2048) of them; calls needing more than 2^20 (N
 * above about 2^31 elements) return ONEBIT_E_WORKSPACE before any launch.
 * The scratch keeps the last call's contents; each call writes every
 * partial it reads, so nothing needs clearing.  Calls that
 * overlap on one device (different streams, or host threads) share the one
 * scratch and race: serialise them.
 */
int onebit_server_reduce_noalloc(const uint32_t* bits, const float* scales, float* ef,
                                 float* sv_scales, uint32_t* sv_bits, float* m_out,
                                 const int64_t* seg_off, const float* seg_k,
                                 const float* seg_err_ratio, int32_t n_seg, int64_t N,
                                 int32_t n, int32_t reset, uint32_t flags, hipStream_t stream);

/*
 * Decompress only: m_out = (B ? S[c] : -S[c]) [/ k_l] from server words and
 * scales (what every worker computes after the all-gather phase).
 */
int onebit_decompress(const uint32_t* sv_bits, const float* sv_scales, float* m_out,
                      const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                      int64_t N, int32_t n, hipStream_t stream);

/*
 * Write out the error e of an error-feedback state:
 *   e[r][j] = ef[r][j] >= 0 ? ef[r][j] - scales[r*n + c] : ef[r][j] + scales[r*n + c]
 * with c = j / (N / n).  rows = n for the worker state, 1 for the server.
 */
int onebit_error_materialize(const float* ef, const float* scales, float* e_out,
                             int64_t N, int32_t rows, int32_t n, hipStream_t stream);

/*
 * Segment-wise layer scaling of a [batch][N] buffer, in place:
 * buf = divide ? buf / k_l : buf * k_l.
 * Source: 1-bit LAMB page, layer-scaling paragraph.
 */
int lamb_layer_scale(float* buf, int64_t N, int32_t batch,
                     const int64_t* seg_off, const float* seg_k, int32_t n_seg,
                     int32_t divide, hipStream_t stream);

/*
 * Frozen-variance parameter step.
 *
 * mode 0, Adam (1-bit Adam article, sections 2.1 and 6; 1-bit LAMB page,
 * algorithm paragraph for the frozen denominator):
 *   x = x - lr * (m / (sqrtf(v) + eps))
 *
 * mode 1, LAMB (1-bit LAMB page, algorithm and analysis paragraphs):
 *   g   = (m - beta1 * m_prev) / (1 - beta1)
 *   v_f = beta2 * v_f + (1 - beta2) * (g * g)
 *   R_l = max over layer l of v / v_f   (NaN skipped, +inf kept, +0 > -0)
 *   r_l = fminf(fmaxf(R_l, (1-thr) r_prev_l), (1+thr) r_prev_l), then the
 *         same clip to [r_min, r_max]; a layer without a valid ratio keeps
 *         r_prev_l
 *   c_l = c_avg_l * r_l
 *   x   = x - (lr * c_used_l) * (m / (sqrtf(v) + eps))
 *   where c_used = c_prev (coefficient of the previous step; default) or the
 *   new c (use_c_t != 0, which costs a second pass).  On return r_prev and
 *   c_prev hold r_t and c_t; ratio_max (optional) holds R (NaN: none).
 *   First compressed step: r_prev = 1, c_prev = c_avg, v_f = v.
 *   ws: device workspace of at least frozen_v_workspace_bytes(N, n_seg)
 *   bytes, 256-byte aligned (layer maxima; mode 1 only, modes 0 and 2 take
 *   none).  Calls that share a workspace must not overlap.
 *
 * mode 2, Adam with the global momentum given packed (the decompression every
 * worker performs, fused into the step): m is ignored and
 *   mbar = m_bits bit ? m_scales[c] : -m_scales[c],  c = j / (N / m_chunks)
 *   x = x - lr * (mbar / (sqrtf(v) + eps))
 * m_bits [N/32], m_scales [m_chunks]; N a multiple of 64 * m_chunks.
 * m_out [N] (optional, 16-byte aligned): also receives mbar, the same values
 * onebit_decompress writes, so a caller that keeps the decompressed momentum
 * reads the packed words once for both.
 *
 * mode 3, LAMB (as mode 1) with the global momentum given packed: m is
 * ignored and
 *   m_t = (m_bits bit ? m_scales[c] : -m_scales[c]) / m_seg_k[l]
 * for element j of chunk c = j / (N / m_chunks) and layer l, the values
 * onebit_decompress writes with the layer table.  m_out [N] receives m_t
 * (the caller's next m_prev); it is optional unless use_c_t is set, whose
 * second pass reads it.  m_out must not overlap m_prev.
 * With mp_bits and mp_scales (both or neither; 4-byte aligned) the previous
 * momentum is read packed as well: the previous step's server words and
 * scales, decoded with the same layer table,
 *   m_{t-1} = (mp_bits bit ? mp_scales[c] : -mp_scales[c]) / m_seg_k[l],
 * which are exactly the values that step's m_out held; m_prev is then not
 * read and may be NULL.  This holds from the second compressed step on (the
 * first one's m_{t-1} is the warmup momentum, given as m_prev).  The words
 * and scales are read only; the caller keeps them from the previous step
 * (the server overwrites its own output buffers).
 */
typedef struct onebit_frozen_v_args {
    int32_t mode;          /* 0: Adam, 1: LAMB, 2: Adam packed, 3: LAMB packed */
    int32_t use_c_t;       /* LAMB: 0 = update with c_{t-1}, 1 = with c_t     */
    int64_t N;
    float lr, eps, beta1, beta2;
    float r_threshold, r_min, r_max;
    int32_t n_seg;         /* LAMB: number of layers                          */
    float* x;              /* [N] parameters, in/out                          */
    const float* m;        /* [N] global (decompressed) momentum m_t          */
    const float* v;        /* [N] frozen variance (v_Tw)                      */
    const float* m_prev;   /* LAMB: [N] m_{t-1}                               */
    float* v_fresh;        /* LAMB: [N] fresh variance, in/out                */
    const int64_t* seg_off;/* LAMB: [n_seg+1]                                 */
    const float* c_avg;    /* LAMB: [n_seg]                                   */
    float* r_prev;         /* LAMB: [n_seg] in r_{t-1}, out r_t               */
    float* c_prev;         /* LAMB: [n_seg] in c_{t-1}, out c_t               */
    float* ratio_max;      /* LAMB: [n_seg] out, or NULL                      */
    const uint32_t* m_bits;/* mode 2: [N/32] packed global momentum           */
    const float* m_scales; /* mode 2: [m_chunks] its chunk scales             */
    int32_t m_chunks;      /* mode 2: number of chunks (server ranks)         */
    float* err_ratio;      /* LAMB: [n_seg] out, or NULL: c_{t-1} / c_t, the  */
                           /* factor for the next step's error feedback      */
    float* m_out;          /* modes 2, 3: [N] out, or NULL: mbar as           */
                           /* decompressed                                    */
    const float* m_seg_k;  /* mode 3: [n_seg] layer coefficients k_l          */
    const uint32_t* mp_bits;  /* mode 3: [N/32] m_{t-1} packed, or NULL       */
    const float* mp_scales;   /* mode 3: [m_chunks] its chunk scales, or NULL */
} onebit_frozen_v_args;

int frozen_v_step(const onebit_frozen_v_args* a, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/*
 * Block-wise INT8 stochastic rounding with optional error feedback.
 *
 * Source: gradient-quantisation tutorial, "FP32 -> INT8" (scale = max/127,
 * block-wise scales, stochastic rounding floor + Bernoulli(fraction), codes
 * clamped to [-127, 127], dequantise q * scale) and error feedback.
 *
 * For block b of `block` consecutive elements and element J:
 *   g'  = err ? g + err : g
 *   M   = max(0, max over the block of non-NaN |g'|);  scale = M / 127
 *   scale == 0: q = 0, deq = 0
 *   else x = g' / scale, f = floorf(x), p = x - f,
 *        q = fminf(fmaxf(f + (u_J < p), -127), 127),  deq = q * scale
 *   err = g' - deq                          (when err != NULL)
 *   u_J = (word J&3 of Philox4x32-10(counter = (J>>2 lo32, J>>2 hi32, step, 0),
 *          key = (seed lo32, seed hi32)) >> 8) * 2^-24
 *
 * g [N] float (read); err [N] float in/out or NULL; codes [N] int8 out;
 * block_scales [N/block] float out; deq [N] float out or NULL.
 * block in {64, 128, 256, 512, 1024}; N a multiple of block.
 */
int int8_sr_quantize(const float* g, float* err, int8_t* codes, float* block_scales,
                     float* deq, int64_t N, int32_t block, uint64_t seed, uint32_t step,
                     hipStream_t stream);

/*
 * int8_sr_quantize with the variants of the tutorial's INT8 recipe:
 *   block 0     one scale for the whole tensor (the PyTorch example's max
 *               over the tensor; one extra read pass), needs ws >= 256 bytes
 *   rounding 1  deterministic rounding to the nearest integer, halves away
 *               from zero ("FP32 -> INT8" step 1), instead of stochastic (0)
 * Otherwise as int8_sr_quantize (block 64 ... 1024; N a multiple of block
 * and of 4).
 */
int int8_quantize(const float* g, float* err, int8_t* codes, float* block_scales, float* deq,
                  int64_t N, int32_t block, int32_t rounding, uint64_t seed, uint32_t step,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Warmup phase (uncompressed steps before the compressed phase) and the
 * inputs it hands over.
 *
 * Sources: 1-bit Adam article, section 2.1 (Adam's moment recursions) and its
 * configuration block (the first warmup steps run without quantisation);
 * 1-bit LAMB page, algorithm paragraph (v_Tw and the warmup moving average
 * c_avg of LAMB's layer coefficient are kept for the compressed phase) and
 * layer-scaling paragraph (a fixed per-layer momentum scale from the average
 * momentum norm at the end of warmup).
 *
 * warmup_adam_step, on the averaged gradient g (every argument [N] float,
 * device memory, 16-byte aligned; N a multiple of 4):
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) (g * g)
 *   x = x - lr * (m / (sqrtf(v) + eps))
 * binary32, one rounding per operation in this order, 1 - beta rounded once;
 * no bias correction, no weight decay.  x, m, v are updated in place.
 * N = 0 returns ONEBIT_OK without launching (pointers may then be NULL).
 */
int warmup_adam_step(float* x, float* m, float* v, const float* g, int64_t N, float lr, float eps,
                     float beta1, float beta2, hipStream_t stream);

/*
 * warmup_lamb_step: the same m and v, u = m / (sqrtf(v) + eps), then per
 * layer l = [seg_off[l], seg_off[l+1]) LAMB's trust ratio
 *   c_l = ||x_l|| / ||u_l||   (x before the step; 1 when either norm is 0)
 *   x   = x - (lr * c_l) * u
 *   c_avg_l = first ? c_l : beta_c * c_avg_l + (1 - beta_c) * c_l
 * Sx and Su are the exact sums of squares rounded once to binary64, and c_l
 * is the binary32 rounding of sqrt(Sx) / sqrt(Su) (binary64 square roots and
 * division).  The library sums in binary64 in a fixed order and certifies
 * that the binary32 result is the one the exact sums give; a layer where it
 * cannot (c_l within about 2^-47 of a rounding boundary) is summed again
 * exactly.  Results do not depend on scheduling.  c [n_seg] receives c_l.
 * seg_off [n_seg + 1] int64, device memory: seg_off[0] = 0, non-decreasing,
 * seg_off[n_seg] = N; any offset (a layer edge may fall inside a float4).
 * ws: at least warmup_workspace_bytes(N, n_seg) bytes, 256-byte aligned.
 * Two streaming passes (about 40 bytes per element).  With N = 0 every layer
 * is empty (c = 1) and x, m, v, g may be NULL.
 */
int warmup_lamb_step(float* x, float* m, float* v, const float* g, int64_t N,
                     const int64_t* seg_off, int32_t n_seg, float lr, float eps, float beta1,
                     float beta2, float beta_c, int32_t first, float* c, float* c_avg, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * lamb_momentum_scale: the per-layer coefficient k_l of the layer-scaling
 * paragraph, from the momentum m [N] at the end of warmup:
 *   a_l = sqrt(sum over layer l of m^2 / d_l)   (RMS, binary64)
 *   k_l = mean of a over layers with a > 0, divided by a_l; 1 if a_l = 0
 * with the sum of squares and the sum over layers exact, each rounded once
 * to binary64, and k_l rounded once to binary32.  As for c_l, binary64
 * sums in a fixed order are certified, and when any k_l cannot be, every
 * layer is summed again exactly.
 * k [n_seg] float out (the seg_k input of the compression entry points).
 * Same seg_off and workspace rules as warmup_lamb_step.
 */
int lamb_momentum_scale(const float* m, int64_t N, const int64_t* seg_off, int32_t n_seg,
                        float* k, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of warmup_lamb_step and lamb_momentum_scale (0 if N < 0,
 * N is not a multiple of 4 or n_seg < 1): about N / 256 bytes. */
size_t warmup_workspace_bytes(int64_t N, int32_t n_seg);

/* Workspace bytes needed by onebit_compress(_ex) / onebit_compress_grad /
 * onebit_server_reduce(_ex) for these sizes (0 if the sizes are invalid). */
size_t onebit_workspace_bytes(int64_t N, int32_t n, int32_t n_seg);

/* Workspace bytes needed by frozen_v_step in mode 1 (LAMB) for N elements
 * in n_seg layers: the layer keys plus one slot per workgroup of the pass,
 * about N / 1024 bytes (0 if N < 0, N is not a multiple of 4 or n_seg < 1). */
size_t frozen_v_workspace_bytes(int64_t N, int32_t n_seg);

/* Static description of a status code. */
const char* onebit_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ONEBIT_H */
