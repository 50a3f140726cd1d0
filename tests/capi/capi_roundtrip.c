/*
 * A plain C consumer of libonebit: device memory from hipMalloc, the C ABI
 * of include/onebit.h, no other runtime.  One reset step of the compressed
 * 1-bit Adam path on inputs whose results follow by hand: every momentum is
 * a small dyadic number and the chunk length a power of two, so each chunk
 * mean, the server average (two workers) and the Adam update (v = 1, eps =
 * 0, lr = 1) are exact, and the expected values are computed here in
 * double and compared bit for bit.
 *
 * Exit status 0 and "capi ok" on success; 1 and the first mismatch
 * otherwise; 2 when no GPU is present.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "onebit.h"

#define NW 2           /* workers */
#define NE 256         /* elements per worker row */
#define LC (NE / NW)   /* chunk length (a power of two) */

#define CHECK_HIP(x)                                                             \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            printf("HIP error %d at line %d\n", (int)e_, __LINE__);              \
            return 1;                                                            \
        }                                                                        \
    } while (0)
#define CHECK_ONEBIT(x)                                                          \
    do {                                                                         \
        int s_ = (x);                                                            \
        if (s_ != ONEBIT_OK) {                                                   \
            printf("libonebit: %s at line %d\n", onebit_strerror(s_), __LINE__); \
            return 1;                                                            \
        }                                                                        \
    } while (0)

static float momentum(int i, int j) {
    /* multiples of 1/8 in [-2, 2], zero included, signs mixed */
    int v = ((j * 7 + i * 13) % 33) - 16;
    return (float)v / 8.0f;
}

static int fail(const char* what, int k, double got, double want) {
    printf("mismatch in %s[%d]: got %.9g, want %.9g\n", what, k, got, want);
    return 1;
}

int main(void) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        printf("no GPU\n");
        return 2;
    }
    float h_m[NW * NE], h_x[NE], h_v[NE];
    for (int i = 0; i < NW; ++i)
        for (int j = 0; j < NE; ++j) h_m[i * NE + j] = momentum(i, j);
    for (int j = 0; j < NE; ++j) {
        h_x[j] = (float)(j % 5) - 2.0f;
        h_v[j] = 1.0f;
    }

    float *m, *ef, *scales, *sv_ef, *sv_scales, *mbar, *x, *v;
    uint32_t *bits, *sv_bits;
    void* ws;
    size_t ws_bytes = onebit_workspace_bytes(NE, NW, 0);
    CHECK_HIP(hipMalloc((void**)&m, sizeof h_m));
    CHECK_HIP(hipMalloc((void**)&ef, sizeof h_m));
    CHECK_HIP(hipMalloc((void**)&scales, NW * NW * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&bits, NW * NE / 8));
    CHECK_HIP(hipMalloc((void**)&sv_ef, NE * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&sv_scales, NW * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&sv_bits, NE / 8));
    CHECK_HIP(hipMalloc((void**)&mbar, NE * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&x, NE * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&v, NE * sizeof(float)));
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_HIP(hipMemcpy(m, h_m, sizeof h_m, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(x, h_x, sizeof h_x, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, h_v, sizeof h_v, hipMemcpyHostToDevice));

    /* an error that an earlier HIP call left as this thread's last error (a
       device ordinal no machine has) is neither reported by the library nor
       kept after its call */
    if (hipSetDevice(ndev + 4096) == hipSuccess || hipPeekAtLastError() == hipSuccess) {
        printf("could not leave a stale HIP error at line %d\n", __LINE__);
        return 1;
    }

    /* one reset step on the null stream */
    CHECK_ONEBIT(onebit_compress(m, ef, scales, bits, NE, NW, 0.0f, 1, NULL, NULL, 0, ws, ws_bytes,
                                 NULL));
    if (hipPeekAtLastError() != hipSuccess) {
        printf("stale HIP error kept at line %d\n", __LINE__);
        return 1;
    }
    CHECK_ONEBIT(onebit_server_reduce(bits, scales, sv_ef, sv_scales, sv_bits, mbar, NULL, NULL, 0,
                                      NE, NW, 1, ws, ws_bytes, NULL));
    onebit_frozen_v_args a;
    memset(&a, 0, sizeof a);
    a.mode = 0;
    a.N = NE;
    a.lr = 1.0f;
    a.eps = 0.0f;
    a.x = x;
    a.m = mbar;
    a.v = v;
    CHECK_ONEBIT(frozen_v_step(&a, NULL, 0, NULL));
    CHECK_HIP(hipDeviceSynchronize());

    float g_scales[NW * NW], g_svs[NW], g_mbar[NE], g_x[NE];
    uint32_t g_bits[NW * NE / 32], g_svb[NE / 32];
    CHECK_HIP(hipMemcpy(g_scales, scales, sizeof g_scales, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g_bits, bits, sizeof g_bits, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g_svs, sv_scales, sizeof g_svs, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g_svb, sv_bits, sizeof g_svb, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g_mbar, mbar, sizeof g_mbar, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g_x, x, sizeof g_x, hipMemcpyDeviceToHost));

    /* worker side: bit = (m >= 0), s[i][c] = mean |m| over the chunk */
    double s[NW][NW];
    for (int i = 0; i < NW; ++i) {
        for (int c = 0; c < NW; ++c) {
            double acc = 0.0;
            for (int j = c * LC; j < (c + 1) * LC; ++j) acc += fabs(h_m[i * NE + j]);
            s[i][c] = acc / LC;
            if (g_scales[i * NW + c] != (float)s[i][c])
                return fail("scales", i * NW + c, g_scales[i * NW + c], s[i][c]);
        }
        for (int j = 0; j < NE; ++j) {
            uint32_t bit = (g_bits[(i * NE + j) >> 5] >> (j & 31)) & 1u;
            if (bit != (h_m[i * NE + j] >= 0.0f ? 1u : 0u)) return fail("bits", i * NE + j, bit, !bit);
        }
    }
    /* server: avg = (+-s[0][c] +- s[1][c]) / 2 (exact), S[c] = mean |avg| */
    double avg[NE];
    for (int c = 0; c < NW; ++c) {
        double acc = 0.0;
        for (int j = c * LC; j < (c + 1) * LC; ++j) {
            double t = 0.0;
            for (int i = 0; i < NW; ++i) t += h_m[i * NE + j] >= 0.0f ? s[i][c] : -s[i][c];
            avg[j] = t / NW;
            acc += fabs(avg[j]);
        }
        double S = acc / LC;
        if (g_svs[c] != (float)S) return fail("server scales", c, g_svs[c], S);
        for (int j = c * LC; j < (c + 1) * LC; ++j) {
            uint32_t bit = (g_svb[j >> 5] >> (j & 31)) & 1u;
            double mb = bit ? S : -S;
            if (bit != (avg[j] >= 0.0 ? 1u : 0u)) return fail("server bits", j, bit, !bit);
            if (g_mbar[j] != (float)mb) return fail("decompressed", j, g_mbar[j], mb);
            /* Adam with v = 1, eps = 0, lr = 1: x - mbar, exact */
            if (g_x[j] != (float)(h_x[j] - mb)) return fail("x", j, g_x[j], h_x[j] - mb);
        }
    }
    printf("capi ok\n");
    return 0;
}
