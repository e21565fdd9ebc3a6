/*
 * A plain C99 caller of libhkg through include/hkg.h and the HIP runtime API
 * only (no Python, no torch): small-integer bf16 and e4m3 GEMMs, one with row
 * pitches, checked bit for bit against sums formed here, plus a rejected call.
 * Small integers keep every fp32 partial sum exact, so the only rounding is
 * the final fp32 -> bf16 round-to-nearest-even, done here the same way.
 * Test infrastructure: built by __graft_entry__.build(), run by the GPU tests.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hkg.h"

#define CHECK_HIP(x)                                                            \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s:%d HIP error %d\n", __FILE__, __LINE__, (int)e_); \
            return 2;                                                           \
        }                                                                       \
    } while (0)

static uint32_t lcg_state = 12345u;
static int small_int(void) /* uniform in -4 .. 4 */
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (int)((lcg_state >> 16) % 9u) - 4;
}

static uint16_t bf16_of_float_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* OCP e4m3 code of an integer in -4 .. 4 (exponent bias 7, 3 mantissa bits). */
static uint8_t e4m3_of_int(int v)
{
    static const uint8_t mag[5] = {0x00, 0x38, 0x40, 0x44, 0x48};
    uint8_t c = mag[v < 0 ? -v : v];
    return (uint8_t)(v < 0 ? (c | 0x80u) : c);
}

/* C[m][n] = sum_k a[m][k] * b[n][k] for one layout; returns mismatches. */
static long check(const int *a, const int *b, const uint16_t *c, int M, int N, int K, long ldc,
                  float scale)
{
    long bad = 0;
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            long s = 0;
            for (int k = 0; k < K; ++k)
                s += (long)a[(long)m * K + k] * b[(long)n * K + k];
            const uint16_t want = bf16_of_float_rne((float)s * scale);
            if (c[(long)m * ldc + n] != want && bad++ < 5)
                fprintf(stderr, "C[%d][%d] = 0x%04x, want 0x%04x\n", m, n, c[(long)m * ldc + n], want);
        }
    return bad;
}

int main(void)
{
    const int M = 300, N = 200, K = 144;      /* ragged tiles; K % 16 == 0 for e4m3 */
    const long lda = K + 16, ldc = N + 8;     /* the pitched call's row pitches      */
    int *a = malloc(sizeof(int) * M * K), *b = malloc(sizeof(int) * N * K);
    uint16_t *ha = malloc(2 * (size_t)M * lda), *hb = malloc(2 * (size_t)N * K);
    uint8_t *qa = malloc((size_t)M * K), *qb = malloc((size_t)N * K);
    uint16_t *hc = malloc(2 * (size_t)M * ldc);
    if (!a || !b || !ha || !hb || !qa || !qb || !hc)
        return 2;
    for (long i = 0; i < (long)M * K; ++i)
        a[i] = small_int();
    for (long i = 0; i < (long)N * K; ++i)
        b[i] = small_int();

    void *dA, *dB, *dC, *qA, *qB;
    CHECK_HIP(hipMalloc(&dA, 2 * (size_t)M * lda));
    CHECK_HIP(hipMalloc(&dB, 2 * (size_t)N * K));
    CHECK_HIP(hipMalloc(&dC, 2 * (size_t)M * ldc));
    CHECK_HIP(hipMalloc(&qA, (size_t)M * K));
    CHECK_HIP(hipMalloc(&qB, (size_t)N * K));

    /* 1. dense bf16 */
    for (long m = 0; m < M; ++m)
        for (long k = 0; k < K; ++k)
            ha[m * K + k] = bf16_of_float_rne((float)a[m * K + k]);
    for (long i = 0; i < (long)N * K; ++i)
        hb[i] = bf16_of_float_rne((float)b[i]);
    CHECK_HIP(hipMemcpy(dA, ha, 2 * (size_t)M * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dB, hb, 2 * (size_t)N * K, hipMemcpyHostToDevice));
    int rc = hkg_gemm_bf16(M, N, K, dA, dB, dC, NULL, NULL);
    if (rc != HKG_OK) {
        fprintf(stderr, "hkg_gemm_bf16: %s (HIP %d)\n", hkg_status_string(rc), hkg_last_hip_error());
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hc, dC, 2 * (size_t)M * N, hipMemcpyDeviceToHost));
    long bad = check(a, b, hc, M, N, K, N, 1.0f);

    /* 2. bf16 with row pitches: A rows lda apart, C rows ldc apart */
    for (long m = 0; m < M; ++m)
        for (long k = 0; k < lda; ++k)
            ha[m * lda + k] = k < K ? bf16_of_float_rne((float)a[m * K + k]) : 0x7FC0u; /* NaN pad */
    for (long i = 0; i < (long)M * ldc; ++i)
        hc[i] = 0x1234u;
    CHECK_HIP(hipMemcpy(dA, ha, 2 * (size_t)M * lda, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dC, hc, 2 * (size_t)M * ldc, hipMemcpyHostToDevice));
    hkg_gemm_opts opts;
    memset(&opts, 0, sizeof opts);
    opts.lda = lda;
    opts.ldc = ldc;
    rc = hkg_gemm_bf16_ex(M, N, K, dA, dB, dC, NULL, NULL, &opts);
    if (rc != HKG_OK) {
        fprintf(stderr, "hkg_gemm_bf16_ex: %s\n", hkg_status_string(rc));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hc, dC, 2 * (size_t)M * ldc, hipMemcpyDeviceToHost));
    bad += check(a, b, hc, M, N, K, ldc, 1.0f);
    for (long m = 0; m < M; ++m)
        for (long n = N; n < ldc; ++n)
            bad += hc[m * ldc + n] != 0x1234u;

    /* 3. e4m3 with scales 0.5 and 4 */
    for (long i = 0; i < (long)M * K; ++i)
        qa[i] = e4m3_of_int(a[i]);
    for (long i = 0; i < (long)N * K; ++i)
        qb[i] = e4m3_of_int(b[i]);
    CHECK_HIP(hipMemcpy(qA, qa, (size_t)M * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(qB, qb, (size_t)N * K, hipMemcpyHostToDevice));
    rc = hkg_gemm_fp8(M, N, K, qA, qB, 0.5f, 4.0f, dC, NULL, NULL);
    if (rc != HKG_OK) {
        fprintf(stderr, "hkg_gemm_fp8: %s\n", hkg_status_string(rc));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hc, dC, 2 * (size_t)M * N, hipMemcpyDeviceToHost));
    bad += check(a, b, hc, M, N, K, N, 2.0f);

    /* 4. a rejected call launches nothing and says why */
    rc = hkg_gemm_bf16(M, N, K - 1, dA, dB, dC, NULL, NULL);
    if (rc != HKG_ERR_SHAPE || strlen(hkg_status_string(rc)) == 0)
        ++bad;

    hipFree(dA);
    hipFree(dB);
    hipFree(dC);
    hipFree(qA);
    hipFree(qB);
    if (bad) {
        fprintf(stderr, "%ld mismatches\n", bad);
        return 1;
    }
    printf("C API OK: %dx%dx%d bf16, bf16 with pitches, e4m3, rejected call\n", M, N, K);
    return 0;
}
