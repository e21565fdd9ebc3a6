/* Every entry point of libhkg called with extreme and invalid arguments on a
 * host without a gfx950: each call must return one of the documented status
 * codes, validation must come before any device work, and every launch plan
 * that is accepted must be well formed.  Built with the host code under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/c/build.py), so an
 * out-of-bounds access or a signed overflow in argument checking fails the
 * run.  Prints "ABI EXTREMES OK" and exits 0 on success. */
#include <inttypes.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "hkg.h"

static int failures = 0;

#define EXPECT(cond, ...)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fputc('\n', stderr);                           \
            ++failures;                                    \
        }                                                  \
    } while (0)

static int is_status(int rc)
{
    return rc == HKG_OK || rc == HKG_ERR_NULL || rc == HKG_ERR_SHAPE || rc == HKG_ERR_ALIGN ||
           rc == HKG_ERR_SIZE || rc == HKG_ERR_OPTS || rc == HKG_ERR_DEVICE ||
           rc == HKG_ERR_LAUNCH || rc == HKG_ERR_OVERLAP;
}

/* values of M, N, K, pitches and grid sides: edges of every bound */
static const int64_t kVals[] = {
    INT64_MIN, -1, 0, 1, 8, 16, 32, 255, 257, 8192, ((int64_t)1 << 22) - 8,
    ((int64_t)1 << 23) - 16, (int64_t)1 << 23, ((int64_t)1 << 31) - 1, (int64_t)1 << 31,
    (int64_t)1 << 32, (int64_t)1 << 56, (int64_t)1 << 62, INT64_MAX - 15, INT64_MAX};
#define NV ((int)(sizeof(kVals) / sizeof(kVals[0])))

/* fake, aligned, never dereferenced device addresses: every call below either
 * fails validation or stops at the device check */
#define FA ((const void *)(uintptr_t)0x10000000)
#define FB ((const void *)(uintptr_t)0x20000000)
#define FC ((void *)(uintptr_t)0x30000000)

static void check_plan(int64_t M, int64_t N, int64_t K, int32_t dt, const hkg_gemm_opts *o)
{
    hkg_launch_plan_t pl;
    const int rc = hkg_launch_plan(M, N, K, dt, o, &pl);
    EXPECT(is_status(rc) && rc != HKG_ERR_DEVICE && rc != HKG_ERR_LAUNCH,
           "plan rc %d for %" PRId64 " %" PRId64 " %" PRId64 " dt %d", rc, M, N, K, dt);
    if (rc != HKG_OK || M == 0 || N == 0)
        return;
    EXPECT(pl.launches == 1 || pl.launches == 2, "launches %d", pl.launches);
    int64_t rows = 0;
    for (int i = 0; i < pl.launches && i < 2; ++i) {
        const int64_t t = pl.tile[i];
        EXPECT(t == 128 || t == 192 || t == 256, "tile %d", pl.tile[i]);
        EXPECT(pl.rows[i] > 0 && pl.grid[i] > 0 && pl.grid[i] < ((int64_t)1 << 30), "rows/grid");
        EXPECT(pl.grid[i] == ((pl.rows[i] + t - 1) / t) * ((N + t - 1) / t), "grid %" PRId64,
               pl.grid[i]);
        EXPECT(pl.W[i] >= 1 && pl.C[i] >= 1, "W/C %d %d", pl.W[i], pl.C[i]);
        rows += pl.rows[i];
    }
    EXPECT(rows == M, "rows %" PRId64 " != M %" PRId64, rows, M);
}

int main(void)
{
    hkg_gemm_opts o = {0};
    for (int a = 0; a < NV; ++a)
        for (int b = 0; b < NV; ++b)
            for (int c = 0; c < NV; ++c) {
                const int64_t M = kVals[a], N = kVals[b], K = kVals[c];
                for (int32_t dt = -1; dt <= 3; ++dt)
                    check_plan(M, N, K, dt, NULL);
                /* no launch can succeed here: HKG_OK only for an empty output */
                const int empty = (M == 0 || N == 0);
                int rc = hkg_gemm_bf16(M, N, K, FA, FB, FC, NULL, NULL);
                EXPECT(is_status(rc) && (rc != HKG_OK || empty) && rc != HKG_ERR_LAUNCH,
                       "bf16 rc %d", rc);
                rc = hkg_gemm_fp8(M, N, K, FA, FB, 1.0f, 1.0f, FC, NULL, NULL);
                EXPECT(is_status(rc) && (rc != HKG_OK || empty) && rc != HKG_ERR_LAUNCH,
                       "fp8 rc %d", rc);
                rc = hkg_gemm_mxfp8(M, N, K, FA, FB, FA, FB, FC, NULL, NULL);
                EXPECT(is_status(rc) && (rc != HKG_OK || empty) && rc != HKG_ERR_LAUNCH,
                       "mx rc %d", rc);
                /* pitches: the three values as lda / ldb / ldc of a fixed shape */
                o = (hkg_gemm_opts){0};
                o.lda = M, o.ldb = N, o.ldc = K;
                rc = hkg_gemm_bf16_ex(300, 200, 64, FA, FB, FC, NULL, NULL, &o);
                EXPECT(is_status(rc) && rc != HKG_OK && rc != HKG_ERR_LAUNCH, "pitch rc %d", rc);
                check_plan(300, 200, 64, 0, &o);
                check_plan(257, 257, 4096, 1, &o);
                /* grid sides, orders and panel sizes of the remap entry points */
                int64_t tm = 0, tn = 0;
                rc = hkg_remap_tile(M, N, (int32_t)(K & 0x7fffffff), 4, 0, &tm, &tn);
                EXPECT(is_status(rc), "remap_tile rc %d", rc);
                if (rc == HKG_OK)
                    EXPECT(tm >= 0 && tm < M && tn >= 0 && tn < N, "tile out of grid");
                if (a % 3 == 0 && b % 3 == 0) {   /* the model walks the grid: keep it small */
                    double l2, llc, bw;
                    rc = hkg_remap_model(M < 4096 ? M : 64, N < 4096 ? N : 64, 8, 32, K, 32, &l2,
                                         &llc, &bw);
                    EXPECT(is_status(rc), "remap_model rc %d", rc);
                    if (rc == HKG_OK)
                        EXPECT(l2 >= 0 && l2 <= 1 && llc >= 0 && llc <= 1 && bw >= 0, "model range");
                }
                if ((a + b + c) % 5 == 0) {   /* ranks 48 orders with the model: a subset */
                    int32_t W[48], C[48], count = -1;
                    double bwc[48];
                    rc = hkg_remap_candidates(M, N, K, 0, 48, W, C, bwc, &count);
                    EXPECT(is_status(rc) && (rc != HKG_OK || (count >= 0 && count <= 48)),
                           "candidates rc %d count %d", rc, count);
                }
                const int64_t pb = hkg_mx_packed_scale_bytes(M, K);
                EXPECT(pb >= 0 || is_status((int)pb), "packed bytes %" PRId64, pb);
                rc = hkg_mx_pack_scales(HKG_MX_OPERAND_A, M, K, FA, FC, NULL);
                EXPECT(is_status(rc) && rc != HKG_ERR_LAUNCH, "pack rc %d", rc);
            }
    /* the autotuner's own checks, and the status strings */
    hkg_gemm_opts best;
    float ms;
    for (int a = 0; a < NV; ++a) {
        const int rc = hkg_tune_remap(kVals[a], 256, 256, 0, FA, FB, FC, 10, &best, &ms, NULL,
                                      NULL, NULL, NULL);
        EXPECT(is_status(rc) && rc != HKG_ERR_LAUNCH, "tune rc %d", rc);
    }
    for (int s = -20; s <= 5; ++s)
        EXPECT(hkg_status_string(s) != NULL, "status string");
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ABI EXTREMES OK\n");
    return 0;
}
