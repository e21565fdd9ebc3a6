/*
 * oracle.c -- the CPU oracle for the tiled dense GEMM C = A * B^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg may load this library; the GPU library never does,
 * and the two share no source.
 *
 * What it computes (HipKittens L2 note, section 3 "Target operation" table:
 * BF16 GEMM and FP8 GEMM, FP32 accumulate; B is used transposed, as the
 * mma_ABt calls in the section 7/9 listing descriptions show):
 *
 *     ref[m][n] = sum_{k=0}^{K-1} a[m][k] * b[n][k]            (k ascending)
 *
 * with A stored [M][K] and B stored [N][K], both row-major (K contiguous).
 * Every input element is decoded exactly into a double and the sum is carried
 * in double (fp64).  For fp8 the sum is multiplied by (double)scale_a *
 * (double)scale_b afterwards.
 *
 *   bf16 products have 8-bit significands, so each product is exact in fp64;
 *   e4m3 products are multiples of 2^-18 below 2^18, so fp8 sums over up to
 *   2^13 terms are exact in fp64.
 *
 * Decoding follows the published formats, written out here:
 *   bf16: the 16 bits are the upper half of an IEEE binary32 value.
 *   OCP e4m3 (FN): S.EEEE.MMM, bias 7, no infinities; E == 0 is subnormal
 *   (M/8 * 2^-6), otherwise (1 + M/8) * 2^(E-7); S.1111.111 is NaN; max 448.
 *
 * MXFP8 (the fp8 input type that the HipKittens L2 note's section 3 table
 * names; the format itself is the OCP Microscaling (MX) Formats
 * specification v1.0): e4m3 elements, and one E8M0 scale per 32 consecutive
 * elements along K of each row.  An E8M0 byte E is the value 2^(E-127), and
 * E == 0xFF is NaN.  Element k of row r stands for
 *     e4m3(a[r][k]) * 2^(SA[r][k/32] - 127),
 * so the reference is the same k-ascending fp64 sum of those products, with
 * SA stored [M][K/32] and SB [N][K/32] row-major.  Each product is an
 * exact fp64 value (8-bit significand, exponent within +-300).
 *
 * Rounding to bf16 is one round-to-nearest-even step from the fp64 value
 * (not via binary32).
 *
 * Output coordinates may be given as explicit (m, n) pairs so that full-size
 * problems can be checked on a sample.  Work is split over POSIX threads;
 * each output is still one plain k-ascending loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3_value(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* One round-to-nearest-even step from double to bfloat16 bits. */
uint16_t oracle_bf16_round(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int E;
    frexp(a, &E);               /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;              /* a in [2^e, 2^(e+1)) */
    if (e < -126)
        e = -126;               /* subnormal range: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, e - 7);    /* 7 stored fraction bits */
    double r = nearbyint(a / quantum) * quantum;   /* default mode: ties to even */
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;
    float f = (float)r;         /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void oracle_bf16_round_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(x[i]);
}

/* OCP MX E8M0 scale: 2^(E - 127); 0xFF is NaN. */
double oracle_e8m0_value(uint8_t e)
{
    if (e == 0xFF)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ---------------------------------------------------------------- GEMM ---- */

enum { ORACLE_BF16 = 0, ORACLE_E4M3 = 1, ORACLE_MXFP8 = 2 };

typedef struct {
    int kind;
    int64_t M, N, K;
    const void *A, *B;
    const uint8_t *SA, *SB;     /* MXFP8 block scales [rows][K/32], else NULL */
    double scale;               /* multiplies the sum (1 for bf16) */
    const int64_t *pm, *pn;     /* pairs, or NULL for the full M x N grid */
    int64_t count;              /* number of outputs */
    double *out;
    int64_t begin, end;
} job_t;

static double dot_row_row(const job_t *j, int64_t m, int64_t n)
{
    double s = 0.0;
    if (j->kind == ORACLE_BF16) {
        const uint16_t *a = (const uint16_t *)j->A + m * j->K;
        const uint16_t *b = (const uint16_t *)j->B + n * j->K;
        for (int64_t k = 0; k < j->K; ++k)
            s += oracle_bf16_value(a[k]) * oracle_bf16_value(b[k]);
    } else if (j->kind == ORACLE_E4M3) {
        const uint8_t *a = (const uint8_t *)j->A + m * j->K;
        const uint8_t *b = (const uint8_t *)j->B + n * j->K;
        for (int64_t k = 0; k < j->K; ++k)
            s += oracle_e4m3_value(a[k]) * oracle_e4m3_value(b[k]);
    } else {
        const int64_t nb = j->K / 32;
        const uint8_t *a = (const uint8_t *)j->A + m * j->K;
        const uint8_t *b = (const uint8_t *)j->B + n * j->K;
        const uint8_t *sa = j->SA + m * nb;
        const uint8_t *sb = j->SB + n * nb;
        for (int64_t k = 0; k < j->K; ++k)
            s += (oracle_e4m3_value(a[k]) * oracle_e8m0_value(sa[k / 32])) *
                 (oracle_e4m3_value(b[k]) * oracle_e8m0_value(sb[k / 32]));
    }
    return s * j->scale;
}

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t i = j->begin; i < j->end; ++i) {
        int64_t m, n;
        if (j->pm) {
            m = j->pm[i];
            n = j->pn[i];
        } else {
            m = i / j->N;
            n = i % j->N;
        }
        j->out[i] = dot_row_row(j, m, n);
    }
    return NULL;
}

static int run(int kind, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
               const uint8_t *SA, const uint8_t *SB, double scale, const int64_t *pm,
               const int64_t *pn, int64_t count, double *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0 || !out)
        return -1;
    if (kind == ORACLE_MXFP8 && (K % 32 != 0 || (M > 0 && N > 0 && K > 0 && (!SA || !SB))))
        return -1;
    if (count == 0)
        return 0;
    if ((M > 0 && N > 0 && K > 0) && (!A || !B))
        return -1;
    if (pm) {
        for (int64_t i = 0; i < count; ++i)
            if (pm[i] < 0 || pm[i] >= M || pn[i] < 0 || pn[i] >= N)
                return -2;
    }
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > count)
        nthreads = (int)count;
    job_t jobs[256];
    pthread_t tids[256];
    int64_t per = (count + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        job_t *j = &jobs[t];
        j->kind = kind; j->M = M; j->N = N; j->K = K; j->A = A; j->B = B;
        j->SA = SA; j->SB = SB;
        j->scale = scale; j->pm = pm; j->pn = pn; j->count = count; j->out = out;
        j->begin = t * per;
        j->end = (t + 1) * per < count ? (t + 1) * per : count;
    }
    int joined[256] = {0};
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].begin >= jobs[t].end)
            continue;
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) == 0)
            joined[t] = 1;
        else
            worker(&jobs[t]);   /* could not start a thread: do the share here */
    }
    worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (joined[t])
            pthread_join(tids[t], NULL);
    return 0;
}

/* Full grid: out is M*N doubles, row-major. */
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                     double *out, int nthreads)
{
    return run(ORACLE_BF16, M, N, K, A, B, NULL, NULL, 1.0, NULL, NULL, M * N, out, nthreads);
}

int oracle_gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t *A, const uint8_t *B,
                    float scale_a, float scale_b, double *out, int nthreads)
{
    return run(ORACLE_E4M3, M, N, K, A, B, NULL, NULL, (double)scale_a * (double)scale_b, NULL,
               NULL, M * N, out, nthreads);
}

/* Sampled outputs: out[i] = ref[pm[i]][pn[i]]. */
int oracle_gemm_bf16_pairs(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                           const uint16_t *B, const int64_t *pm, const int64_t *pn,
                           int64_t count, double *out, int nthreads)
{
    if (count > 0 && (!pm || !pn))
        return -1;
    return run(ORACLE_BF16, M, N, K, A, B, NULL, NULL, 1.0, pm, pn, count, out, nthreads);
}

int oracle_gemm_fp8_pairs(int64_t M, int64_t N, int64_t K, const uint8_t *A, const uint8_t *B,
                          float scale_a, float scale_b, const int64_t *pm, const int64_t *pn,
                          int64_t count, double *out, int nthreads)
{
    if (count > 0 && (!pm || !pn))
        return -1;
    return run(ORACLE_E4M3, M, N, K, A, B, NULL, NULL, (double)scale_a * (double)scale_b, pm, pn,
               count, out, nthreads);
}

/* MXFP8: A, B e4m3 codes [rows][K]; SA [M][K/32], SB [N][K/32] E8M0 bytes;
 * K must be a multiple of 32. */
int oracle_gemm_mxfp8(int64_t M, int64_t N, int64_t K, const uint8_t *A, const uint8_t *B,
                      const uint8_t *SA, const uint8_t *SB, double *out, int nthreads)
{
    return run(ORACLE_MXFP8, M, N, K, A, B, SA, SB, 1.0, NULL, NULL, M * N, out, nthreads);
}

int oracle_gemm_mxfp8_pairs(int64_t M, int64_t N, int64_t K, const uint8_t *A,
                            const uint8_t *B, const uint8_t *SA, const uint8_t *SB,
                            const int64_t *pm, const int64_t *pn, int64_t count, double *out,
                            int nthreads)
{
    if (count > 0 && (!pm || !pn))
        return -1;
    return run(ORACLE_MXFP8, M, N, K, A, B, SA, SB, 1.0, pm, pn, count, out, nthreads);
}
