// hkg_api.cpp -- the C ABI of libhkg: argument validation, launch plan
// (tile grid, K steps, grid-remap parameters) and kernel launch.
//
// Every check runs before the first HIP call, so a rejected call launches
// nothing and leaves C untouched.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/hkg.h"
#include "api_internal.h"
#include "kernels.h"
#include "remap.h"
#include "remap_model.h"

namespace hkg::api {

thread_local int g_last_hip_error = 0;

void set_last_hip_error(int e) { g_last_hip_error = e; }

// Whether a device is a gfx950, cached per device ordinal (0 = not yet
// asked, 1 = gfx950, -1 = another architecture).  The kernels are built for
// gfx950 only.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_arch[kMaxDevices];

// The device work on `stream` runs on (NULL: the calling thread's current
// device) must be a gfx950.  Called after argument validation, right before
// the first launch of a call; a device query, no launch.
int check_device(void *stream)
{
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                          : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        g_last_hip_error = static_cast<int>(e);
        return HKG_ERR_DEVICE;
    }
    int known = dev < kMaxDevices ? g_device_arch[dev].load(std::memory_order_relaxed) : 0;
    if (known == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            g_last_hip_error = static_cast<int>(e);
            return HKG_ERR_DEVICE;
        }
        known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if (dev < kMaxDevices)
            g_device_arch[dev].store(known, std::memory_order_relaxed);
    }
    return known == 1 ? HKG_OK : HKG_ERR_DEVICE;
}

// Device check, then clear any error an earlier, unrelated HIP call left
// pending, so that the hipGetLastError() read after a launch reports that
// launch only.
int prepare_launch(void *stream)
{
    const int rc = check_device(stream);
    if (rc == HKG_OK)
        (void)hipGetLastError();
    return rc;
}

constexpr int64_t kTile = 256;
constexpr int64_t kKStepBf16 = 64;     // K elements per step (one 128-byte LDS row)
constexpr int64_t kKStepFp8 = 128;
constexpr int64_t kKAlignMx = 32;      // one E8M0 scale per 32 elements along K
constexpr int64_t kMxGroupRows = 128;  // packed scales: 128-row groups ...
constexpr int64_t kMxStepBytes = 512;  // ... of 64 lanes x 8 bytes per K step
static_assert(kTile % kMxGroupRows == 0, "a launch's first row starts a scale group");

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t mx_packed_bytes(int64_t rows, int64_t K)
{
    return ceil_div(rows, kMxGroupRows) * ceil_div(K, kKStepFp8) * kMxStepBytes;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void clamp_remap(int64_t Gm, int64_t Gn, int64_t *W, int64_t *C)
{
    hkg::clamp_order(Gm, Gn, *W, *C);
}

// (W, C) used when the caller does not choose one; row_bytes = K x element
// size.  Both choices give each XCD's 32 concurrent tiles a patch that
// shares 12 operand panels in its L2 (the L2 term of the pages' Eq. 1; the
// cache model of remap_model.h predicts 81 % L2 hits for both):
//  - (8, 32): chunks of 32 consecutive remapped ids per XCD, an 8 x 4 patch;
//    the 256 tiles in flight on the chip form an 8 x 32 strip of the grid
//    (40 panels);
//  - (16, 4): chunks of 4, a 4 x 8 patch per XCD; the 256 tiles in flight
//    form a 16 x 16 block (32 panels).
// The second keeps the chip-wide working set (panels x 256 rows x row_bytes)
// inside the last-level cache when the first's would not fit (the LLC term
// of Eq. 1).  Measured at square sizes: (8, 32) is as good or better while 40
// panels stay below ~185 MiB (bf16 n <= 9216, e4m3 n <= 12288, K = 4096
// shapes), and (16, 4) wins above (bf16 10000, 12288, 14592, 16384: +5.4,
// +1.6, +1.0, +5.1 %).  Ranking every candidate by the model's Eq. 1
// bandwidth agrees at 8192, 12288, 14592 and 16384 bf16 but not at 10000
// bf16, e4m3 12288 or K = 4096 (its LLC term is too coarse there), so the
// measured rule stays the default and the model serves as hkg_remap_model.
constexpr int64_t kLlcPanelBudget = int64_t(185) << 20;
constexpr int64_t kBigRowBytes = kLlcPanelBudget / (40 * kTile);   // 18944 B (bf16 K > 9472)

void default_remap(int64_t Gm, int64_t Gn, int64_t row_bytes, int32_t *W, int32_t *C)
{
    const bool big = row_bytes > kBigRowBytes;
    int64_t w = big ? 16 : 8, c = big ? 4 : 32;
    clamp_remap(Gm, Gn, &w, &c);
    *W = static_cast<int32_t>(w);
    *C = static_cast<int32_t>(c);
}

// Row pitches of a call in elements (hkg_gemm_opts lda / ldb / ldc; 0 means
// dense rows: K, K and N).
struct Layout {
    int64_t lda, ldb, ldc;
};

// The layout the options ask for.  HKG_ERR_OPTS for a pitch below its row's
// extent (or negative), HKG_ERR_ALIGN for an operand pitch whose rows would
// not start 16-byte aligned.
int resolve_layout(const hkg_gemm_opts *opts, int64_t N, int64_t K, int64_t elem, Layout *L)
{
    L->lda = opts && opts->lda ? opts->lda : K;
    L->ldb = opts && opts->ldb ? opts->ldb : K;
    L->ldc = opts && opts->ldc ? opts->ldc : N;
    if (L->lda < K || L->ldb < K || L->ldc < N)
        return HKG_ERR_OPTS;
    if ((L->lda * elem) % 16 || (L->ldb * elem) % 16)
        return HKG_ERR_ALIGN;
    return HKG_OK;
}

// Bytes from the first element of a [rows][cols] matrix with row pitch ld to
// just past its last element (0 when empty).
int64_t extent(int64_t rows, int64_t cols, int64_t ld, int64_t elem)
{
    return rows > 0 && cols > 0 ? ((rows - 1) * ld + cols) * elem : 0;
}

// One 256-row operand panel is addressed through a buffer resource with a
// 32-bit byte range, and tile counts / element offsets / pitches use 32-bit
// ints.
bool sizes_fit(int64_t M, int64_t N, const Layout &L, int64_t elem)
{
    return kTile * L.lda * elem < (int64_t(1) << 31) && kTile * L.ldb * elem < (int64_t(1) << 31) &&
           L.ldc < (int64_t(1) << 31) && M < (int64_t(1) << 31) && N < (int64_t(1) << 31) &&
           ceil_div(M, kTile) * ceil_div(N, kTile) < (int64_t(1) << 30);
}

// Whether byte ranges [p, p + pb) and [q, q + qb) share a byte.
bool overlaps(const void *p, int64_t pb, const void *q, int64_t qb)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return p && q && pb > 0 && qb > 0 && a < b + static_cast<uintptr_t>(qb) &&
           b < a + static_cast<uintptr_t>(pb);
}

int validate_layout(int64_t M, int64_t N, int64_t K, int64_t kalign, int64_t elem,
                    const Layout &L, const void *A, const void *B, const void *C,
                    const float *C_f32)
{
    if (M < 0 || N < 0 || K < 0)
        return HKG_ERR_SHAPE;
    if (K % kalign)
        return HKG_ERR_SHAPE;
    if (M == 0 || N == 0)
        return HKG_OK;
    if (!C || (K > 0 && (!A || !B)))
        return HKG_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (C_f32 && !aligned16(C_f32)))
        return HKG_ERR_ALIGN;
    if (!sizes_fit(M, N, L, elem))
        return HKG_ERR_SIZE;
    // Tiles read operand panels while other tiles write C: an output that
    // shares a byte with an input, or the two outputs with each other, would
    // give a wrong result.  (A and B may alias: both are only read.)  With
    // pitches, each matrix is taken to span its first to its last element.
    const int64_t ab = extent(M, K, L.lda, elem), bb = extent(N, K, L.ldb, elem),
                  cb = extent(M, N, L.ldc, 2), fb = extent(M, N, L.ldc, 4);
    if (overlaps(C, cb, A, ab) || overlaps(C, cb, B, bb) || overlaps(C_f32, fb, A, ab) ||
        overlaps(C_f32, fb, B, bb) || overlaps(C_f32, fb, C, cb))
        return HKG_ERR_OVERLAP;
    return HKG_OK;
}

int validate(int64_t M, int64_t N, int64_t K, int64_t kalign, int64_t elem, const void *A,
             const void *B, const void *C, const float *C_f32)
{
    return validate_layout(M, N, K, kalign, elem, Layout{K, K, N}, A, B, C, C_f32);
}

// Output tile edge of a schedule's kernel.
int64_t tile_edge(hkg::Schedule s)
{
    return s == hkg::kInterleave128 ? 128 : s == hkg::kInterleave192 ? 192 : kTile;
}

// The default schedule: the 4-wave kernel on 256 x 256 tiles, or on 128 x 128
// tiles when the 256 x 256 grid would leave more than half of the 256 CUs
// idle (at most 128 tiles; 128 x 128 tiles give four times as many, two per
// CU).  bf16 and e4m3 also have 192 x 192 tiles, taken
//  - when they fit one round on the 256 CUs (at most 256 tiles) while
//    128 x 128 ones would not (more than 256, so some CU runs two): each CU
//    then runs one 192-tile instead of two 128-tiles or a single 256-tile;
//  - when they fill whole rounds while the 256 x 256 grid ends in a round at
//    least a quarter full (a smaller remainder costs the split launch less).
// Square sizes: 1024^3 .. 2048^3 run 1.9-2.6x faster on 128 x 128 tiles than
// on 256 x 256; 2304^3 .. 3072^3 4-36 % faster on 192 x 192 tiles than on
// either other tile, 6144^3 3-8 % faster than 256 x 256 tiles with the split
// (9216^3, whose 256 x 256 remainder is 16 tiles, 5 % slower).
hkg::Schedule default_schedule(hkg::Dtype dt, int64_t M, int64_t N)
{
    const int64_t g256 = ceil_div(M, kTile) * ceil_div(N, kTile);
    const int64_t g192 = ceil_div(M, 192) * ceil_div(N, 192);
    const int64_t g128 = ceil_div(M, 128) * ceil_div(N, 128);
    if (dt != hkg::kMx) {
        if (g192 <= 256 && g128 > 256)
            return hkg::kInterleave192;
        if (g256 > 256 && g192 % 256 == 0 && g256 % 256 >= 64)
            return hkg::kInterleave192;
    }
    return g256 <= 128 ? hkg::kInterleave128 : hkg::kInterleave;
}

// Rows of a default 256 x 256 launch to keep when the rest goes to a second
// launch on 128 x 128 tiles (0: no split).  A grid of G > 256 tiles with a
// partial last round runs that round on a fraction of the CUs; instead the
// tile rows that fill whole rounds stay on 256 x 256 tiles and the remaining
// rows (fewer than a round's worth) run as 128 x 128 tiles spread over the
// whole chip, if those fit in one pass at two workgroups per CU and the
// idle share of the plain launch, (256 - G % 256) / 256 of a round out of
// G / 256 + 1, is at least a tenth (measured: 4352^3 +23 %, 6144^3 +4-9 %,
// 9216^3 +3 %, 10000^3 +1-2 %; 16448^3, 3 % idle, was 3 % slower split).
// Every kernel sums a block's K steps in the same order, so the output is
// the same bit for bit as with one launch.
int64_t split_rows(int64_t M, int64_t N)
{
    const int64_t Gm = ceil_div(M, kTile), Gn = ceil_div(N, kTile), G = Gm * Gn;
    if (G <= 256 || G % 256 == 0)
        return 0;
    if ((256 - G % 256) * 10 < 256 * (G / 256 + 1))
        return 0;
    const int64_t Gm1 = (G / 256) * 256 / Gn;   // tile rows that fit in the whole rounds
    if (Gm1 < 1 || Gm1 >= Gm)
        return 0;
    const int64_t rest = ceil_div(M - Gm1 * kTile, 128) * ceil_div(N, 128);
    return rest <= 512 ? Gm1 * kTile : 0;
}

// Schedule, tile grid (Gm x Gn tiles of the schedule's edge) and grid order
// of a call; M, N > 0.
int resolve_opts(hkg::Dtype dt, const hkg_gemm_opts *opts, int64_t M, int64_t N, int64_t row_bytes,
                 int64_t *Gm, int64_t *Gn, int32_t *W, int32_t *C, hkg::Schedule *sched)
{
    *sched = default_schedule(dt, M, N);
    if (opts) {
        switch (opts->schedule) {
        case HKG_SCHED_DEFAULT:
            break;
        case HKG_SCHED_PINGPONG:
            *sched = hkg::kPingPong;
            break;
        case HKG_SCHED_LOCKSTEP:
            *sched = hkg::kLockstep;
            break;
        case HKG_SCHED_INTERLEAVE:
            *sched = hkg::kInterleave;
            break;
        case HKG_SCHED_INTERLEAVE_128:
            *sched = hkg::kInterleave128;
            break;
        case HKG_SCHED_INTERLEAVE_192:
            *sched = hkg::kInterleave192;
            break;
        default:
            return HKG_ERR_OPTS;
        }
    }
    const int64_t t = tile_edge(*sched);
    *Gm = ceil_div(M, t);
    *Gn = ceil_div(N, t);
    if (*Gm * *Gn >= (int64_t(1) << 30))
        return HKG_ERR_SIZE;
    default_remap(*Gm, *Gn, row_bytes, W, C);
    if (!opts)
        return HKG_OK;
    switch (opts->remap) {
    case HKG_REMAP_DEFAULT:
        break;
    case HKG_REMAP_ROW_MAJOR:
        *W = 1;
        *C = 1;
        break;
    case HKG_REMAP_XCD:
        if (opts->W < 1 || opts->C < 1)
            return HKG_ERR_OPTS;
        {
            int64_t w = opts->W, c = opts->C;
            clamp_remap(*Gm, *Gn, &w, &c);
            *W = static_cast<int32_t>(w);
            *C = static_cast<int32_t>(c);
        }
        break;
    default:
        return HKG_ERR_OPTS;
    }
    return HKG_OK;
}

bool opts_in_range(const hkg_gemm_opts *opts)
{
    return !opts || (opts->remap >= 0 && opts->remap <= 2 && opts->schedule >= 0 &&
                     opts->schedule <= 5 && opts->lda >= 0 && opts->ldb >= 0 && opts->ldc >= 0);
}

// Only the 4-wave kernel on 256 x 256 and 128 x 128 tiles has the
// block-scaled MFMA path (its packed scales follow 128-row groups).
bool schedule_supported(hkg::Dtype dt, const hkg_gemm_opts *opts)
{
    return dt != hkg::kMx || !opts || opts->schedule == HKG_SCHED_DEFAULT ||
           opts->schedule == HKG_SCHED_INTERLEAVE || opts->schedule == HKG_SCHED_INTERLEAVE_128;
}

// What one call launches: one or two GEMMs over consecutive row ranges of C
// (the second only for the default split of a partial last round).
struct Plan {
    int launches;
    hkg::Schedule sched[2];
    int64_t rows[2], Gm[2], Gn[2];
    int32_t W[2], C[2];
};

// The launches of a call with valid shapes and M, N > 0.
int plan_gemm(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const hkg_gemm_opts *opts, Plan *pl)
{
    if (!schedule_supported(dt, opts))
        return HKG_ERR_OPTS;
    const int64_t row_bytes = K * (dt == hkg::kBf16 ? 2 : 1);
    pl->launches = 1;
    pl->rows[0] = M;
    int rc = resolve_opts(dt, opts, M, N, row_bytes, &pl->Gm[0], &pl->Gn[0], &pl->W[0], &pl->C[0],
                          &pl->sched[0]);
    if (rc != HKG_OK)
        return rc;
    // default schedule and order on a 256 x 256 grid with a partial last
    // round: the whole rounds in launch 0, the remaining rows as launch 1
    const bool defaults = !opts || (opts->schedule == HKG_SCHED_DEFAULT &&
                                    opts->remap == HKG_REMAP_DEFAULT);
    if (defaults && pl->sched[0] == hkg::kInterleave) {
        const int64_t keep = split_rows(M, N);
        if (keep > 0) {
            pl->launches = 2;
            pl->rows[0] = keep;
            pl->Gm[0] = ceil_div(keep, kTile);
            default_remap(pl->Gm[0], pl->Gn[0], row_bytes, &pl->W[0], &pl->C[0]);
            pl->sched[1] = hkg::kInterleave128;
            pl->rows[1] = M - keep;
            pl->Gm[1] = ceil_div(M - keep, 128);
            pl->Gn[1] = ceil_div(N, 128);
            default_remap(pl->Gm[1], pl->Gn[1], row_bytes, &pl->W[1], &pl->C[1]);
        }
    }
    return HKG_OK;
}

int gemm(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const void *A, const void *B, float sa,
         float sb, const void *SA, const void *SB, void *C, float *C_f32, void *stream,
         const hkg_gemm_opts *opts)
{
    const int64_t kstep = dt == hkg::kBf16 ? kKStepBf16 : kKStepFp8;
    const int64_t kalign =
        dt == hkg::kBf16 ? kKAlignBf16 : (dt == hkg::kFp8 ? kKAlignFp8 : kKAlignMx);
    const int64_t elem = dt == hkg::kBf16 ? 2 : 1;
    if (M < 0 || N < 0 || K < 0 || K % kalign)
        return HKG_ERR_SHAPE;
    if (!opts_in_range(opts))
        return HKG_ERR_OPTS;
    Layout L;
    int rc = resolve_layout(opts, N, K, elem, &L);
    if (rc != HKG_OK)
        return rc;
    rc = validate_layout(M, N, K, kalign, elem, L, A, B, C, C_f32);
    if (rc != HKG_OK)
        return rc;
    const int64_t cb = extent(M, N, L.ldc, 2), fb = extent(M, N, L.ldc, 4);
    if (dt == hkg::kMx && M > 0 && N > 0 && K > 0) {
        if (!SA || !SB)
            return HKG_ERR_NULL;
        if (!aligned16(SA) || !aligned16(SB))
            return HKG_ERR_ALIGN;
        // the packed scales are read through 32-bit buffer ranges
        if (mx_packed_bytes(M, K) >= (int64_t(1) << 31) || mx_packed_bytes(N, K) >= (int64_t(1) << 31))
            return HKG_ERR_SIZE;
        const int64_t sab = mx_packed_bytes(M, K), sbb = mx_packed_bytes(N, K);
        if (overlaps(C, cb, SA, sab) || overlaps(C, cb, SB, sbb) || overlaps(C_f32, fb, SA, sab) ||
            overlaps(C_f32, fb, SB, sbb))
            return HKG_ERR_OVERLAP;
    }
    if (M == 0 || N == 0)
        return opts_in_range(opts) && schedule_supported(dt, opts) ? HKG_OK : HKG_ERR_OPTS;
    Plan pl;
    rc = plan_gemm(dt, M, N, K, opts, &pl);
    if (rc != HKG_OK)
        return rc;
    uint64_t *trace = opts ? opts->trace : nullptr;
    if (trace) {
        // 8 words per workgroup of every launch of the call
        int64_t wgs = 0;
        for (int i = 0; i < pl.launches; ++i)
            wgs += pl.Gm[i] * pl.Gn[i];
        const int64_t tb = 64 * wgs, ab = extent(M, K, L.lda, elem), bb = extent(N, K, L.ldb, elem);
        if ((reinterpret_cast<uintptr_t>(trace) & 7u) != 0)
            return HKG_ERR_ALIGN;
        if (overlaps(trace, tb, A, ab) || overlaps(trace, tb, B, bb) || overlaps(trace, tb, C, cb) ||
            overlaps(trace, tb, C_f32, fb))
            return HKG_ERR_OVERLAP;
    }

    rc = prepare_launch(stream);
    if (rc != HKG_OK)
        return rc;

    hkg::GemmParams p;
    p.B = B;
    p.N = static_cast<int>(N);
    p.K = static_cast<int>(K);
    p.lda = static_cast<int>(L.lda);
    p.ldb = static_cast<int>(L.ldb);
    p.ldc = static_cast<int>(L.ldc);
    p.nk = static_cast<int>(ceil_div(K, kstep));
    // The product of the two per-tensor scales, rounded once to fp32.
    p.scale = dt == hkg::kFp8 ? static_cast<float>(static_cast<double>(sa) * sb) : 1.0f;
    p.SB = SB;
    p.sb_bytes = dt == hkg::kMx ? static_cast<int>(mx_packed_bytes(N, K)) : 0;
    int64_t row = 0;
    for (int i = 0; i < pl.launches; ++i) {
        // launch i covers output rows [row, row + rows[i]); row is 0 or a
        // multiple of 256, so the offset pointers keep 16-byte alignment, and
        // A's packed scales start at the group of 128 rows that holds row
        p.A = static_cast<const char *>(A) + row * L.lda * elem;
        if (dt == hkg::kMx) {
            p.SA = static_cast<const char *>(SA) + mx_packed_bytes(row, K);
            p.sa_bytes = static_cast<int>(mx_packed_bytes(pl.rows[i], K));
        } else {
            p.SA = nullptr;
            p.sa_bytes = 0;
        }
        p.C = static_cast<uint16_t *>(C) + row * L.ldc;
        p.C_f32 = C_f32 ? C_f32 + row * L.ldc : nullptr;
        p.M = static_cast<int>(pl.rows[i]);
        p.Gm = static_cast<int>(pl.Gm[i]);
        p.Gn = static_cast<int>(pl.Gn[i]);
        p.W = pl.W[i];
        p.Cc = pl.C[i];
        p.trace = trace;
        const hipError_t e = hkg::launch_gemm(dt, pl.sched[i], p, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) {
            g_last_hip_error = static_cast<int>(e);
            return HKG_ERR_LAUNCH;
        }
        row += pl.rows[i];
        if (trace)
            trace += 8 * pl.Gm[i] * pl.Gn[i];
    }
    return HKG_OK;
}

}  // namespace hkg::api

using namespace hkg::api;

extern "C" {

int hkg_gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
                  float *C_f32, void *stream)
{
    return gemm(hkg::kBf16, M, N, K, A, B, 1.0f, 1.0f, nullptr, nullptr, C, C_f32, stream,
                nullptr);
}

int hkg_gemm_fp8(int64_t M, int64_t N, int64_t K, const void *A, const void *B, float scale_a,
                 float scale_b, void *C, float *C_f32, void *stream)
{
    return gemm(hkg::kFp8, M, N, K, A, B, scale_a, scale_b, nullptr, nullptr, C, C_f32, stream,
                nullptr);
}

int hkg_gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
                     float *C_f32, void *stream, const hkg_gemm_opts *opts)
{
    return gemm(hkg::kBf16, M, N, K, A, B, 1.0f, 1.0f, nullptr, nullptr, C, C_f32, stream, opts);
}

int hkg_gemm_fp8_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                    float scale_a, float scale_b, void *C, float *C_f32, void *stream,
                    const hkg_gemm_opts *opts)
{
    return gemm(hkg::kFp8, M, N, K, A, B, scale_a, scale_b, nullptr, nullptr, C, C_f32, stream,
                opts);
}

int hkg_gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                   const void *SA_packed, const void *SB_packed, void *C, float *C_f32,
                   void *stream)
{
    return gemm(hkg::kMx, M, N, K, A, B, 1.0f, 1.0f, SA_packed, SB_packed, C, C_f32, stream,
                nullptr);
}

int hkg_gemm_mxfp8_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                      const void *SA_packed, const void *SB_packed, void *C, float *C_f32,
                      void *stream, const hkg_gemm_opts *opts)
{
    return gemm(hkg::kMx, M, N, K, A, B, 1.0f, 1.0f, SA_packed, SB_packed, C, C_f32, stream,
                opts);
}

int64_t hkg_mx_packed_scale_bytes(int64_t rows, int64_t K)
{
    if (rows < 0 || K < 0 || K % kKAlignMx)
        return HKG_ERR_SHAPE;
    return mx_packed_bytes(rows, K);
}

int hkg_mx_pack_scales(int32_t operand, int64_t rows, int64_t K, const void *scales,
                       void *packed, void *stream)
{
    if (operand != HKG_MX_OPERAND_A && operand != HKG_MX_OPERAND_B)
        return HKG_ERR_OPTS;
    if (rows < 0 || K < 0 || K % kKAlignMx)
        return HKG_ERR_SHAPE;
    if (rows == 0 || K == 0)
        return HKG_OK;
    if (!scales || !packed)
        return HKG_ERR_NULL;
    if (!aligned16(packed))
        return HKG_ERR_ALIGN;
    // the same K bound as the GEMM (one 256-row e4m3 panel below 2 GiB)
    if (rows >= (int64_t(1) << 31) || kTile * K >= (int64_t(1) << 31) ||
        mx_packed_bytes(rows, K) >= (int64_t(1) << 31))
        return HKG_ERR_SIZE;
    if (overlaps(packed, mx_packed_bytes(rows, K), scales, rows * (K / kKAlignMx)))
        return HKG_ERR_OVERLAP;
    const int rc = prepare_launch(stream);
    if (rc != HKG_OK)
        return rc;
    hipError_t e = hkg::launch_mx_pack(
        operand, static_cast<int>(rows), static_cast<int>(K / kKAlignMx),
        static_cast<int>(ceil_div(K, kKStepFp8)), static_cast<int>(ceil_div(rows, kMxGroupRows)),
        static_cast<const uint8_t *>(scales), static_cast<uint8_t *>(packed),
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return HKG_ERR_LAUNCH;
    }
    return HKG_OK;
}

int hkg_default_remap(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t *W, int32_t *C)
{
    if (!W || !C)
        return HKG_ERR_NULL;
    hkg_launch_plan_t pl;
    const int rc = hkg_launch_plan(M, N, K, dtype, nullptr, &pl);
    if (rc != HKG_OK)
        return rc;
    if (pl.launches == 0)
        return HKG_ERR_SHAPE;
    *W = pl.W[0];
    *C = pl.C[0];
    return HKG_OK;
}

int hkg_launch_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, const hkg_gemm_opts *opts,
                    hkg_launch_plan_t *plan)
{
    if (!plan)
        return HKG_ERR_NULL;
    if (dtype < 0 || dtype > 2)
        return HKG_ERR_SHAPE;
    const hkg::Dtype dt = dtype == 0 ? hkg::kBf16 : (dtype == 1 ? hkg::kFp8 : hkg::kMx);
    const int64_t kalign = dtype == 0 ? kKAlignBf16 : (dtype == 1 ? kKAlignFp8 : kKAlignMx);
    const int64_t elem = dtype == 0 ? 2 : 1;
    if (M < 0 || N < 0 || K < 0 || K % kalign)
        return HKG_ERR_SHAPE;
    *plan = hkg_launch_plan_t{};
    if (!opts_in_range(opts))
        return HKG_ERR_OPTS;
    Layout L;
    const int lrc = resolve_layout(opts, N, K, elem, &L);
    if (lrc != HKG_OK)
        return lrc;
    if (M == 0 || N == 0)   // as the entry points: no launch, only the options checked
        return schedule_supported(dt, opts) ? HKG_OK : HKG_ERR_OPTS;
    if (!sizes_fit(M, N, L, elem))
        return HKG_ERR_SIZE;
    Plan pl;
    const int rc = plan_gemm(dt, M, N, K, opts, &pl);
    if (rc != HKG_OK)
        return rc;
    plan->launches = pl.launches;
    for (int i = 0; i < pl.launches; ++i) {
        static const int32_t kSched[] = {HKG_SCHED_PINGPONG, HKG_SCHED_LOCKSTEP, HKG_SCHED_INTERLEAVE,
                                         HKG_SCHED_INTERLEAVE_128, HKG_SCHED_INTERLEAVE_192};
        plan->schedule[i] = kSched[pl.sched[i]];
        plan->tile[i] = static_cast<int32_t>(tile_edge(pl.sched[i]));
        plan->rows[i] = pl.rows[i];
        plan->grid[i] = pl.Gm[i] * pl.Gn[i];
        plan->W[i] = pl.W[i];
        plan->C[i] = pl.C[i];
    }
    return HKG_OK;
}

int hkg_remap_model(int64_t Gm, int64_t Gn, int32_t W, int32_t C, int64_t panel_bytes,
                    int32_t per_xcd, double *l2_hit, double *llc_hit, double *eq1_bw_tbs)
{
    if (!l2_hit || !llc_hit || !eq1_bw_tbs)
        return HKG_ERR_NULL;
    if (Gm < 1 || Gn < 1 || W < 1 || C < 1 || Gm * Gn >= (int64_t(1) << 30) || panel_bytes < 0 ||
        per_xcd < 1 || per_xcd > 1024)
        return HKG_ERR_SHAPE;
    int64_t w = W, c = C;
    clamp_remap(Gm, Gn, &w, &c);
    const hkg::RemapModel m =
        hkg::model_remap(static_cast<int>(Gm), static_cast<int>(Gn), static_cast<int>(w),
                         static_cast<int>(c), panel_bytes, per_xcd);
    *l2_hit = m.l2_hit;
    *llc_hit = m.llc_hit;
    *eq1_bw_tbs = m.bw_tbs;
    return HKG_OK;
}

int hkg_remap_tile(int64_t Gm, int64_t Gn, int32_t W, int32_t C, int64_t b, int64_t *tile_m,
                   int64_t *tile_n)
{
    if (!tile_m || !tile_n)
        return HKG_ERR_NULL;
    if (Gm < 1 || Gn < 1 || W < 1 || C < 1 || Gm * Gn >= (int64_t(1) << 30) || b < 0 ||
        b >= Gm * Gn)
        return HKG_ERR_SHAPE;
    int64_t w = W, c = C;
    clamp_remap(Gm, Gn, &w, &c);
    int tm = 0, tn = 0;
    hkg::remap_tile(static_cast<int>(b), static_cast<int>(Gm), static_cast<int>(Gn),
                    static_cast<int>(w), static_cast<int>(c), tm, tn);
    *tile_m = tm;
    *tile_n = tn;
    return HKG_OK;
}

int hkg_remap_tiles_device(int64_t Gm, int64_t Gn, int32_t W, int32_t C, int32_t *out,
                           void *stream)
{
    if (!out)
        return HKG_ERR_NULL;
    if (Gm < 1 || Gn < 1 || W < 1 || C < 1 || Gm * Gn >= (int64_t(1) << 30))
        return HKG_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0)
        return HKG_ERR_ALIGN;
    int64_t w = W, c = C;
    clamp_remap(Gm, Gn, &w, &c);
    const int rc = prepare_launch(stream);
    if (rc != HKG_OK)
        return rc;
    hipError_t e = hkg::launch_remap_tiles(static_cast<int>(Gm), static_cast<int>(Gn),
                                           static_cast<int>(w), static_cast<int>(c), out,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return HKG_ERR_LAUNCH;
    }
    return HKG_OK;
}

int hkg_probe_xcd(int64_t workgroups, int32_t full_lds, int32_t spin_cycles, int32_t *out,
                  void *stream)
{
    if (!out)
        return HKG_ERR_NULL;
    if (workgroups < 1 || workgroups > (int64_t(1) << 24) || spin_cycles < 0 ||
        spin_cycles > (1 << 24) || (full_lds != 0 && full_lds != 1))
        return HKG_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0)
        return HKG_ERR_ALIGN;
    const int rc = prepare_launch(stream);
    if (rc != HKG_OK)
        return rc;
    hipError_t e = hkg::launch_xcd_probe(static_cast<int>(workgroups), full_lds != 0, spin_cycles,
                                         out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return HKG_ERR_LAUNCH;
    }
    return HKG_OK;
}

const char *hkg_status_string(int status)
{
    switch (status) {
    case HKG_OK: return "ok";
    case HKG_ERR_NULL: return "a required pointer is NULL";
    case HKG_ERR_SHAPE:
        return "unsupported shape (negative, or K not a multiple of 8 bf16 / 16 e4m3 / 32 MXFP8)";
    case HKG_ERR_ALIGN: return "pointer not 16-byte aligned";
    case HKG_ERR_SIZE: return "operand panel exceeds the 32-bit buffer range";
    case HKG_ERR_OPTS: return "invalid hkg_gemm_opts";
    case HKG_ERR_DEVICE: return "the stream's device is not a gfx950, or could not be queried";
    case HKG_ERR_LAUNCH: return "kernel launch failed";
    case HKG_ERR_OVERLAP: return "an output overlaps an input or the other output";
    default: return "unknown status";
    }
}

int hkg_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
