// launch.cpp -- what a GEMM call runs: the default schedule and tile, the
// default grid order, the split of a partial last round into two launches,
// and the kernel launches of a call whose arguments the entry points have
// checked (hkg_api.cpp).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hkg.h"
#include "api_internal.h"
#include "kernels.h"
#include "remap.h"

namespace hkg::api {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t mx_packed_bytes(int64_t rows, int64_t K)
{
    return ceil_div(rows, kMxGroupRows) * ceil_div(K, kKStepFp8) * kMxStepBytes;
}

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

// Only the 4-wave kernel on 256 x 256 and 128 x 128 tiles has the
// block-scaled MFMA path (its packed scales follow 128-row groups).
bool schedule_supported(hkg::Dtype dt, const hkg_gemm_opts *opts)
{
    return dt != hkg::kMx || !opts || opts->schedule == HKG_SCHED_DEFAULT ||
           opts->schedule == HKG_SCHED_INTERLEAVE || opts->schedule == HKG_SCHED_INTERLEAVE_128;
}

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

// The kernel launches of plan `pl` for a call whose arguments are checked and
// whose device is ready (prepare_launch).
int run_plan(hkg::Dtype dt, int64_t N, int64_t K, const Layout &L, const Plan &pl, const void *A,
             const void *B, float sa, float sb, const void *SA, const void *SB, void *C,
             float *C_f32, uint64_t *trace, void *stream)
{
    hkg::GemmParams p;
    p.B = B;
    p.N = static_cast<int>(N);
    p.K = static_cast<int>(K);
    p.lda = static_cast<int>(L.lda);
    p.ldb = static_cast<int>(L.ldb);
    p.ldc = static_cast<int>(L.ldc);
    p.nk = static_cast<int>(ceil_div(K, dt == hkg::kBf16 ? kKStepBf16 : kKStepFp8));
    // The product of the two per-tensor scales, rounded once to fp32.
    p.scale = dt == hkg::kFp8 ? static_cast<float>(static_cast<double>(sa) * sb) : 1.0f;
    p.SB = SB;
    p.sb_bytes = dt == hkg::kMx ? static_cast<int>(mx_packed_bytes(N, K)) : 0;
    int64_t row = 0;
    for (int i = 0; i < pl.launches; ++i) {
        // launch i covers output rows [row, row + rows[i]); row is 0 or a
        // multiple of 256, so the offset pointers keep 16-byte alignment, and
        // A's packed scales start at the group of 128 rows that holds row
        p.A = static_cast<const char *>(A) + row * L.lda * (dt == hkg::kBf16 ? 2 : 1);
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
            set_last_hip_error(static_cast<int>(e));
            return HKG_ERR_LAUNCH;
        }
        row += pl.rows[i];
        if (trace)
            trace += 8 * pl.Gm[i] * pl.Gn[i];
    }
    return HKG_OK;
}

}  // namespace hkg::api
