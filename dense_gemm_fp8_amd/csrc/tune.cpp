// tune.cpp -- grid-order candidates and the autotuner of the C ABI
// (hkg_remap_candidates, hkg_tune_remap).  The HipKittens L2 note tunes the
// window height W and chunk C of the grid remap per shape (section 5 Table 4)
// against the bandwidth of its single equation (section 4); here the cache
// model of remap_model.h ranks the orders and timed launches decide.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/hkg.h"
#include "api_internal.h"
#include "kernels.h"
#include "remap_model.h"

using namespace hkg::api;

namespace {

struct Candidate {
    int32_t W, C;
    double bw;   // the cache model's Eq. 1 bandwidth, TB/s
};
constexpr int kMaxCandidates = 48;
constexpr int kTunedOrders = 6;         // one model-ranked order per window height
constexpr double kTuneSettleMs = 100.0;
constexpr int kTuneMaxLaunches = 1000;

// Every order (W, C) of the default schedule's grid for the shape (M, N > 0),
// clamped and deduplicated, best first by the model's Eq. 1 bandwidth.
int rank_candidates(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, Candidate *out)
{
    static const int kW[] = {1, 2, 4, 8, 16, 32};
    static const int kC[] = {1, 2, 4, 8, 16, 32, 64, 128};
    const hkg::Schedule s = default_schedule(dt, M, N);
    const int64_t t = tile_edge(s);
    const int64_t Gm = ceil_div(M, t), Gn = ceil_div(N, t);
    const int64_t panel = t * K * (dt == hkg::kBf16 ? 2 : 1);
    const int per_xcd = t == 128 ? 64 : 32;   // 32 CUs x workgroups per CU
    int n = 0;
    for (int w : kW) {
        for (int c : kC) {
            int64_t ww = w, cc = c;
            clamp_remap(Gm, Gn, &ww, &cc);
            bool seen = false;
            for (int i = 0; i < n; ++i)
                seen = seen || (out[i].W == ww && out[i].C == cc);
            if (seen)
                continue;
            const hkg::RemapModel m =
                hkg::model_remap(static_cast<int>(Gm), static_cast<int>(Gn), static_cast<int>(ww),
                                 static_cast<int>(cc), panel, per_xcd);
            out[n++] = Candidate{static_cast<int32_t>(ww), static_cast<int32_t>(cc), m.bw_tbs};
        }
    }
    std::stable_sort(out, out + n,
                     [](const Candidate &a, const Candidate &b) { return a.bw > b.bw; });
    return n;
}

// Mean time per launch of `n` launches of one configuration (after one
// untimed launch), measured with the two events on `stream`.
int time_launches(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                  void *C, void *stream, const hkg_gemm_opts *opts, int n, hipEvent_t e0,
                  hipEvent_t e1, float *ms)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = gemm(dt, M, N, K, A, B, 1.0f, 1.0f, nullptr, nullptr, C, nullptr, stream, opts);
    if (rc != HKG_OK)
        return rc;
    hipError_t e = hipEventRecord(e0, st);
    for (int i = 0; i < n && e == hipSuccess && rc == HKG_OK; ++i)
        rc = gemm(dt, M, N, K, A, B, 1.0f, 1.0f, nullptr, nullptr, C, nullptr, stream, opts);
    if (rc != HKG_OK)
        return rc;
    if (e == hipSuccess)
        e = hipEventRecord(e1, st);
    if (e == hipSuccess)
        e = hipEventSynchronize(e1);
    float t = 0.0f;
    if (e == hipSuccess)
        e = hipEventElapsedTime(&t, e0, e1);
    if (e != hipSuccess) {
        set_last_hip_error(static_cast<int>(e));
        return HKG_ERR_LAUNCH;
    }
    *ms = t / static_cast<float>(n);
    return HKG_OK;
}

// The tuner proper, once the arguments are checked (M, N > 0).
int tune(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
         int launches, hkg_gemm_opts *best, float *best_ms, hkg_gemm_opts *tried,
         float *tried_ms, int32_t *n_tried, void *stream, hipEvent_t e0, hipEvent_t e1)
{
    Candidate ranked[kMaxCandidates];
    const int nr = rank_candidates(dt, M, N, K, ranked);
    // slot 0: the default launch (opts NULL); then, for each window height W
    // in the list, its best-ranked order (the model ties many orders that
    // differ only in C, so the top of the list alone would time near-copies);
    // and row-major order if none of those is it
    static_assert(kTunedOrders + 2 <= HKG_TUNE_MAX_CANDIDATES, "report arrays");
    hkg_gemm_opts cand[kTunedOrders + 2];
    int nc = 1;
    bool row_major = false;
    for (int i = 0; i < nr && nc < kTunedOrders + 1; ++i) {
        bool have_w = false;
        for (int j = 1; j < nc; ++j)
            have_w = have_w || cand[j].W == ranked[i].W;
        if (have_w)
            continue;
        cand[nc++] = hkg_gemm_opts{HKG_REMAP_XCD, ranked[i].W, ranked[i].C, HKG_SCHED_DEFAULT,
                                   nullptr};
        row_major = row_major || (ranked[i].W == 1 && ranked[i].C == 1);
    }
    if (!row_major)
        cand[nc++] = hkg_gemm_opts{HKG_REMAP_ROW_MAJOR, 1, 1, HKG_SCHED_DEFAULT, nullptr};

    // settle the clock with default launches
    float one = 0.0f;
    int rc = time_launches(dt, M, N, K, A, B, C, stream, nullptr, 1, e0, e1, &one);
    if (rc != HKG_OK)
        return rc;
    const int settle = static_cast<int>(
        std::min<double>(kTuneMaxLaunches, std::max(1.0, kTuneSettleMs / std::max(one, 1e-3f))));
    rc = time_launches(dt, M, N, K, A, B, C, stream, nullptr, settle, e0, e1, &one);
    if (rc != HKG_OK)
        return rc;

    double total[kTunedOrders + 2] = {};
    for (int pass = 0; pass < 2; ++pass) {
        for (int j = 0; j < nc; ++j) {
            const int i = pass == 0 ? j : nc - 1 - j;
            float ms = 0.0f;
            rc = time_launches(dt, M, N, K, A, B, C, stream, i == 0 ? nullptr : &cand[i], launches,
                               e0, e1, &ms);
            if (rc != HKG_OK)
                return rc;
            total[i] += ms;
        }
    }
    hkg_launch_plan_t pl;
    rc = hkg_launch_plan(M, N, K, dt == hkg::kBf16 ? 0 : 1, nullptr, &pl);
    if (rc != HKG_OK)
        return rc;
    cand[0] = hkg_gemm_opts{HKG_REMAP_DEFAULT, pl.W[0], pl.C[0], HKG_SCHED_DEFAULT, nullptr};
    int w = 0;
    for (int i = 1; i < nc; ++i)
        if (total[i] < total[w])
            w = i;
    *best = cand[w];
    if (best_ms)
        *best_ms = static_cast<float>(total[w] / 2.0);
    if (tried) {
        for (int i = 0; i < nc; ++i) {
            tried[i] = cand[i];
            tried_ms[i] = static_cast<float>(total[i] / 2.0);
        }
        *n_tried = nc;
    }
    return HKG_OK;
}

}  // namespace

extern "C" {

int hkg_remap_candidates(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t max,
                         int32_t *W, int32_t *C, double *eq1_bw_tbs, int32_t *count)
{
    if (!count || (max > 0 && (!W || !C || !eq1_bw_tbs)))
        return HKG_ERR_NULL;
    hkg_launch_plan_t plan;
    const int rc = hkg_launch_plan(M, N, K, dtype, nullptr, &plan);   // shape and size checks
    if (rc != HKG_OK)
        return rc;
    *count = 0;
    if (M == 0 || N == 0)
        return HKG_OK;
    const hkg::Dtype dt = dtype == 0 ? hkg::kBf16 : (dtype == 1 ? hkg::kFp8 : hkg::kMx);
    Candidate ranked[kMaxCandidates];
    const int n = rank_candidates(dt, M, N, K, ranked);
    for (int i = 0; i < n && i < max; ++i) {
        W[i] = ranked[i].W;
        C[i] = ranked[i].C;
        eq1_bw_tbs[i] = ranked[i].bw;
    }
    *count = n;
    return HKG_OK;
}

int hkg_tune_remap(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B,
                   void *C, int32_t launches, hkg_gemm_opts *best, float *best_ms,
                   hkg_gemm_opts *tried, float *tried_ms, int32_t *n_tried, void *stream)
{
    if (!best)
        return HKG_ERR_NULL;
    const int given = (tried != nullptr) + (tried_ms != nullptr) + (n_tried != nullptr);
    if (given != 0 && given != 3)
        return HKG_ERR_NULL;
    if (dtype != 0 && dtype != 1)
        return HKG_ERR_SHAPE;
    const hkg::Dtype dt = dtype == 0 ? hkg::kBf16 : hkg::kFp8;
    int rc = validate(M, N, K, dtype == 0 ? kKAlignBf16 : kKAlignFp8, dtype == 0 ? 2 : 1, A, B, C,
                      nullptr);
    if (rc != HKG_OK)
        return rc;
    if (launches < 1 || launches > kTuneMaxLaunches)
        return HKG_ERR_OPTS;
    if (M == 0 || N == 0) {
        int32_t w = 1, c = 1;
        *best = hkg_gemm_opts{HKG_REMAP_DEFAULT, w, c, HKG_SCHED_DEFAULT, nullptr};
        if (best_ms)
            *best_ms = 0.0f;
        if (n_tried)
            *n_tried = 0;
        return HKG_OK;
    }
    rc = prepare_launch(stream);
    if (rc != HKG_OK)
        return rc;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess)
        e = hipEventCreate(&e1);
    if (e != hipSuccess) {
        set_last_hip_error(static_cast<int>(e));
        if (e0)
            (void)hipEventDestroy(e0);
        return HKG_ERR_LAUNCH;
    }
    hkg_gemm_opts out;
    rc = tune(dt, M, N, K, A, B, C, launches, &out, best_ms, tried, tried_ms, n_tried, stream, e0,
              e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (rc == HKG_OK)
        *best = out;
    return rc;
}

}  // extern "C"
