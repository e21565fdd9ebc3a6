// api_internal.h -- host logic of the C ABI shared between its source files
// (hkg_api.cpp: argument checks and the entry points; launch.cpp: schedule,
// tile, grid order and the kernel launches; tune.cpp: the grid-order
// autotuner).  Not part of the installed interface.
#pragma once

#include <stdint.h>

#include "../../include/hkg.h"
#include "kernels.h"

namespace hkg::api {

constexpr int64_t kKAlignBf16 = 8;     // K granule: operand rows stay 16-byte aligned
constexpr int64_t kKAlignFp8 = 16;
constexpr int64_t kTile = 256;
constexpr int64_t kKStepBf16 = 64;     // K elements per step (one 128-byte LDS row)
constexpr int64_t kKStepFp8 = 128;
constexpr int64_t kKAlignMx = 32;      // one E8M0 scale per 32 elements along K
constexpr int64_t kMxGroupRows = 128;  // packed scales: 128-row groups ...
constexpr int64_t kMxStepBytes = 512;  // ... of 64 lanes x 8 bytes per K step
static_assert(kTile % kMxGroupRows == 0, "a launch's first row starts a scale group");

// Row pitches of a call in elements (hkg_gemm_opts lda / ldb / ldc; 0 means
// dense rows: K, K and N).
struct Layout {
    int64_t lda, ldb, ldc;
};

// What one call launches: one or two GEMMs over consecutive row ranges of C
// (the second only for the default split of a partial last round).
struct Plan {
    int launches;
    hkg::Schedule sched[2];
    int64_t rows[2], Gm[2], Gn[2];
    int32_t W[2], C[2];
};

int64_t ceil_div(int64_t a, int64_t b);
// bytes of one MXFP8 operand's packed scales (rows and K already bounded)
int64_t mx_packed_bytes(int64_t rows, int64_t K);
// record a HIP error for hkg_last_hip_error()
void set_last_hip_error(int e);
// argument checks of the GEMM entry points (no HIP call)
int validate(int64_t M, int64_t N, int64_t K, int64_t kalign, int64_t elem, const void *A,
             const void *B, const void *C, const float *C_f32);
// gfx950 check of the stream's device, then clear a stale HIP error
int prepare_launch(void *stream);
// one GEMM call as the entry points make it (validation included)
int gemm(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const void *A, const void *B, float sa,
         float sb, const void *SA, const void *SB, void *C, float *C_f32, void *stream,
         const hkg_gemm_opts *opts);
// the default schedule of a shape, a schedule's tile edge, the remap's clamp
hkg::Schedule default_schedule(hkg::Dtype dt, int64_t M, int64_t N);
int64_t tile_edge(hkg::Schedule s);
void clamp_remap(int64_t Gm, int64_t Gn, int64_t *W, int64_t *C);
// whether opts' schedule runs dtype dt (MXFP8: the 4-wave kernel only)
bool schedule_supported(hkg::Dtype dt, const hkg_gemm_opts *opts);
// the launches of a call with valid shapes and M, N > 0
int plan_gemm(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const hkg_gemm_opts *opts, Plan *pl);
// launch plan pl (arguments checked, device prepared)
int run_plan(hkg::Dtype dt, int64_t N, int64_t K, const Layout &L, const Plan &pl, const void *A,
             const void *B, float sa, float sb, const void *SA, const void *SB, void *C,
             float *C_f32, uint64_t *trace, void *stream);

}  // namespace hkg::api
