// api_internal.h -- host logic of the C ABI shared between its source files
// (hkg_api.cpp: validation, launch planning and the GEMM calls; tune.cpp: the
// grid-order autotuner).  Not part of the installed interface.
#pragma once

#include <stdint.h>

#include "../../include/hkg.h"
#include "kernels.h"

namespace hkg::api {

constexpr int64_t kKAlignBf16 = 8;     // K granule: operand rows stay 16-byte aligned
constexpr int64_t kKAlignFp8 = 16;

int64_t ceil_div(int64_t a, int64_t b);
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

}  // namespace hkg::api
