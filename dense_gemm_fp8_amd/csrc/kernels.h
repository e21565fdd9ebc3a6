// kernels.h -- launch interface between the C ABI (hkg_api.cpp) and the gfx950
// kernels (gemm_kernels.hip).  Internal to libhkg.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkg {

// Arguments of one GEMM launch.  All shape checks are done by the caller.
struct GemmParams {
    const void *A;      // [M][K] row-major, K contiguous
    const void *B;      // [N][K] row-major, K contiguous
    void *C;            // [M][N] bf16 row-major
    float *C_f32;       // optional [M][N] fp32 pre-rounding copy (nullptr = none)
    int M, N, K;
    int Gm, Gn;         // tile grid (M/256, N/256)
    int W, Cc;          // remap window height and per-XCD chunk
    int nk;             // number of K steps
    float scale;        // fp32(scale_a * scale_b) for e4m3, 1 for bf16
};

enum Dtype { kBf16 = 0, kFp8 = 1 };
enum Schedule { kPingPong = 0, kLockstep = 1, kInterleave = 2 };

hipError_t launch_gemm(Dtype dt, Schedule s, const GemmParams &p, hipStream_t stream);
hipError_t launch_remap_tiles(int Gm, int Gn, int W, int C, int32_t *out, hipStream_t stream);

}  // namespace hkg
