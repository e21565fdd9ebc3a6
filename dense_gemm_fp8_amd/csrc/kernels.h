// kernels.h -- launch interface between the C ABI (launch.cpp) and the gfx950
// kernels (gemm_kernels.hip).  Internal to libhkg.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkg {

// Arguments of one GEMM launch.  All shape checks are done by the caller.
struct GemmParams {
    const void *A;      // [M][K] row-major, K contiguous, rows lda elements apart
    const void *B;      // [N][K] row-major, K contiguous, rows ldb elements apart
    void *C;            // [M][N] bf16 row-major, rows ldc elements apart
    float *C_f32;       // optional [M][N] fp32 pre-rounding copy, same ldc (nullptr = none)
    int M, N, K;
    int lda, ldb, ldc;  // row pitches in elements (>= K, K, N)
    int Gm, Gn;         // tile grid (M/256, N/256)
    int W, Cc;          // remap window height and per-XCD chunk
    int nk;             // number of K steps
    float scale;        // fp32(scale_a * scale_b) for e4m3, 1 for bf16 and MXFP8
    const void *SA;     // MXFP8: packed E8M0 scales of A (see hkg_mx_pack_scales), else null
    const void *SB;     // MXFP8: packed E8M0 scales of B
    int sa_bytes;       // sizes of the packed scale buffers
    int sb_bytes;
    uint64_t *trace;    // nullptr, or 8 words per workgroup of timestamps (hkg_gemm_opts::trace)
};

enum Dtype { kBf16 = 0, kFp8 = 1, kMx = 2 };
// kInterleave128 / kInterleave192: the 4-wave kernel on 128 x 128 / 192 x 192
// tiles (Gm, Gn count those)
enum Schedule {
    kPingPong = 0,
    kLockstep = 1,
    kInterleave = 2,
    kInterleave128 = 3,
    kInterleave192 = 4
};

hipError_t launch_gemm(Dtype dt, Schedule s, const GemmParams &p, hipStream_t stream);
hipError_t launch_remap_tiles(int Gm, int Gn, int W, int C, int32_t *out, hipStream_t stream);
// Diagnostic: the XCD and HW_ID of each of `workgroups` workgroups (out: 2 ints each).
hipError_t launch_xcd_probe(int workgroups, bool full_lds, int spin, int32_t *out,
                            hipStream_t stream);
// MXFP8 scale packing: src [rows][nblk] E8M0 bytes -> dst, groups x nk x 64 lanes x 8 bytes.
hipError_t launch_mx_pack(int operand, int rows, int nblk, int nk, int groups,
                          const uint8_t *src, uint8_t *dst, hipStream_t stream);

}  // namespace hkg
