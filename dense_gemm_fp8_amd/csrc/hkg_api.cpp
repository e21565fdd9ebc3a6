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

// Operand sizes the MX scale entry points accept: rows below 2^31, one
// 256-row e4m3 panel (256 x K bytes) below 2 GiB as in the GEMM, and the
// packed scales below 2 GiB.  Each bound is checked before the next product
// is formed, so no caller value can wrap one into range.
bool mx_sizes_fit(int64_t rows, int64_t K)
{
    return rows < (int64_t(1) << 31) && K < (int64_t(1) << 31) / kTile &&
           mx_packed_bytes(rows, K) < (int64_t(1) << 31);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
    if (L->lda % (16 / elem) || L->ldb % (16 / elem))   // elem is 1 or 2
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
// ints.  The pitches are compared with a quotient, not multiplied, so that
// any int64_t a caller passes is rejected rather than wrapped.
bool sizes_fit(int64_t M, int64_t N, const Layout &L, int64_t elem)
{
    const int64_t max_pitch = (int64_t(1) << 31) / (kTile * elem);   // exact: a power of two
    return L.lda < max_pitch && L.ldb < max_pitch && L.ldc < (int64_t(1) << 31) &&
           M < (int64_t(1) << 31) && N < (int64_t(1) << 31) &&
           ceil_div(M, kTile) * ceil_div(N, kTile) < (int64_t(1) << 30);
}

// A tile grid the remap entry points accept: each side, then the product,
// below 2^30 (each side first, so that the product cannot wrap).
bool grid_fits(int64_t Gm, int64_t Gn)
{
    return Gm >= 1 && Gn >= 1 && Gm < (int64_t(1) << 30) && Gn < (int64_t(1) << 30) &&
           Gm * Gn < (int64_t(1) << 30);
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

bool opts_in_range(const hkg_gemm_opts *opts)
{
    return !opts || (opts->remap >= 0 && opts->remap <= 2 && opts->schedule >= 0 &&
                     opts->schedule <= 5 && opts->lda >= 0 && opts->ldb >= 0 && opts->ldc >= 0);
}

int gemm(hkg::Dtype dt, int64_t M, int64_t N, int64_t K, const void *A, const void *B, float sa,
         float sb, const void *SA, const void *SB, void *C, float *C_f32, void *stream,
         const hkg_gemm_opts *opts)
{
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
        if (!mx_sizes_fit(M, K) || !mx_sizes_fit(N, K))
            return HKG_ERR_SIZE;
        const int64_t sab = mx_packed_bytes(M, K), sbb = mx_packed_bytes(N, K);
        if (overlaps(C, cb, SA, sab) || overlaps(C, cb, SB, sbb) || overlaps(C_f32, fb, SA, sab) ||
            overlaps(C_f32, fb, SB, sbb))
            return HKG_ERR_OVERLAP;
    }
    if (M == 0 || N == 0)
        return schedule_supported(dt, opts) ? HKG_OK : HKG_ERR_OPTS;
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
    return run_plan(dt, N, K, L, pl, A, B, sa, sb, SA, SB, C, C_f32, trace, stream);
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
    if (!mx_sizes_fit(rows, K))
        return HKG_ERR_SIZE;
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
    if (!mx_sizes_fit(rows, K))
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
    if (!grid_fits(Gm, Gn) || W < 1 || C < 1 || panel_bytes < 0 || per_xcd < 1 || per_xcd > 1024)
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
    if (!grid_fits(Gm, Gn) || W < 1 || C < 1 || b < 0 || b >= Gm * Gn)
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
    if (!grid_fits(Gm, Gn) || W < 1 || C < 1)
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
    case HKG_ERR_SIZE:
        return "size beyond the 32-bit limits (a 2 GiB operand panel, M, N or ldc of 2^31, "
               "2^30 tiles, or 2 GiB of packed MXFP8 scales)";
    case HKG_ERR_OPTS: return "invalid hkg_gemm_opts";
    case HKG_ERR_DEVICE: return "the stream's device is not a gfx950, or could not be queried";
    case HKG_ERR_LAUNCH: return "kernel launch failed";
    case HKG_ERR_OVERLAP: return "an output overlaps an input or the other output";
    default: return "unknown status";
    }
}

int hkg_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
