/*
 * hkg.h -- C ABI of libhkg, a tiled dense GEMM for AMD MI355X (gfx950).
 *
 *     C[M][N] = A[M][K] * B[N][K]^T        fp32 accumulation
 *
 * The operation is the BF16 GEMM / FP8 GEMM of the HipKittens L2 note (section 3
 * "Target operation" table: BF16 inputs, FP32 accumulator, BF16 output), with
 * B used transposed as in the mma_ABt calls of the GEMM listing descriptions
 * (same note, sections 7 and 9.2).  Both operands are row-major with K contiguous
 * ("K-major"); C is row-major.  The fp8 variant takes OCP e4m3 bytes with one
 * fp32 scale per tensor and writes bf16  C = bf16(scale_a * scale_b * A*B^T).
 *
 * Launch shape (same note, section 3 "Launch config" and section 8 "Launch
 * shape"): one workgroup per 256 x 256 output tile -- 256 threads (4 waves,
 * the default 4-wave interleave) or 512 threads (8 waves, the ping-pong and
 * lockstep schedules) -- on a flat grid of ceil(M/256) * ceil(N/256)
 * workgroups (HKG_SCHED_INTERLEAVE_128 / _192: 128 x 128 / 192 x 192 tiles,
 * ceil(M/t) * ceil(N/t) workgroups of 256 threads), K consumed 64 (bf16) or
 * 128 (e4m3) at a time; rows past M or N and K past the end read as zeros.
 * Rows of A, B and C may be further apart than their length (row pitches,
 * hkg_gemm_opts lda / ldb / ldc).  Workgroup ids are remapped to tiles by the
 * chiplet-aware schedule of the same note, section 2 (Pillar 3) / section 7
 * (Algorithm 1), with window height W and per-XCD chunk C.
 *
 * Conventions for every entry point:
 *  - Pointers named A, B, C, C_f32 are DEVICE pointers allocated, owned and
 *    freed by the caller; the library never allocates, frees, copies to the
 *    host or synchronises (the one exception is the autotuner,
 *    hkg_tune_remap, which creates, waits for and destroys two HIP events).
 *    Work is enqueued on `stream` (a hipStream_t;
 *    NULL = the default stream) and completes asynchronously; buffers must
 *    stay alive until the stream has passed the kernel.
 *  - All arguments are validated before any HIP call.  On a validation error
 *    nothing is launched and C is untouched (a launch failure of the second
 *    of two default launches can leave the rows of the first written).
 *  - Return value: HKG_OK (0) or a negative hkg_status.
 *  - After validation and before its first launch, a call checks (once per
 *    device, then from a cache) that the device of `stream` is a gfx950
 *    (HKG_ERR_DEVICE otherwise) and clears any HIP error an earlier call left
 *    pending, so HKG_ERR_LAUNCH always names this call's own launch.
 *  - The library holds no mutable state apart from a thread-local copy of the
 *    last HIP error and that per-device architecture cache; it is safe to call
 *    from several host threads.
 */
#ifndef HKG_H
#define HKG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HKG_OK = 0,
    HKG_ERR_NULL = -1,    /* a required pointer is NULL                              */
    HKG_ERR_SHAPE = -2,   /* M, N, K negative, or K not a multiple of 8 (bf16) / 16 (e4m3)
                             / 32 (MXFP8)                                            */
    HKG_ERR_ALIGN = -3,   /* a pointer is not 16-byte aligned                        */
    HKG_ERR_SIZE = -4,    /* beyond the 32-bit limits: a 256-row operand panel of
                             2 GiB or more (256 * pitch * element size), M, N or
                             ldc of 2^31 or more, 2^30 tiles, or 2 GiB of packed
                             MXFP8 scales                                         */
    HKG_ERR_OPTS = -5,    /* invalid hkg_gemm_opts                                   */
    HKG_ERR_DEVICE = -6,  /* the device of `stream` (NULL: the current device) is not
                             a gfx950, or could not be queried; nothing launched  */
    HKG_ERR_LAUNCH = -7,  /* a kernel launch failed; see hkg_last_hip_error().  When
                             the call was split into two launches (hkg_launch_plan),
                             the rows of the first may already be written         */
    HKG_ERR_OVERLAP = -8  /* C or C_f32 shares bytes with A, B, the packed MXFP8
                             scales or the other output (A and B may alias)          */
} hkg_status;

/* Grid order (the remap of the HipKittens L2 note, section 2 Pillar 3 / section 7 Algorithm 1). */
enum {
    HKG_REMAP_DEFAULT = 0,  /* library's per-shape choice of (W, C)                */
    HKG_REMAP_ROW_MAJOR = 1,/* identity order (W = 1, C = 1)                       */
    HKG_REMAP_XCD = 2       /* explicit window height W >= 1 and chunk C >= 1       */
};

/* In-CU schedule (HipKittens L2 note, section 2 Pillar 2 and section 9.2). */
enum {
    HKG_SCHED_DEFAULT = 0,  /* 4-wave interleave: HKG_SCHED_INTERLEAVE, or
                               HKG_SCHED_INTERLEAVE_128 when
                               ceil(M/256) * ceil(N/256) <= 128, i.e. when 256 x 256
                               tiles would leave over half of the 256 CUs idle.
                               bf16 and e4m3: HKG_SCHED_INTERLEAVE_192 instead when
                               ceil(M/192) * ceil(N/192) <= 256 while
                               ceil(M/128) * ceil(N/128) > 256 (one 192 x 192 tile
                               per CU in one round, where 128 x 128 ones would not
                               fit one round), or when the 192 x 192 tiles fill
                               whole rounds of 256 while the 256 x 256 grid ends
                               in a round at least a quarter full.
                               With the default order, a 256 x 256
                               grid whose last round is partial may run as two
                               launches on `stream`: the tile rows of the whole
                               rounds on 256 x 256 tiles, the remaining rows on
                               128 x 128 tiles (same result bit for bit)          */
    HKG_SCHED_PINGPONG = 1, /* 8-wave ping-pong: 2 groups of 4 waves alternate the
                               MFMA and HBM->LDS roles via s_setprio + barriers      */
    HKG_SCHED_LOCKSTEP = 2, /* all 8 waves compute the same K step (ablation only)   */
    HKG_SCHED_INTERLEAVE = 3,/* 4 waves (one per SIMD), each 128 x 128 of the tile,
                               loads and LDS reads slotted between its own MFMAs
                               (the note's 4-wave interleave: section 2 Pillar 2,
                               section 5 GEMM, Figure 6 right)                       */
    HKG_SCHED_INTERLEAVE_128 = 4, /* the same schedule on 128 x 128 output tiles (each
                               wave 64 x 64; 80 KiB of LDS, two workgroups per CU):
                               four times the tiles, for grids too small to fill the
                               GPU with 256 x 256 ones                              */
    HKG_SCHED_INTERLEAVE_192 = 5  /* the same schedule on 192 x 192 output tiles (each
                               wave 96 x 96; 120 KiB of LDS, one workgroup per CU),
                               for grids that fit one round of 256 CUs in 192 x 192
                               tiles but not in 128 x 128 ones; bf16 and e4m3        */
};

typedef struct {
    int32_t remap;     /* HKG_REMAP_*                                  */
    int32_t W;         /* window height in tile rows (HKG_REMAP_XCD)   */
    int32_t C;         /* consecutive tiles per XCD (HKG_REMAP_XCD)    */
    int32_t schedule;  /* HKG_SCHED_*                                  */
    uint64_t *trace;   /* NULL, or a per-workgroup time record (below) */
    int64_t lda;       /* row pitches in elements, 0 = dense rows: A (K), */
    int64_t ldb;       /* B (K) and C / C_f32 (N); see "Row pitches"     */
    int64_t ldc;
} hkg_gemm_opts;

/*
 * Row pitches (hkg_gemm_opts lda, ldb, ldc).  Row m of A starts lda elements
 * after row m - 1 (likewise B with ldb, and C and C_f32 with ldc), so a caller
 * can pass a sub-matrix of a wider one, or pad rows: operand rows of m x 8 KiB
 * with m not a power of two (e.g. bf16 K = 12288 or 28672) make the L2 stall
 * on tag lookups, which a pitch 128 bytes longer avoids.  Rules: lda, ldb >= K
 * with lda * element size and ldb * element size multiples of 16
 * (HKG_ERR_ALIGN); ldc >= N (C rows are then written element by element unless
 * N and ldc are multiples of 8); 0 selects the dense pitch; a pitch below its
 * extent or negative is HKG_ERR_OPTS; 256 * pitch * element size must stay
 * below 2^31 and ldc below 2^31 (HKG_ERR_SIZE; any larger value, up to
 * INT64_MAX, is refused without being multiplied).  The bytes between rows
 * are neither read into the result nor written.  Overlap checks take each
 * matrix to span its first to its last element.
 */

/*
 * Time record (hkg_gemm_opts.trace): a device buffer, 8-byte aligned, of
 * 8 uint64 per workgroup of the call (the sum of grid[i] over its launches,
 * see hkg_launch_plan; launch i's workgroups follow those of launches < i).
 * Workgroup b writes, from one lane, words 8b .. 8b+7:
 *   0, 1, 2  the 100 MHz real-time counter at its start, at the end of its K
 *            loop and after its last store was issued (one wave's view)
 *   3, 4, 5  the shader-clock counter at the same three points, so that
 *            (w4 - w3) / (w1 - w0) * 100 MHz is the clock the K loop ran at
 *   6        the XCC_ID hardware register (bits 3:0: the XCD it ran on)
 *   7        (tile_m << 32) | tile_n, the output tile it computed
 * The buffer must not overlap A, B, C or C_f32 (HKG_ERR_OVERLAP).  Writing the
 * record costs one 64-byte store per workgroup; the arithmetic is unchanged.
 */

/*
 * bf16 GEMM.
 *   A      [M][K] bfloat16, row-major (K contiguous), device, 16-byte aligned
 *   B      [N][K] bfloat16, row-major (K contiguous), device, 16-byte aligned
 *   C      [M][N] bfloat16, row-major, device, 16-byte aligned; written
 *          with round-to-nearest-even from the fp32 accumulator
 *   C_f32  NULL, or [M][N] fp32 row-major: the pre-rounding accumulator
 *          (validation launches only; costs extra stores)
 * Shapes: any M, N >= 0; K >= 0 with K % 8 == 0 so operand rows stay 16-byte
 * aligned (K == 0 writes zeros; M == 0 or N == 0 is a no-op).  Edge tiles
 * (M or N not multiples of 256, K not a multiple of 64) are handled inside the
 * kernels.  C and C_f32 must not share a byte with A, B or each other
 * (HKG_ERR_OVERLAP); A and B may be the same buffer.
 */
int hkg_gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                  void *C, float *C_f32, void *stream);

/*
 * fp8 (OCP e4m3) GEMM with per-tensor scales.
 *   A [M][K], B [N][K]: e4m3 bytes (S.EEEE.MMM, bias 7, max 448), row-major
 *   scale_a, scale_b: host fp32 per-tensor dequantisation scales
 *   C [M][N] bfloat16 = RNE(fp32(scale_a*scale_b) * fp32 accumulator)
 *   C_f32: NULL or the scaled fp32 value before rounding
 * Shapes: any M, N >= 0; K >= 0 with K % 16 == 0.  Otherwise as above.
 * Accuracy: K is consumed in steps of 128 (a partial step first when K is not
 * a multiple of 128).  The gfx950 e4m3 matrix instruction sums the 128
 * products of a step with about 13 bits below the largest of them before
 * adding the fp32 accumulator, so for any inputs
 *   |C_f32 - exact| <= sa*sb * ( 2^-6 * sum_steps max_k |a_k b_k|
 *                                + steps * 2^-24 * sum_k |a_k b_k| ),
 * and sums whose products all lie within that window (e.g. small integers)
 * are exact.  For per-tensor-quantised N(0,1) data the error is far smaller
 * (8192^3, every entry: max 0.009 against 1e-3 * sqrt(K) = 0.09).
 */
int hkg_gemm_fp8(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                 float scale_a, float scale_b, void *C, float *C_f32, void *stream);

/* As above with an explicit grid order / schedule (opts may be NULL = defaults). */
int hkg_gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                     void *C, float *C_f32, void *stream, const hkg_gemm_opts *opts);
int hkg_gemm_fp8_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                    float scale_a, float scale_b, void *C, float *C_f32, void *stream,
                    const hkg_gemm_opts *opts);

/*
 * MXFP8 GEMM: the "MXFP8" input type of the HipKittens L2 note (section 3,
 * "Target operation" table), in the OCP Microscaling Formats v1.0 encoding.
 *   A [M][K], B [N][K]: e4m3 bytes, row-major
 *   each run of 32 consecutive elements along K of a row has one E8M0 scale
 *   byte E standing for 2^(E-127) (0xFF = NaN); element k of row r of A means
 *   e4m3(A[r][k]) * 2^(SA[r][k/32]-127), likewise for B
 *   SA_packed, SB_packed: those scales after hkg_mx_pack_scales (operand A
 *   resp. B), device, 16-byte aligned, hkg_mx_packed_scale_bytes(M resp. N, K)
 *   bytes
 *   C [M][N] bfloat16 = RNE(fp32 accumulator); C_f32: NULL or that fp32 value
 * Shapes: any M, N >= 0; K >= 0 with K % 32 == 0.  Otherwise as the bf16
 * entry point.  Runs the 4-wave interleave kernel on either tile
 * (opts->schedule must be HKG_SCHED_DEFAULT, HKG_SCHED_INTERLEAVE or
 * HKG_SCHED_INTERLEAVE_128, else HKG_ERR_OPTS); one packed layout serves
 * both tiles.
 */
int hkg_gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                   const void *SA_packed, const void *SB_packed, void *C, float *C_f32,
                   void *stream);
int hkg_gemm_mxfp8_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                      const void *SA_packed, const void *SB_packed, void *C, float *C_f32,
                      void *stream, const hkg_gemm_opts *opts);

/* Which operand a packed scale buffer is for. */
enum { HKG_MX_OPERAND_A = 0, HKG_MX_OPERAND_B = 1 };

/*
 * Bytes of the packed scales of one MXFP8 operand with `rows` rows:
 * ceil(rows/128) * ceil(K/128) * 512 (host only).  Negative hkg_status:
 * HKG_ERR_SHAPE if rows < 0, K < 0 or K % 32 != 0; HKG_ERR_SIZE for sizes
 * hkg_mx_pack_scales refuses (rows >= 2^31, K >= 2^23, or 2 GiB of packed
 * scales).
 */
int64_t hkg_mx_packed_scale_bytes(int64_t rows, int64_t K);

/*
 * Rearrange one operand's E8M0 scales into the order the GEMM kernel reads.
 *   scales  [rows][K/32] bytes, row-major, device (no alignment needed)
 *   packed  device, 16-byte aligned, hkg_mx_packed_scale_bytes(rows, K) bytes,
 *           caller-owned; must not overlap `scales` (HKG_ERR_OVERLAP)
 * Layout: byte e (0..7) of lane l (0..63) of K step t of 128-row group g, at
 * offset ((g * ceil(K/128) + t) * 64 + l) * 8 + e, is the scale of row
 * 128 g + rho(e, l) and k block 4 t + l / 16, where with x = l % 16
 *   operand A: rho = 16 e + x
 *   operand B: rho = 32 (e >> 1) + 4 (e & 1) + (x & 3) + 8 (x >> 2)
 * Rows past `rows` and blocks past K/32 read 127 (scale 1).  Enqueued on
 * `stream`; weights' scales can be packed once and reused.  HKG_ERR_SIZE if
 * rows >= 2^31, K >= 2^23 (the GEMM's own bound) or the packed size reaches
 * 2 GiB.
 */
int hkg_mx_pack_scales(int32_t operand, int64_t rows, int64_t K, const void *scales,
                       void *packed, void *stream);

/*
 * The (W, C) the library uses for HKG_REMAP_DEFAULT on a shape (host only, no
 * HIP call).  dtype: 0 = bf16, 1 = fp8, 2 = MXFP8.  Returns HKG_ERR_NULL,
 * HKG_ERR_SHAPE or HKG_ERR_SIZE as hkg_launch_plan does on bad input.  The
 * grid is that of the default call's first launch (hkg_launch_plan: W[0],
 * C[0]; tiles of 256, or of 128 / 192 where HKG_SCHED_DEFAULT picks them).
 * Rule (the L2 and LLC terms of the HipKittens L2 note's section 4
 * equation): (8, 32) while an operand row
 * holds at most 18944 bytes (K x element size), else (16, 4).  Both keep each
 * XCD's 32 concurrent tiles on 12 operand panels (the same L2 hit rate); the
 * second's 256 concurrent tiles share fewer panels (32 instead of 40), which
 * keeps a round's panels inside the last-level cache for long rows.  Both
 * are clamped to the grid (W <= tile rows, C <= tiles/8 + 1).
 */
int hkg_default_remap(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t *W, int32_t *C);

/*
 * What a GEMM call with these shapes and options launches (host only, no HIP
 * call; the entry points build their launches from the same plan).  Up to two
 * launches, over consecutive ranges of output rows (the second only for the
 * default split of a partial last round, see HKG_SCHED_DEFAULT).
 *   launches     0 (M == 0 or N == 0), 1 or 2
 *   schedule[i]  HKG_SCHED_* that launch i runs (never HKG_SCHED_DEFAULT)
 *   tile[i]      its output tile edge, 256, 192 or 128
 *   rows[i]      output rows it covers; launch 1 starts at row rows[0]
 *   grid[i]      its workgroups (tiles)
 *   W[i], C[i]   its grid order
 * dtype: 0 = bf16, 1 = e4m3, 2 = MXFP8; opts may be NULL (defaults).  Returns
 * the status the GEMM entry point would return for the shape and options
 * (HKG_ERR_SHAPE, HKG_ERR_SIZE, HKG_ERR_OPTS) or HKG_ERR_NULL for plan == NULL.
 */
typedef struct {
    int32_t launches;
    int32_t schedule[2];
    int32_t tile[2];
    int64_t rows[2];
    int64_t grid[2];
    int32_t W[2];
    int32_t C[2];
} hkg_launch_plan_t;

int hkg_launch_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, const hkg_gemm_opts *opts,
                    hkg_launch_plan_t *plan);

/*
 * The cache model behind the default grid order (host only, no HIP call):
 * for a Gm x Gn tile grid walked in order (W, C), with operand panels of
 * panel_bytes (tile rows x K x element size) and per_xcd workgroups in
 * flight per XCD (32 CUs x workgroups per CU: 32 for 256 x 256 and 192 x 192
 * tiles, 64 for 128 x 128), the predicted
 *   l2_hit      fraction of operand-panel requests served by an XCD's L2
 *               (its concurrent tiles stream the same K steps together, so a
 *               panel misses once per round: 1 - distinct panels / requests)
 *   llc_hit     fraction of L2 misses served by the 256 MiB last-level cache
 *               (a panel another XCD fetches in the same round, or one used in
 *               the previous round when that round's panels fit the cache)
 *   eq1_bw_tbs  5.99 * llc_hit + 17.05 * l2_hit (TB/s; the constants fit every
 *               row of the note's Table 4, section 5)
 * Workgroup b is taken to run on XCD b mod 8 (hkg_probe_xcd checks it), and
 * rounds of 8 * per_xcd workgroups to run together; the first 8 rounds are
 * simulated.  An analysis aid: the default order (hkg_default_remap) is the
 * measured rule, which this model's L2 term explains.
 * Returns HKG_ERR_NULL / HKG_ERR_SHAPE on bad input.
 */
int hkg_remap_model(int64_t Gm, int64_t Gn, int32_t W, int32_t C, int64_t panel_bytes,
                    int32_t per_xcd, double *l2_hit, double *llc_hit, double *eq1_bw_tbs);

/*
 * Candidate grid orders of a shape, best first by the cache model's Eq. 1
 * bandwidth (HipKittens L2 note, section 4 equation; section 5 Table 4 tunes W
 * and C per shape).  Host only, no HIP call.  The grid is the one the default
 * schedule picks for the shape (tiles of 256, 192 or 128, one launch); the
 * candidates are W in {1, 2, 4, 8, 16, 32} x C in {1, 2, 4, 8, 16, 32, 64,
 * 128}, clamped to the grid as hkg_remap_model clamps them and with duplicates
 * removed (at most 48), ranked by eq1_bw_tbs of hkg_remap_model (ties keep that
 * enumeration order).  Writes the first min(max, count) entries to W[i], C[i],
 * eq1_bw_tbs[i] and the number of candidates to *count (0 for M == 0 or
 * N == 0).  dtype: 0 = bf16, 1 = e4m3, 2 = MXFP8.  Returns HKG_ERR_NULL for a
 * NULL pointer (W, C, eq1_bw_tbs may be NULL when max == 0), HKG_ERR_SHAPE as
 * hkg_launch_plan does, HKG_ERR_SIZE for grids the entry points refuse.
 */
int hkg_remap_candidates(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t max,
                         int32_t *W, int32_t *C, double *eq1_bw_tbs, int32_t *count);

/*
 * Grid-order autotuner (HipKittens L2 note, section 5 Table 4: the order is
 * tuned per shape).  Times, on the caller's buffers and stream, the default
 * launch of this GEMM and, with the default schedule, the best-ranked order of
 * hkg_remap_candidates for each window height W that occurs in that list (at
 * most 6; the model often ties orders that differ only in C) plus row-major
 * order if it is not among them, and returns the fastest as options for the
 * _ex entry points.
 *   dtype     0 = bf16, 1 = e4m3 (MXFP8 moves the same operand bytes as e4m3:
 *             tune it with dtype 1 on its element arrays)
 *   A, B, C   as for hkg_gemm_bf16 / hkg_gemm_fp8 (same checks); C is
 *             overwritten, every time with the product A·Bᵀ (unit scales for e4m3)
 *   launches  timed launches per candidate and pass, 1 .. 1000
 *   best      out: {HKG_REMAP_DEFAULT, default W, default C, HKG_SCHED_DEFAULT,
 *             NULL} when the default launch won, else {HKG_REMAP_ROW_MAJOR or
 *             HKG_REMAP_XCD, W, C, HKG_SCHED_DEFAULT, NULL}
 *   best_ms   out (may be NULL): the winner's mean time per launch, ms
 *   tried, tried_ms, n_tried
 *             out (all NULL, or arrays of HKG_TUNE_MAX_CANDIDATES entries and
 *             a count): every configuration timed, the default launch first,
 *             with its mean time per launch, ms
 * Procedure: about 100 ms of default launches first (the clock of an idle GPU
 * takes that long to settle under its power cap), then every candidate is
 * timed twice, in forward and then reverse order, each time after one untimed
 * launch, with HIP events on `stream`.  Unlike the GEMM entry points this call
 * creates two HIP events, waits for them on the host and destroys them; it
 * returns when its last launch has finished.  M == 0 or N == 0: no launch,
 * best = the defaults, *best_ms = 0, *n_tried = 0.  Returns the entry points'
 * status codes, plus HKG_ERR_NULL for best == NULL or for only some of tried,
 * tried_ms, n_tried given, HKG_ERR_SHAPE for another dtype and
 * HKG_ERR_OPTS for launches outside 1 .. 1000; on HKG_ERR_LAUNCH (event or
 * launch failure, see hkg_last_hip_error) `best` is left unchanged.
 */
#define HKG_TUNE_MAX_CANDIDATES 8
int hkg_tune_remap(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B,
                   void *C, int32_t launches, hkg_gemm_opts *best, float *best_ms,
                   hkg_gemm_opts *tried, float *tried_ms, int32_t *n_tried, void *stream);

/*
 * The grid remap itself (HipKittens L2 note, section 7 Algorithm 1 reading): flat
 * workgroup id b of a Gm x Gn tile grid -> output tile (tile_m, tile_n) for
 * window height W and chunk C.  Host function, no HIP call.  Returns
 * HKG_ERR_NULL for a NULL output, HKG_ERR_SHAPE if Gm or Gn is below 1, either
 * side or Gm*Gn reaches 2^30, W or C is below 1, or b is outside [0, Gm*Gn).
 * W and C are clamped to the grid as hkg_remap_model describes.
 */
int hkg_remap_tile(int64_t Gm, int64_t Gn, int32_t W, int32_t C, int64_t b,
                   int64_t *tile_m, int64_t *tile_n);

/*
 * The same remap evaluated by the device code the GEMM kernels use: writes
 * out[2*b] = tile_m, out[2*b+1] = tile_n for every b in [0, Gm*Gn).
 *   out: device int32 array of 2*Gm*Gn elements, caller-owned, 4-byte aligned
 *        (HKG_ERR_ALIGN).
 * Grid checks as hkg_remap_tile (HKG_ERR_NULL, HKG_ERR_SHAPE), then the device
 * check of every launching entry point.
 */
int hkg_remap_tiles_device(int64_t Gm, int64_t Gn, int32_t W, int32_t C, int32_t *out,
                           void *stream);

/*
 * Diagnostic of the premise behind the grid remap: the remap (HipKittens L2
 * note, section 2 Pillar 3 and section 7 code citation 5, Algorithm 1's
 * "de-interleave round-robin" step) assumes that the hardware hands
 * workgroup b of a launch to XCD b mod 8.  This launches `workgroups`
 * workgroups of 256 threads; each records where it ran:
 *   out[2*b]     the XCC_ID hardware register (bits 3:0: the XCD)
 *   out[2*b + 1] the HW_ID hardware register (wave slot, SIMD, CU, shader
 *                array and engine ids)
 * full_lds = 1: each workgroup declares the whole 160 KiB of LDS, as the
 * 256 x 256 GEMM kernels do (at most one per CU); 0: 256 bytes.  Workgroup b
 * first waits ((b*37) % 64) * spin_cycles / 64 shader clock cycles (a bounded
 * wait), so that workgroups finish out of order.
 *   out: device int32[2*workgroups], caller-owned, 4-byte aligned.
 * 1 <= workgroups <= 2^24 and 0 <= spin_cycles <= 2^24, else HKG_ERR_SHAPE.
 */
int hkg_probe_xcd(int64_t workgroups, int32_t full_lds, int32_t spin_cycles, int32_t *out,
                  void *stream);

/* Static description of a status code. */
const char *hkg_status_string(int status);

/* hipError_t behind the last HKG_ERR_LAUNCH / HKG_ERR_DEVICE on this thread. */
int hkg_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HKG_H */
