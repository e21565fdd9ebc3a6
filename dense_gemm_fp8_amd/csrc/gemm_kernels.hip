// gemm_kernels.hip -- gfx950 (MI355X) kernels for C = A * B^T.
//
// One workgroup computes one 256 x 256 output tile (HipKittens L2 note,
// section 3 "Launch config": BLOCK 256 x 256, K_STEP 64, DOT_SLICE 32, MFMA
// 16x16x32).  Two kernels share the data path and the LDS ring below:
//   gemm_kernel   512 threads, 8 waves as WARPS_M = 2 x WARPS_N = 4 (the
//                 ping-pong and lockstep schedules)
//   gemm4_kernel  256 threads, 4 waves of 128 x 128 each (the 4-wave
//                 interleave, the library's default; see its section below)
//
// Data path of one K step:
//   HBM/L2 --buffer_load_dwordx4 ... lds--> LDS stage --ds_read_b128--> VGPR
//   fragments --v_mfma--> fp32 accumulators (HipKittens L2 note, section 2 Pillar 1:
//   direct HBM->LDS loads that bypass the register file, with the XOR swizzle
//   applied to the HBM address).
//
// LDS (the full 160 KiB of a gfx950 CU):
//   A ring: 2 panels [256 rows][128 B] (K step k in panel k % 2)
//   B ring: 3 panels [256 rows][128 B] (K step k in panel k % 3)
//   one 128-byte row = one K step of one operand row (64 bf16 or 128 e4m3)
//   row r stores its eight 16-byte chunks permuted: chunk c lives in slot
//   c ^ x(r), with x = slot_xor_a for A panels and slot_xor_b for B panels
//   (defined below; one map per operand).
// The pages keep a 2-deep LDS double buffer (HipKittens L2 note, section 4 "Pipeline
// depth"); the third B panel here exists so that the ping-pong below can
// prefetch register fragments one phase early while the shared B panel still
// has three phases to arrive from HBM.
//
// Edges: the buffer resource of a tile's panel spans exactly its valid rows,
// and a buffer load whose offset (voffset + soffset) is out of range writes
// zeros into LDS, so rows past M or N arrive as zeros.  In a last, partial K
// step the lanes whose 16-byte chunk lies past K get an out-of-range voffset
// (chunks never straddle K: K is a multiple of 8 bf16 / 16 e4m3).  Stores
// skip rows >= M and columns >= N.
//
// A buffer load with the LDS bit writes lane l's 16 bytes to LDS address
// M0 + 16*l, so one instruction fills 8 consecutive rows (1 KiB).  The lane
// therefore cannot choose where its bytes land; instead each lane fetches the
// global chunk that belongs in its fixed slot: lane l -> row 8u + l/8,
// slot l%8, global chunk (l%8) ^ x(row).  This is the "swizzle applied
// to the HBM address" of the HipKittens L2 note (section 2) and summary page.
//
// Waves and the output tile (WARPS_M = 2 x WARPS_N = 4):
//   wave w: group g = w / 4 owns tile rows [128 g, 128 g + 128),
//           wn = w % 4 owns tile columns [64 wn, 64 wn + 64)
//   -> a 128 x 64 fp32 sub-tile = 8 x 4 MFMA blocks of 16 x 16 = 128 fp32
//      accumulator registers per lane (HipKittens L2 note, section 4 "Tile / launch
//      optimality": the register budget at 2 waves per SIMD).
//
// MFMA operand order: the B fragment is the instruction's first (row) operand
// and the A fragment its second (column) operand, so each 16 x 16 result block
// is C^T and a lane holds 4 consecutive output COLUMNS of one output row.  The
// B rows fed to the four column blocks j are interleaved (block j, operand row
// 4a + b -> tile column 8a + b + 4 (j & 1) + 32 (j >> 1)) so that blocks j = 0,1
// give a lane 8 consecutive bf16 (one 16-byte store) and j = 2,3 another 8.
//
// Schedules (HipKittens L2 note, section 2 Pillar 2; the ping-pong in
// sections 9.1 and 9.2, the 4-wave interleave in section 4 "% peak
// derivation" and section 5, GEMM, Figure 6 right):
//   kPingPong  8-wave ping-pong.  Group 0 (waves 0-3, one per SIMD) and group
//              1 (waves 4-7) run one barrier apart: while one group issues its
//              MFMA cluster at s_setprio 3 the other issues the next K steps'
//              HBM->LDS loads and reads all of its own next cluster's
//              fragments from LDS into registers, so a cluster holds no LDS
//              instruction and starts with MFMAs.  Group 1 starts
//              with a memory phase, which staggers it one phase behind group 0:
//              the conditional extra barrier wait that the pages' GEMM entry
//              gives one wave group (HipKittens L2 note, section 7 code
//              citation 1 and section 9.1) does the same there; s_barrier is
//              the only synchronisation.
//   kLockstep  all 8 waves compute the same K step and share the loads
//              (no ping-pong; kept as an ablation).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.h"
#include "remap.h"

namespace hkg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTile = 256;                        // output tile edge
constexpr int kRowBytes = 128;                    // one K step of one row
constexpr int kPanelBytes = kTile * kRowBytes;    // 32 KiB
constexpr int kAPanels = 2;                       // A ring depth
constexpr int kBPanels = 3;                       // B ring depth
constexpr int kBRing = kAPanels * kPanelBytes;    // byte offset of the B ring
constexpr int kLdsBytes = (kAPanels + kBPanels) * kPanelBytes;   // 160 KiB
constexpr int kDmaBytes = 64 * 16;                // one wave-wide 16 B/lane load
constexpr int kDmaRows = kDmaBytes / kRowBytes;   // = 8 rows per load

// Slot permutations of LDS row r, one per operand.  A 16-lane group of a
// ds_read_b128 reads one 16-byte chunk from 16 rows; for conflict-free
// banking those 16 reads must hit 16 different 16-byte slots of a 256-byte
// bank line (64 banks x 4 B).  Two rows share a bank line (row bit 0), so for
// each row parity the 8 rows of a group must get 8 different XOR values.  The
// A fragment reads vary row bits 1,2,3 within a 16-lane group and B's
// interleaved reads bits 1,3,4, so
//   A: slot = chunk ^ (b1 | b3 << 1 | b2 << 2)   (independent of row bit 4)
//   B: slot = chunk ^ (b1 | b3 << 1 | b4 << 2)   (independent of row bit 2)
// are bank-conflict free, and the two row parities of a fragment pair (A
// rows 16 apart, B rows 4 apart) lie a constant 2048 / 512 bytes apart, so
// one lane base per operand and chunk half serves every block.
__device__ __forceinline__ int slot_xor_a(int r)
{
    return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2);
}
__device__ __forceinline__ int slot_xor_b(int r)
{
    return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 4) & 1) << 2);
}

// An empty asm that claims to change x.  Applied to the lane base address of
// a half, it stops the optimiser from folding a panel's offset into a
// separate precomputed address per fragment read (one register each, and one
// vector add each per K step): every read stays one ds_read of
// (base + constant block offset).
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroup barrier that is also a compiler barrier for memory accesses; it
// deliberately does not wait for outstanding HBM->LDS loads (the schedules
// wait for exactly the loads they need with wait_vmcnt).
__device__ __forceinline__ void block_barrier()
{
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // dword3 0x00020000: raw (untyped) 32-bit buffer access on gfx9-family parts.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

constexpr int kOutOfRange = int(0x80000000u);   // voffset past any panel's range

// Byte range of a panel of `rows` operand rows `pitch` bytes apart, each
// holding kb bytes of K: it ends with the last row's K bytes, so loads past
// them (a partial K step's lanes, or the padding after the last row) read
// zeros.
__device__ __forceinline__ uint32_t panel_bytes(int rows, int pitch, int kb)
{
    return rows > 0 ? (uint32_t)(rows - 1) * (uint32_t)pitch + (uint32_t)kb : 0u;
}

// voffset for K step k: the lane's own offset, or out of range if its chunk
// (at byte cbytes of the K step) lies past the row's kb bytes of K.
__device__ __forceinline__ int kstep_voff(int voff, int cbytes, int k, int kb)
{
    return k * kRowBytes + cbytes < kb ? voff : kOutOfRange;
}

// One wave-wide HBM->LDS load of 8 panel rows (u = row group, 0..31) of an
// operand whose rows are `pitch` bytes apart.
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, char *panel, int u, int voff,
                                         int soff_kstep, int pitch)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(panel + u * kDmaBytes), 16, voff,
                                             soff_kstep + u * kDmaRows * pitch, 0, 0);
}

// Row groups u = base + (wave & 3) + 4 v, v < count: every lane of a wave
// then shares the same row bits 3,4 ((u & 3) == (wave & 3)), so one per-lane
// offset serves all its loads.
template <int kCount>
__device__ __forceinline__ void dma_panel_part(__amdgpu_buffer_rsrc_t rs, char *panel, int base,
                                               int w4, int voff, int soff_kstep, int pitch)
{
#pragma unroll
    for (int v = 0; v < kCount; ++v)
        dma_rows(rs, panel, base + w4 + 4 * v, voff, soff_kstep, pitch);
}

template <int kDtype>
struct Frag;
template <>
struct Frag<kBf16> {
    using T = bf16x8;
    static constexpr int kSlices = 2;   // DOT_SLICE 32 twice per K step of 64
    __device__ __forceinline__ static T load(const char *p, int off0, int off1, int s)
    {
        return *reinterpret_cast<const bf16x8 *>(p + (s ? off1 : off0));
    }
    __device__ __forceinline__ static f32x4 mma(const T &x, const T &y, const f32x4 &c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    }
};
template <>
struct Frag<kFp8> {
    using T = i32x8;
    static constexpr int kSlices = 1;   // one 16x16x128 step per K step of 128
    __device__ __forceinline__ static T load(const char *p, int off0, int off1, int)
    {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(p + off0);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(p + off1);
        return T{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    __device__ __forceinline__ static f32x4 mma(const T &x, const T &y, const f32x4 &c)
    {
        // format selectors 0/0 = OCP e4m3 for both operands; the zero scale
        // operands select the unscaled instruction.
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
    }
};

// Lane part of a fragment read, chunk half h (chunk 4 h + q): A row x, B row
// (x & 3) + 8 (x >> 2) of a block pair, x = lane % 16, q = lane / 16.  For
// bf16 the halves are the two DOT_SLICEs.  For e4m3 this is the 16x16x128
// MFMA's own k order (lane group q supplies k 16q..16q+15 and 64 + 16q..+15,
// probed on gfx950); the block-scaled form applies the scale in lane group b
// to the 32 k of block b, so the MXFP8 scales follow the same order.
struct QuadLane {
    int a[2], b[2];
};
__device__ __forceinline__ QuadLane quad_lane(int lane)
{
    const int x = lane & 15, q = lane >> 4;
    const int rb = (x & 3) + 8 * (x >> 2);
    QuadLane l;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        l.a[h] = x * kRowBytes + (((4 * h + q) ^ slot_xor_a(x)) << 4);
        l.b[h] = rb * kRowBytes + (((4 * h + q) ^ slot_xor_b(rb)) << 4);
    }
    return l;
}

// Per-lane LDS byte offsets of the fragment reads (relative to a 32-row
// group).  [parity][h]: h selects chunk q (h = 0) or chunk 4 + q (h = 1),
// i.e. the two DOT_SLICEs of bf16 or the two halves of an e4m3 fragment.
struct LaneOffsets {
    int a[2][2];
    int b[2][2];
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane)
{
    const int x = lane & 15;      // operand row inside a 16-row block
    const int q = lane >> 4;      // k chunk group
    LaneOffsets o;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int ra = 16 * p + x;
        const int rb = (x & 3) + 4 * p + 8 * (x >> 2);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            o.a[p][h] = ra * kRowBytes + (((4 * h + q) ^ slot_xor_a(ra)) << 4);
            o.b[p][h] = rb * kRowBytes + (((4 * h + q) ^ slot_xor_b(rb)) << 4);
        }
    }
    return o;
}

// Offsets of fragment i of A (16-row block) and j of B (32-row half) from a
// wave's first row in a panel (lockstep schedule).
__device__ __forceinline__ constexpr int a_blk(int i) { return 16 * (i & ~1) * kRowBytes; }
__device__ __forceinline__ constexpr int b_blk(int j) { return 32 * (j >> 1) * kRowBytes; }

// The MFMA cluster of one K step for one wave, all fragments read inside the
// cluster (used by the lockstep schedule): 8 x 4 blocks of 16 x 16.
template <int kDtype>
__device__ __forceinline__ void compute_kstep(const char *a_base, const char *b_base,
                                              const LaneOffsets &o, f32x4 (&acc)[8][4])
{
    using F = Frag<kDtype>;
#pragma unroll
    for (int s = 0; s < F::kSlices; ++s) {
        typename F::T bf[4], af[8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = F::load(b_base + b_blk(j), o.b[j & 1][0], o.b[j & 1][1], s);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            af[i] = F::load(a_base + a_blk(i), o.a[i & 1][0], o.a[i & 1][1], s);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = F::mma(bf[j], af[i], acc[i][j]);
    }
}

// Fragments of one K step for the ping-pong.  A wave reads all of them
// (24 ds_read_b128, 96 VGPRs per lane) in its memory phase, after issuing its
// loads, while its partner runs MFMAs, so the MFMA cluster itself contains no LDS
// instruction and issues back to back.  Every read is one ds_read_b128 of a
// lane base plus an immediate block offset (the per-operand swizzles make
// one base per operand and chunk half serve every block):
//   bf16: 2 DOT_SLICEs x (8 A + 4 B) fragments of 8 bf16, slice s from base [s]
//   e4m3: 8 A + 4 B fragments of 32 e4m3, chunk halves from bases [0], [1]
// A fragment i: tile rows 16 i + x; B fragment j: rows 32 (j >> 1) + 4 (j & 1)
// + (x & 3) + 8 (x >> 2) of the wave's 64 (the epilogue's column interleave).
__device__ __forceinline__ constexpr int qa_blk(int i) { return 16 * i * kRowBytes; }
__device__ __forceinline__ constexpr int qb_blk(int j) { return (32 * (j >> 1) + 4 * (j & 1)) * kRowBytes; }

template <int kDtype>
struct Pipe;

template <>
struct Pipe<kBf16> {
    using F = Frag<kBf16>;
    struct Frags {
        bf16x8 a[2][8], b[2][4];
    };
    __device__ __forceinline__ static void read(Frags &f, const char *smem, const int (&ba)[2],
                                                const int (&bb)[2])
    {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f.b[s][j] = *reinterpret_cast<const bf16x8 *>(smem + qb_blk(j) + bb[s]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f.a[s][i] = *reinterpret_cast<const bf16x8 *>(smem + qa_blk(i) + ba[s]);
        }
    }
    __device__ __forceinline__ static void cluster(const Frags &f, f32x4 (&acc)[8][4])
    {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = F::mma(f.b[s][j], f.a[s][i], acc[i][j]);
    }
};

template <>
struct Pipe<kFp8> {
    using F = Frag<kFp8>;
    struct Frags {
        i32x8 a[8], b[4];
    };
    __device__ __forceinline__ static i32x8 frag(const char *smem, int blk, int base0, int base1)
    {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(smem + blk + base0);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(smem + blk + base1);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    __device__ __forceinline__ static void read(Frags &f, const char *smem, const int (&ba)[2],
                                                const int (&bb)[2])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f.b[j] = frag(smem, qb_blk(j), bb[0], bb[1]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            f.a[i] = frag(smem, qa_blk(i), ba[0], ba[1]);
    }
    __device__ __forceinline__ static void cluster(const Frags &f, f32x4 (&acc)[8][4])
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = F::mma(f.b[j], f.a[i], acc[i][j]);
    }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// Write a wave's 128-row sub-tile of kCols / 16 column blocks, whose top-left
// corner is (row_off, col_off) inside the tile: per 16-row block i a lane owns
// output row m = 16 i + (lane % 16) and, per 32-column group h, columns
// 32 h + 8 q .. 32 h + 8 q + 7 (blocks 2 h and 2 h + 1, interleaved as above).
// Tiles inside M x N with N % 8 == 0 use 16-byte stores; edge tiles store
// only rows < M and columns < N (element by element when N % 8 != 0).
// kRB x kCB blocks of 16 x 16 of a kT x kT output tile (tile (tm, tn)), the
// wave's part starting at (row_off, col_off) inside it.
// The fp32 values of output blocks (i, 2h) and (i, 2h + 1), scaled by p.scale
// if kScale (per-tensor e4m3; bf16 and MXFP8 have scale 1 and skip the
// multiply).  kAgpr: the accumulators live in AGPRs; an empty asm keeps each
// pair there until this point, so the epilogue copies 8 values at a time
// into VGPRs instead of all of them at once (which spills).
template <bool kScale, bool kAgpr, int kRB, int kCB>
__device__ __forceinline__ void block_pair(f32x4 (&acc)[kRB][kCB], int i, int h, float sc,
                                           f32x4 &lo, f32x4 &hi)
{
    if (kAgpr)
        asm volatile("" : "+a"(acc[i][2 * h]), "+a"(acc[i][2 * h + 1]));
    lo = kScale ? acc[i][2 * h] * sc : acc[i][2 * h];
    hi = kScale ? acc[i][2 * h + 1] * sc : acc[i][2 * h + 1];
}
// The same for a whole 16-row block i (kCB of 6 or 8 blocks): one pin for
// the row, so that its conversions and stores can overlap.
template <int kRB, int kCB>
__device__ __forceinline__ void pin_row(f32x4 (&acc)[kRB][kCB], int i)
{
    static_assert(kCB == 6 || kCB == 8, "row pin for the AGPR tiles");
    if constexpr (kCB == 8)
        asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                          "+a"(acc[i][4]), "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
    else
        asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                          "+a"(acc[i][4]), "+a"(acc[i][5]));
}

template <int kRB, int kCB, int kT, bool kScale, bool kAgpr>
__device__ __forceinline__ void store_tile(const GemmParams &p, int tm, int tn, int row_off,
                                           int col_off, int lane, f32x4 (&acc)[kRB][kCB])
{
    const int q = lane >> 4;
    const int64_t row0 = (int64_t)tm * kT + row_off + (lane & 15);
    const int64_t col0 = (int64_t)tn * kT + col_off + 8 * q;
    const float sc = p.scale;
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const int64_t ldc = p.ldc;
    const bool vec = ((p.N | p.ldc) & 7) == 0;   // 16-byte stores of 8 columns
    const bool inside = (tm + 1) * kT <= p.M && (tn + 1) * kT <= p.N && vec;
    // Whole tiles without the fp32 copy (every timed launch): one buffer
    // resource over the wave's 16 kRB rows of C, a lane offset fixed for the
    // whole epilogue, a scalar offset per 16-row block and the 32-column group
    // in the instruction's immediate offset -- no per-store address
    // arithmetic and no branches.  The resource's 32-bit range bounds N.
    if (inside && !p.C_f32 && (uint64_t)32 * kRB * (uint64_t)p.ldc < (uint64_t(1) << 32)) {
        const int64_t origin = ((int64_t)tm * kT + row_off) * ldc + (int64_t)tn * kT + col_off;
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(C + origin, (uint32_t)(32 * kRB) * (uint32_t)p.ldc);
        const int voff = ((lane & 15) * p.ldc + 8 * q) * 2;
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
            const int soff = __builtin_amdgcn_readfirstlane((int)((uint32_t)(32 * i) * (uint32_t)p.ldc));
            if constexpr (kAgpr)
                pin_row(acc, i);
#pragma unroll
            for (int h = 0; h < kCB / 2; ++h) {
                f32x4 lo, hi;
                block_pair<kScale, false>(acc, i, h, sc, lo, hi);
                const u32x4 packed = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                      pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
                __builtin_amdgcn_raw_buffer_store_b128(packed, rc, voff + 64 * h, soff, 0);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
        const int64_t m = row0 + 16 * i;
        if (!inside && m >= p.M)
            continue;
#pragma unroll
        for (int h = 0; h < kCB / 2; ++h) {
            f32x4 lo, hi;
            block_pair<kScale, kAgpr>(acc, i, h, sc, lo, hi);
            const int64_t n0 = col0 + 32 * h;
            const int64_t off = m * ldc + n0;
            u32x4 packed = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                            pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
            if (inside || (vec && n0 < p.N)) {
                *reinterpret_cast<u32x4 *>(C + off) = packed;
                if (p.C_f32) {
                    *reinterpret_cast<f32x4 *>(p.C_f32 + off) = lo;
                    *reinterpret_cast<f32x4 *>(p.C_f32 + off + 4) = hi;
                }
            } else if (!vec) {
                const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (n0 + e < p.N) {
                        C[off + e] = (uint16_t)(packed[e >> 1] >> (16 * (e & 1)));
                        if (p.C_f32)
                            p.C_f32[off + e] = v[e];
                    }
                }
            }
        }
    }
}

// Counters for callers that ask for a per-workgroup time record
// (GemmParams::trace): the 100 MHz real-time counter and the shader-clock
// counter.  Workgroup b writes 8 words at trace + 8 b from lane 0 of wave 0:
// real time at entry, at the end of its K loop and after its last store was
// issued; the shader clock at the same three points; the XCC_ID register;
// (tile_m << 32) | tile_n.
struct Stamp {
    uint64_t rt, mt;
};
__device__ __forceinline__ Stamp stamp()
{
    return Stamp{__builtin_amdgcn_s_memrealtime(), __builtin_amdgcn_s_memtime()};
}
__device__ __forceinline__ void write_trace(const GemmParams &p, const Stamp &s0, const Stamp &s1,
                                            int tm, int tn)
{
    if (!p.trace || threadIdx.x != 0)
        return;
    const Stamp s2 = stamp();
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    uint64_t *t = p.trace + 8 * (uint64_t)blockIdx.x;
    t[0] = s0.rt;
    t[1] = s1.rt;
    t[2] = s2.rt;
    t[3] = s0.mt;
    t[4] = s1.mt;
    t[5] = s2.mt;
    t[6] = xcc;
    t[7] = ((uint64_t)(uint32_t)tm << 32) | (uint32_t)tn;
}

template <int kDtype, int kSched>
__global__ __launch_bounds__(512, 1) void gemm_kernel(const GemmParams p)
{
    __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = wave >> 2;     // ping-pong group, also the 128-row half of the tile
    const int wn = wave & 3;     // 64-column quarter of the tile
    const int w4 = wave & 3;
    const Stamp s0 = stamp();

    int tm, tn;
    remap_tile(blockIdx.x, p.Gm, p.Gn, p.W, p.Cc, tm, tn);

    constexpr int kElem = kDtype == kBf16 ? 2 : 1;
    const int kb = p.K * kElem;                           // bytes of K per operand row
    const int pa = p.lda * kElem, pb = p.ldb * kElem;     // row pitches in bytes
    const int rows_a = min(kTile, p.M - tm * kTile);      // valid rows of this tile's panels
    const int rows_b = min(kTile, p.N - tn * kTile);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(
        static_cast<const char *>(p.A) + (int64_t)tm * kTile * pa, panel_bytes(rows_a, pa, kb));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(
        static_cast<const char *>(p.B) + (int64_t)tn * kTile * pb, panel_bytes(rows_b, pb, kb));

    // This lane's source offsets inside a row group: row 8u + lane/8, slot
    // lane%8; row bits 3,4 equal (u & 3) == w4 for every load this wave
    // issues, so one offset per operand serves all its loads.
    const int r8 = lane >> 3;
    const int cb_a = ((lane & 7) ^ slot_xor_a(r8 | (w4 << 3))) << 4;
    const int cb_b = ((lane & 7) ^ slot_xor_b(r8 | (w4 << 3))) << 4;
    // K step k covers row bytes [128 k - shift, +128): a partial step is step
    // 0, whose lanes with a chunk below byte 0 load zeros, and every later
    // step is whole.  Loads of steps >= nk fetch bytes no MFMA uses (in-range
    // bytes of the panel's next rows, or zeros past its last row) into panels
    // no one reads any more.
    const int shift = __builtin_amdgcn_readfirstlane(p.nk * kRowBytes - kb);
    const int va = r8 * pa + cb_a, vb = r8 * pb + cb_b;
    const int va_first = cb_a >= shift ? va - shift : kOutOfRange;
    const int vb_first = cb_b >= shift ? vb - shift : kOutOfRange;
    auto soff = [&](int k) { return k == 0 ? 0 : k * kRowBytes - shift; };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = p.nk;
    // K step k lives in A panel k % 2 and B panel k % 3 (lockstep: k % 2).
    auto a_off = [&](int k) { return (k & 1) * kPanelBytes; };
    auto b_off = [&](int k) { return kBRing + (k % kBPanels) * kPanelBytes; };
    auto b_off2 = [&](int k) { return kBRing + (k & 1) * kPanelBytes; };
    // this wave's 4 of the 8-row groups u = base + w4 + 4 v of a K step's panel.
    // The K step's scalar offset goes through readfirstlane: it is uniform,
    // but the compiler otherwise keeps its per-group strength-reduced copies
    // in vector registers and wraps every e4m3 ping-pong load in a loop over
    // the distinct lane values (about 9 % more cycles per K step).
    auto load_a = [&](int k, int off, int base) {
        dma_panel_part<4>(ra, smem + off, base, w4, k == 0 ? va_first : va,
                          __builtin_amdgcn_readfirstlane(soff(k)), pa);
    };
    auto load_b = [&](int k, int off, int base) {
        dma_panel_part<4>(rb, smem + off, base, w4, k == 0 ? vb_first : vb,
                          __builtin_amdgcn_readfirstlane(soff(k)), pb);
    };

    if (kSched == kLockstep) {
        const LaneOffsets lo = lane_offsets(lane);
        // Each wave loads its 16 of the 64 row groups of a K step.
        if (nk > 0) {
            load_a(0, a_off(0), 16 * g);
            load_b(0, b_off2(0), 16 * g);
        }
        if (nk > 1) {
            load_a(1, a_off(1), 16 * g);
            load_b(1, b_off2(1), 16 * g);
            wait_vmcnt<8>();
        } else {
            wait_vmcnt<0>();
        }
        block_barrier();
        for (int t = 0; t < nk; ++t) {
            compute_kstep<kDtype>(smem + a_off(t) + 128 * g * kRowBytes,
                                  smem + b_off2(t) + 64 * wn * kRowBytes, lo, acc);
            wait_lgkmcnt0();
            block_barrier();                       // every wave is done with K step t
            if (t + 2 < nk) {
                load_a(t + 2, a_off(t), 16 * g);
                load_b(t + 2, b_off2(t), 16 * g);
                wait_vmcnt<8>();                   // K step t+1 has landed
            } else {
                wait_vmcnt<0>();
            }
            block_barrier();                       // K step t+1 visible to all waves
        }
    } else {
        // ---- 8-wave ping-pong ------------------------------------------------
        // Phases alternate between the groups and end at a barrier:
        //   group 0:  c(0) | m(0) | c(1) | m(1) | ...
        //   group 1:  m(-1)| c(0) | m(0) | c(1) | ...
        // c(t) is the MFMA cluster of K step t at s_setprio 3, its fragments
        // already in registers; m(t) issues HBM->LDS loads for later K steps,
        // then reads all fragments of c(t+1) from LDS (they land while the
        // partner's cluster runs; reading first measured 4 % more cycles per
        // K step).  Loads (k = K step, into A panel
        // k % 2 / B panel k % 3), 32 KiB per memory phase for either group:
        //   A rows   0..127 of k: group 0 in m(k-2), awaited at the end of c(k-1)
        //   B rows   0..127 of k: group 0 in m(k-2), awaited at the end of c(k-1)
        //   A rows 128..255 of k: group 1 in m(k-2), awaited at the end of c(k-1)
        //   B rows 128..255 of k: group 1 in m(k-3), awaited at the end of m(k-2)
        // so every panel is complete and published by a barrier before the
        // memory phase that reads its fragments, and no load targets a panel
        // that a phase in flight still reads.  The loop body is the same for
        // every t (loads of steps >= nk are harmless, see above).  Group 1
        // ends after c(nk-1); group 0 skips the barriers after its last
        // cluster, keeping the counts equal.
        using P = Pipe<kDtype>;
        typename P::Frags frags;
        const QuadLane ql = quad_lane(lane);
        const int a_rows = 128 * g * kRowBytes, b_rows = 64 * wn * kRowBytes;
        // fragments of step k: four lane bases (one vector add each), then 24
        // reads of base + immediate
        auto read = [&](int k) {
            const int ao = __builtin_amdgcn_readfirstlane(a_rows + a_off(k));
            const int bo = __builtin_amdgcn_readfirstlane(b_rows + b_off(k));
            const int ba[2] = {opaque(ql.a[0] + ao), opaque(ql.a[1] + ao)};
            const int bb[2] = {opaque(ql.b[0] + bo), opaque(ql.b[1] + bo)};
            P::read(frags, smem, ba, bb);
        };
        auto cluster = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(3);
            P::cluster(frags, acc);
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        };
        if (nk > 0) {   // K step 0: both groups share every panel
            load_a(0, a_off(0), 16 * g);
            load_b(0, b_off(0), 16 * g);
            if (g == 0) {
                load_a(1, a_off(1), 0);
                load_b(1, b_off(1), 0);
                wait_vmcnt<8>();                   // K step 0 landed
            } else {
                load_b(1, b_off(1), 16);
                wait_vmcnt<4>();                   // K step 0 landed
            }
            block_barrier();

            if (g == 0) {
                read(0);
                for (int t = 0; t < nk; ++t) {
                    cluster();
                    wait_lgkmcnt0();
                    if (t == nk - 1)
                        break;
                    wait_vmcnt<0>();               // rows 0..127 of A and B of t+1 landed
                    block_barrier();               // end of c(t)
                    load_a(t + 2, a_off(t + 2), 0);
                    load_b(t + 2, b_off(t + 2), 0);
                    __builtin_amdgcn_sched_barrier(0);
                    read(t + 1);
                    block_barrier();               // end of m(t)
                }
            } else {
                // m(-1)
                load_a(1, a_off(1), 16);
                load_b(2, b_off(2), 16);
                __builtin_amdgcn_sched_barrier(0);
                read(0);
                wait_vmcnt<8>();                   // B rows 128..255 of step 1 landed
                if (nk > 1)
                    block_barrier();               // end of m(-1)
                for (int t = 0; t < nk; ++t) {
                    cluster();
                    wait_lgkmcnt0();
                    if (t == nk - 1)
                        break;
                    wait_vmcnt<4>();               // A rows 128..255 of t+1 landed
                    block_barrier();               // end of c(t)
                    load_a(t + 2, a_off(t + 2), 16);
                    load_b(t + 3, b_off(t + 3), 16);
                    __builtin_amdgcn_sched_barrier(0);
                    read(t + 1);
                    wait_vmcnt<8>();               // B rows 128..255 of step t+2 landed
                    if (t != nk - 2)
                        block_barrier();           // end of m(t)
                }
            }
        }
    }
    wait_vmcnt<0>();                               // no load still writes LDS at exit
    const Stamp s1 = stamp();
    store_tile<8, 4, kTile, kDtype == kFp8, false>(p, tm, tn, 128 * g, 64 * wn, lane, acc);
    write_trace(p, s0, s1, tm, tn);
}

// ---- 4-wave interleave (one wave per SIMD) --------------------------------
// HipKittens L2 note, section 2 (Q2, Pillar 2), section 4 ("% peak
// derivation", FP8 line) and section 5 (GEMM, Figure 6 right), and the
// summary page's "4-wave interleave": each wave issues its own loads and LDS
// reads between its MFMAs.  Wave w owns the
// 128 x 128 quarter (wm, wn) = (w >> 1, w & 1) of the tile: 8 x 8 blocks of
// 16 x 16, i.e. 256 fp32 accumulators per lane, which fit next to the
// fragments only because a single wave per SIMD has the whole register file.
// Per K step a wave reads 16 fragments of 128 rows of A and B each, a third
// fewer LDS bytes per CU than the 8-wave split (8 x 4 blocks per wave).
//
// A K step is two halves of MFMAs with one barrier between them; all four
// waves run the same program:
//   half 0 of step t: the first half of the MFMAs; the loads of B(t+2) into
//                     B panel (t+2) % 3; fragment reads that complete step t
//   barrier:          every wave waited for its own loads of step t+1 and
//                     has its reads of A panel t % 2 back in registers
//   half 1 of step t: the second half of the MFMAs; the loads of A(t+2) into
//                     A panel t % 2; fragment reads that begin step t+1
// Each memory instruction is slotted after a given MFMA (sched_barrier after
// every slot), so the matrix core is fed by one MFMA after another while the
// loads and reads issue in its shadow.  The loop body is the same for every
// t: the loads of K steps >= nk fetch bytes no MFMA uses -- in-range bytes of
// the panel's next rows, or zeros past the panel's last row -- into panels no
// one reads any more, and the reads of "step nk" in the last half are unused.
// MXFP8 scales of one K step for one lane l: byte e of a[e >> 2] is the E8M0
// scale of A fragment e's row for lane l and k block 4 t + l / 16 (the block
// the MFMA scales with lane group l / 16's value), b likewise for B fragment
// e.  Unused by the other dtypes.
struct MxScales {
    uint32_t a[2], b[2];
};

// v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands: the scale byte
// (chosen by op_sel) of lane group b multiplies the products of k block b of
// that lane's row (probed on gfx950); the first scale goes with the first
// operand.  op_sel must be a constant: the switch
// folds away once the caller's block indices are unrolled.
template <int kOx, int kOy>
__device__ __forceinline__ f32x4 mma_mx_c(const i32x8 &x, const i32x8 &y, const f32x4 &c,
                                          uint32_t sx, uint32_t sy)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, kOx, (int)sx, kOy,
                                                            (int)sy);
}
__device__ __forceinline__ f32x4 mma_mx(const i32x8 &x, const i32x8 &y, const f32x4 &c,
                                        uint32_t sx, uint32_t sy, int ox, int oy)
{
    switch (ox * 4 + oy) {
    case 0: return mma_mx_c<0, 0>(x, y, c, sx, sy);
    case 1: return mma_mx_c<0, 1>(x, y, c, sx, sy);
    case 2: return mma_mx_c<0, 2>(x, y, c, sx, sy);
    case 3: return mma_mx_c<0, 3>(x, y, c, sx, sy);
    case 4: return mma_mx_c<1, 0>(x, y, c, sx, sy);
    case 5: return mma_mx_c<1, 1>(x, y, c, sx, sy);
    case 6: return mma_mx_c<1, 2>(x, y, c, sx, sy);
    case 7: return mma_mx_c<1, 3>(x, y, c, sx, sy);
    case 8: return mma_mx_c<2, 0>(x, y, c, sx, sy);
    case 9: return mma_mx_c<2, 1>(x, y, c, sx, sy);
    case 10: return mma_mx_c<2, 2>(x, y, c, sx, sy);
    case 11: return mma_mx_c<2, 3>(x, y, c, sx, sy);
    case 12: return mma_mx_c<3, 0>(x, y, c, sx, sy);
    case 13: return mma_mx_c<3, 1>(x, y, c, sx, sy);
    case 14: return mma_mx_c<3, 2>(x, y, c, sx, sy);
    default: return mma_mx_c<3, 3>(x, y, c, sx, sy);
    }
}


// The accumulators leave the K loop in the accumulation registers (AGPRs),
// whatever the epilogue does with them: without this, how the epilogue reads
// them feeds back into the loop's register assignment, and the allocator
// then moves accumulators between AGPRs and VGPRs inside the loop.
template <int kR, int kC>
__device__ __forceinline__ void pin_acc(f32x4 (&acc)[kR][kC])
{
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int j = 0; j < kC; ++j)
            asm volatile("" : "+a"(acc[i][j]));
}

// Scalar counterparts.  Instruction selection orders a whole K step (one
// basic block) as a single graph, so plain arithmetic drifts away from the
// MFMA slot it is written in and bunches up; bunched, it delays the next
// MFMA (one wave per SIMD issues only a few other instructions for free in
// an MFMA's shadow).  Arithmetic whose inputs come out of pin_s() and whose
// result goes into pin_s() in one slot stays in that slot.
__device__ __forceinline__ int pin_s(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}
// A copy into a fresh register, issued here: a loop-carried value is then
// rotated in a chosen slot rather than by copies at the loop's back edge.
__device__ __forceinline__ int mov_s(int x)
{
    int y;
    asm volatile("s_mov_b32 %0, %1" : "=s"(y) : "s"(x));
    return y;
}
__device__ __forceinline__ uint32_t mov_v(uint32_t x)
{
    uint32_t y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

// f(std::integral_constant<int, n>) for n = 0 .. kN-1, in order: a slot loop
// whose slot number is a constant in the body without relying on the unroller
// (a long body exceeds its full-unroll threshold, and a run-time slot number
// would index the accumulators dynamically).
template <class F, int... kN>
__device__ __forceinline__ void for_slots_seq(F &&f, std::integer_sequence<int, kN...>)
{
    (f(std::integral_constant<int, kN>{}), ...);
}
template <int kN, class F>
__device__ __forceinline__ void for_slots(F &&f)
{
    for_slots_seq(f, std::make_integer_sequence<int, kN>{});
}

// One wave-wide HBM->LDS load of 8 panel rows into LDS byte ring_off +
// fixed_off + u * 1 KiB, K step offset soff_kstep, row group u (callers pin
// ring_off and soff_kstep so that the address arithmetic stays at the call).
__device__ __forceinline__ void dma_rows_at(__amdgpu_buffer_rsrc_t rs, char *smem, int ring_off,
                                            int fixed_off, int u, int voff, int soff_kstep,
                                            int pitch)
{
    const int m = ring_off + fixed_off + u * kDmaBytes;
    const int so = soff_kstep + u * kDmaRows * pitch;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(smem + m), 16, voff, so, 0, 0);
}

// LDS lane bases of one half's fragment reads (opaque, see above): A and B,
// one per 16-byte chunk h of a fragment (bf16 fragments use h = 0 only).
struct Bases {
    int a[2], b[2];
};

// kB: 16 x 16 blocks per side of a wave's quarter of the tile -- 8 for the
// 256 x 256 tile (a 128 x 128 quarter), 4 for the 128 x 128 tile.
template <int kDtype, int kB>
struct Quad;

template <int kB>
struct Quad<kBf16, kB> {
    // half h runs DOT_SLICE h of all kB x kB blocks (i-major); half 0 reads
    // slice 1 of step t, half 1 reads slice 0 of step t+1 (B fragments
    // first, then A fragments: the order the next half's MFMAs need them).
    using F = Frag<kBf16>;
    struct Frags {
        bf16x8 a[2][kB], b[2][kB];   // [slice][block]
    };
    static constexpr int kBlk = kB;
    static constexpr int kMfmas = kB * kB;   // per half
    // The MFMA after which load v (0..kB-1) of half h / fragment read r
    // (0..2kB-1) issues.  kB = 8: half 1's A loads go early (their panel is
    // free once the barrier has passed), which leaves them 85 MFMAs to land
    // before the next barrier waits for them, against 68 when spread like
    // the B loads.  kB = 6 (36 MFMAs a half) and kB = 4 (16): reads on even
    // gaps, loads on odd ones, A loads again early.
    __device__ static constexpr int dma_slot(int h, int v)
    {
        return kB == 8   ? (h == 0 ? 8 * v + 4 : 6 * v + 1)
               : kB == 6 ? (h == 0 ? 6 * v + 3 : 4 * v + 1)
                         : (h == 0 ? 4 * v + 1 : 2 * v + 1);
    }
    __device__ static constexpr int read_slot(int r) { return kB == 8 ? 3 * r : 2 * r; }
    // gaps (no load there) for the step's bookkeeping: the next half's A and
    // B lane bases (late, so that fragments have died to make room), the
    // three B-ring moves, and the A ring / K offset update after the half's
    // last load
    // (base_slot(h, w): half h forms lane base w = A, -, B, - ; -1 = none)
    __device__ static constexpr int base_slot(int h, int w)
    {
        return kB == 8   ? (w == 0 ? 50 : w == 2 ? 53 : -1)
               : kB == 6 ? (w == 0 ? 24 : w == 2 ? 26 : -1)
                         : (w == 0 ? (h == 0 ? 7 : 9) : w == 2 ? 11 : -1);
    }
    __device__ static constexpr int rot_slot(int i)
    {
        return kB == 8 ? 55 + i : kB == 6 ? 28 + i : 12 + i;
    }
    static constexpr int kSlotTail = kB == 8 ? 61 : kB == 6 ? 34 : 15;

    // lane base w of half kH's reads: slice 1 - kH of the panel at off
    template <int kH, int kW>
    __device__ __forceinline__ static void base(Bases &bs, const QuadLane &l, int off)
    {
        if constexpr (kW == 0)
            bs.a[0] = opaque(l.a[1 - kH] + off);
        if constexpr (kW == 2)
            bs.b[0] = opaque(l.b[1 - kH] + off);
    }

    __device__ __forceinline__ static void read_first(Frags &f, const char *smem,
                                                      const QuadLane &l, int a_off, int b_off)
    {
        const int ba = opaque(l.a[0] + a_off), bb = opaque(l.b[0] + b_off);
#pragma unroll
        for (int j = 0; j < kB; ++j)
            f.b[0][j] = *reinterpret_cast<const bf16x8 *>(smem + qb_blk(j) + bb);
#pragma unroll
        for (int i = 0; i < kB; ++i)
            f.a[0][i] = *reinterpret_cast<const bf16x8 *>(smem + qa_blk(i) + ba);
    }
    // bs: this half's read bases; dma(v) issues the half's load v; hook(n)
    // runs after MFMA n (the caller's per-slot work).
    template <int kH, class Dma, class Hook>
    __device__ __forceinline__ static void half(Frags &f, f32x4 (&acc)[kB][kB], const char *smem,
                                                const Bases &bs, const MxScales &, Dma &&dma,
                                                Hook &&hook)
    {
        constexpr int s = 1 - kH;
        const int ba = bs.a[0], bb = bs.b[0];
        for_slots<kMfmas>([&](auto slot) __attribute__((always_inline)) {
            constexpr int n = decltype(slot)::value;
            constexpr int i = n / kB, j = n % kB;
            acc[i][j] = F::mma(f.b[kH][j], f.a[kH][i], acc[i][j]);
#pragma unroll
            for (int v = 0; v < kB; ++v)
                if (dma_slot(kH, v) == n)
                    dma(v);
#pragma unroll
            for (int r = 0; r < 2 * kB; ++r) {
                if (read_slot(r) != n)
                    continue;
                if (r < kB)
                    f.b[s][r] = *reinterpret_cast<const bf16x8 *>(smem + qb_blk(r) + bb);
                else
                    f.a[s][r - kB] = *reinterpret_cast<const bf16x8 *>(smem + qa_blk(r - kB) + ba);
            }
            hook(slot);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
};

template <bool kMxScaled, int kB>
struct QuadF8 {
    // e4m3 with per-tensor scales (kMxScaled false) or MXFP8 block scales.
    // half 0 runs blocks (i, j < kB/2), half 1 blocks (i, j >= kB/2), both
    // i-major.  Half 0 reads the B fragments of its second half of step t;
    // half 1 reads the first B fragments of step t+1 and A fragment i of
    // step t+1 right after the last MFMA that uses A fragment i of step t,
    // so one K step of fragments is all a wave holds.  A fragment is two
    // 16-byte chunks (halves h = 0, 1).
    using F = Frag<kFp8>;
    struct Frags {
        i32x8 a[kB], b[kB];
    };
    static constexpr int kBlk = kB;
    static constexpr int kHalfCols = kB / 2;
    static constexpr int kMfmas = kB * kHalfCols;   // per half
    // kB = 4 (8 MFMAs a half, each 32 cycles): half 1 loads on even gaps so
    // that its tail gap (7) follows the last one.  kB = 6 (18 MFMAs a half):
    // loads after MFMA 3 v + 1, reads and A-fragment reads after 3 r + 2.
    __device__ static constexpr int dma_slot(int h, int v)
    {
        return kB == 8 ? 4 * v + 1 : kB == 6 ? 3 * v + 1 : (h == 0 ? 2 * v + 1 : 2 * v);
    }
    // B fragment kB/2 + r (half 0) or r (half 1)
    __device__ static constexpr int b_read_slot(int h, int r)
    {
        return h == 0 ? (kB == 6 ? 3 * r + 2 : 4 * r + 2) : r;
    }
    // bookkeeping gaps, as for bf16 (kB = 8: no load or read there in either
    // half; lane bases w = A chunk 0, A chunk 1, B chunk 0, B chunk 1; no slot
    // just before a load slot, whose address arithmetic tends to move up a gap)
    __device__ static constexpr int base_slot(int h, int w)
    {
        return kB == 8   ? (h == 0 ? 18 : 6) + 4 * w
               : kB == 6 ? (h == 0 ? (w < 2 ? 11 + 3 * w : 17) : 3 + 3 * w)
                         : (h == 0 ? 2 * w : (w < 2 ? -1 : 2 * w - 1));
    }
    __device__ static constexpr int rot_slot(int i)
    {
        return kB == 8 ? 20 + 4 * i : kB == 6 ? (i < 2 ? 3 + 3 * i : 15) : 2 + 2 * i;
    }
    static constexpr int kSlotTail = kB == 8 ? 30 : kB == 6 ? 17 : 7;
    // MXFP8 only: half 0 forms step t+2's masked A load offset after MFMA
    // kSlotMaskA; half 1 forms step t+3's B offset after MFMA kSlotMaskB and
    // (kB = 8) moves the next scales of B blocks 0..3 (last used in half 0)
    // and A blocks 0..3 (last used by MFMA 15) into fresh registers after
    // MFMA 8 and 16.  kB = 4 uses one 32-bit scale word per operand, needed
    // by every MFMA of the step.
    static constexpr int kSlotMaskA = kB == 8 ? 23 : 4, kSlotMaskB = kB == 8 ? 12 : 2;
    static constexpr int kSlotScaleB = 8, kSlotScaleA = 16;

    // lane base w of half kH's reads at panel offset off (half 0 reads B only)
    template <int kH, int kW>
    __device__ __forceinline__ static void base(Bases &bs, const QuadLane &l, int off)
    {
        if constexpr (kW < 2) {
            if constexpr (kH == 1)
                bs.a[kW] = opaque(l.a[kW] + off);
        } else {
            bs.b[kW - 2] = opaque(l.b[kW - 2] + off);
        }
    }

    __device__ __forceinline__ static i32x8 frag(const char *smem, int blk, int base0, int base1)
    {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(smem + blk + base0);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(smem + blk + base1);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    __device__ __forceinline__ static void read_first(Frags &f, const char *smem,
                                                      const QuadLane &l, int a_off, int b_off)
    {
        const int ba0 = opaque(l.a[0] + a_off), ba1 = opaque(l.a[1] + a_off);
        const int bb0 = opaque(l.b[0] + b_off), bb1 = opaque(l.b[1] + b_off);
#pragma unroll
        for (int j = 0; j < kHalfCols; ++j)
            f.b[j] = frag(smem, qb_blk(j), bb0, bb1);
#pragma unroll
        for (int i = 0; i < kB; ++i)
            f.a[i] = frag(smem, qa_blk(i), ba0, ba1);
    }
    template <int kH, class Dma, class Hook>
    __device__ __forceinline__ static void half(Frags &f, f32x4 (&acc)[kB][kB], const char *smem,
                                                const Bases &bs, const MxScales &sc, Dma &&dma,
                                                Hook &&hook)
    {
        const int ba0 = bs.a[0], ba1 = bs.a[1], bb0 = bs.b[0], bb1 = bs.b[1];
        for_slots<kMfmas>([&](auto slot) __attribute__((always_inline)) {
            constexpr int n = decltype(slot)::value;
            constexpr int i = n / kHalfCols, j = kHalfCols * kH + n % kHalfCols;
            if (kMxScaled)
                acc[i][j] = mma_mx(f.b[j], f.a[i], acc[i][j], sc.b[j >> 2], sc.a[i >> 2], j & 3,
                                   i & 3);
            else
                acc[i][j] = F::mma(f.b[j], f.a[i], acc[i][j]);
#pragma unroll
            for (int v = 0; v < kB; ++v)
                if (dma_slot(kH, v) == n)
                    dma(v);
#pragma unroll
            for (int r = 0; r < kHalfCols; ++r) {
                if (b_read_slot(kH, r) != n)
                    continue;
                const int jb = kHalfCols * (1 - kH) + r;
                f.b[jb] = frag(smem, qb_blk(jb), bb0, bb1);
            }
            if (kH == 1 && n % kHalfCols == kHalfCols - 1)
                f.a[i] = frag(smem, qa_blk(i), ba0, ba1);
            hook(slot);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
};

template <int kB>
struct Quad<kFp8, kB> : QuadF8<false, kB> {
};
template <int kB>
struct Quad<kMx, kB> : QuadF8<true, kB> {
};

// Every memory instruction and bookkeeping slot of a half has an MFMA to
// follow, and the tail (A ring / K offset update) comes after the half's
// last load (the loads read the values it replaces).
template <class Q>
constexpr bool slots_ok()
{
    bool ok = Q::kSlotTail > Q::dma_slot(1, Q::kBlk - 1) && Q::kSlotTail < Q::kMfmas;
    for (int h = 0; h < 2; ++h)
        for (int v = 0; v < Q::kBlk; ++v)
            ok = ok && Q::dma_slot(h, v) < Q::kMfmas;
    for (int h = 0; h < 2; ++h)
        for (int w = 0; w < 4; ++w)
            ok = ok && Q::base_slot(h, w) < Q::kMfmas;
    for (int i = 0; i < 3; ++i)
        ok = ok && Q::rot_slot(i) < Q::kMfmas;
    return ok;
}
static_assert(slots_ok<Quad<kBf16, 8>>() && slots_ok<Quad<kBf16, 6>>() &&
                  slots_ok<Quad<kBf16, 4>>(),
              "bf16 slot plans");
static_assert(slots_ok<Quad<kFp8, 8>>() && slots_ok<Quad<kFp8, 6>>() &&
                  slots_ok<Quad<kFp8, 4>>(),
              "e4m3 slot plans");
static_assert(Quad<kBf16, 8>::read_slot(15) < 64 && Quad<kBf16, 6>::read_slot(11) < 36 &&
                  Quad<kBf16, 4>::read_slot(7) < 16 &&
                  Quad<kFp8, 8>::b_read_slot(0, 3) < 32 && Quad<kFp8, 6>::b_read_slot(0, 2) < 18 &&
                  Quad<kFp8, 4>::b_read_slot(0, 1) < 8,
              "read slots");

// What the 4-wave loop of one workgroup works on.
struct QuadCtx {
    __amdgpu_buffer_rsrc_t ra, rb;   // this tile's A and B rows
    char *smem;
    int wave;                        // 0..3, also the row group phase of its loads
    int a_rows, b_rows;              // LDS bytes of the wave's rows in an A / B panel 0
    int voff_a, voff_b;              // lane's load offsets (swizzled chunk of its row)
    int cb_a, cb_b;                  // byte of that chunk inside a K step
    int shift;                       // K step k covers row bytes [128 k - shift, +128)
    int pitch_a, pitch_b;            // row pitches of A and B in bytes
    QuadLane l;
    // MXFP8 only: the packed scales (hkg_mx_pack_scales layout) and the byte
    // offsets of this wave's 128-row groups in them at K step 0
    __amdgpu_buffer_rsrc_t rsa, rsb;
    int sa_group, sb_group;
    int s_off_a, s_off_b;            // lane's byte in a K step's 512 scale bytes
};

// MXFP8: this lane's scales of K step k (kB = 8: the lane's 8 bytes per
// operand; kB = 4: the 4 of them that the wave's 64-row quarter of the
// 128-row group uses; steps past the end read other groups' or out-of-range
// bytes and are never used).
template <int kB>
__device__ __forceinline__ MxScales mx_load_scales(const QuadCtx &c, int k)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int so = __builtin_amdgcn_readfirstlane(k * 512);
    if constexpr (kB == 8) {
        const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(c.rsa, c.s_off_a, c.sa_group + so, 0);
        const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(c.rsb, c.s_off_b, c.sb_group + so, 0);
        return MxScales{{a[0], a[1]}, {b[0], b[1]}};
    } else {
        const uint32_t a = __builtin_amdgcn_raw_buffer_load_b32(c.rsa, c.s_off_a, c.sa_group + so, 0);
        const uint32_t b = __builtin_amdgcn_raw_buffer_load_b32(c.rsb, c.s_off_b, c.sb_group + so, 0);
        return MxScales{{a, 0u}, {b, 0u}};
    }
}

// LDS byte offsets of the panels step t uses: A panel of step t (step t+1
// has the other one), B panels of steps t, t+1 and t+2 (being loaded); and
// the scalar K offset of step t+2's loads.  Carried from step to step.
struct Ring {
    int pa, pb, pb1, pb2, so;
    // MXFP8 only: byte offsets of step t+1's packed scales (A, B), row bytes
    // left from step t+2's start, and step t+2's masked B load offset
    int ma, mb, rem, vb;
};

// K step t: the loads it issues are of step t+2.
// kMasked (MXFP8): step t+2 may be a partial or absent one, and lanes whose
// chunk lies past K load zeros.  Otherwise the partial step (if any) is step
// 0, loaded before the loop (c.shift), so every step the loop loads is
// either whole or absent; an absent one's loads fill a panel no MFMA reads
// (reads past the tile's rows return zeros, as for any out-of-range offset).
// MXFP8: sc holds the scales of step t on entry and of step t+1 on exit (the
// load is issued first, so the barrier's vmcnt wait also covers it).
// bs0 holds the bases of half 0 of step t on entry and of step t+1 on exit.
// All of the step's bookkeeping (next bases, ring rotation, K offset) is
// issued in fixed MFMA gaps of the halves, none of it at the loop's head or
// back edge.
template <int kDtype, bool kMasked, int kB>
__device__ __forceinline__ void quad_step(typename Quad<kDtype, kB>::Frags &f,
                                          f32x4 (&acc)[kB][kB], MxScales &sc, const QuadCtx &c,
                                          int t, int lane, Ring &rg, Bases &bs0)
{
    using Q = Quad<kDtype, kB>;
    constexpr int kP = 32 * kB * kRowBytes;   // panel bytes (32 kB rows)
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    // Each ring value is threaded through one chain of pins in program
    // order (every pin is then its value's last use, so none needs a copy).
    int pa = rg.pa, pb1 = rg.pb1, pb2 = rg.pb2, so = rg.so;
    int ma = rg.ma, mb = rg.mb, rem = rg.rem;
    // MXFP8: step t+1's scales, loaded first (the barrier's vmcnt wait then
    // covers them); the masked load offsets of step t+2 (va: formed in half
    // 0; vb: carried from the previous step)
    u32x2 next_a = {0u, 0u}, next_b = {0u, 0u};
    if constexpr (kDtype == kMx) {
        ma = pin_s(ma);
        mb = pin_s(mb);
        if constexpr (kB == 8) {
            next_a = __builtin_amdgcn_raw_buffer_load_b64(c.rsa, c.s_off_a, ma, 0);
            next_b = __builtin_amdgcn_raw_buffer_load_b64(c.rsb, c.s_off_b, mb, 0);
        } else {
            next_a[0] = __builtin_amdgcn_raw_buffer_load_b32(c.rsa, c.s_off_a, ma, 0);
            next_b[0] = __builtin_amdgcn_raw_buffer_load_b32(c.rsb, c.s_off_b, mb, 0);
        }
    }
    int va = c.voff_a;
    const int vb = kMasked ? rg.vb : c.voff_b;
    uint32_t nsc_a0 = 0u, nsc_b0 = 0u;
    // lane base w of the half reading slice 0 (half 1) or 1 (next step's
    // half 0) of step t+1: A panel pa ^ kP, B panel pb1
    auto next_base = [&](Bases &bs, auto kh, auto w) __attribute__((always_inline)) {
        constexpr int kW = decltype(w)::value;
        if constexpr (kW < 2) {
            pa = pin_s(pa);
            Q::template base<decltype(kh)::value, kW>(bs, c.l, pin_s(c.a_rows + (pa ^ kP)));
        } else {
            pb1 = pin_s(pb1);
            Q::template base<decltype(kh)::value, kW>(bs, c.l, pin_s(c.b_rows + pb1));
        }
    };
    // (kh: the half whose bases these are; the running half is the other one)
    auto bases_at = [&](Bases &bs, auto kh, auto slot) __attribute__((always_inline)) {
        constexpr int n = decltype(slot)::value;
        if constexpr (n == Q::base_slot(1 - decltype(kh)::value, 0))
            next_base(bs, kh, std::integral_constant<int, 0>{});
        if constexpr (n == Q::base_slot(1 - decltype(kh)::value, 1))
            next_base(bs, kh, std::integral_constant<int, 1>{});
        if constexpr (n == Q::base_slot(1 - decltype(kh)::value, 2))
            next_base(bs, kh, std::integral_constant<int, 2>{});
        if constexpr (n == Q::base_slot(1 - decltype(kh)::value, 3))
            next_base(bs, kh, std::integral_constant<int, 3>{});
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    Bases bs1;
    Ring nr;
    __builtin_amdgcn_sched_barrier(0);
    Q::template half<0>(
        f, acc, c.smem, bs0, sc,
        [&](int v) {
            pb2 = pin_s(pb2);
            so = pin_s(so);
            dma_rows_at(c.rb, c.smem, pb2, 2 * kP, c.wave + 4 * v, vb, so, c.pitch_b);
        },
        [&](auto slot) __attribute__((always_inline)) {
            bases_at(bs1, H1{}, slot);
            if constexpr (kMasked) {
                if constexpr (decltype(slot)::value == Q::kSlotMaskA) {
                    rem = pin_s(rem);
                    va = opaque(c.cb_a < rem ? c.voff_a : kOutOfRange);
                }
            }
        });
    wait_lgkmcnt0();
    wait_vmcnt<kB>();                              // step t+1 landed (B(t+2) in flight)
    block_barrier();
    Q::template half<1>(
        f, acc, c.smem, bs1, sc,
        [&](int v) {
            pa = pin_s(pa);
            so = pin_s(so);
            dma_rows_at(c.ra, c.smem, pa, 0, c.wave + 4 * v, va, so, c.pitch_a);
        },
        [&](auto slot) __attribute__((always_inline)) {
            constexpr int n = decltype(slot)::value;
            bases_at(bs0, H0{}, slot);
            if constexpr (n == Q::rot_slot(0))
                nr.pb = mov_s(pb1);
            if constexpr (n == Q::rot_slot(1))
                nr.pb1 = mov_s(pb2);
            if constexpr (n == Q::rot_slot(2))
                nr.pb2 = mov_s(rg.pb);
            if constexpr (n == Q::kSlotTail) {
                nr.pa = pin_s(pin_s(pa) ^ kP);
                nr.so = pin_s(pin_s(so) + kRowBytes);
            }
            if constexpr (kMasked) {
                if constexpr (n == Q::kSlotMaskB) {
                    rem = pin_s(rem);
                    nr.vb = opaque(c.cb_b < pin_s(rem - kRowBytes) ? c.voff_b : kOutOfRange);
                }
                if constexpr (kB == 8 && n == Q::kSlotScaleB)
                    nsc_b0 = mov_v(next_b[0]);
                if constexpr (kB == 8 && n == Q::kSlotScaleA)
                    nsc_a0 = mov_v(next_a[0]);
                if constexpr (n == Q::kSlotTail) {
                    nr.rem = pin_s(pin_s(rem) - kRowBytes);
                    nr.ma = pin_s(pin_s(ma) + 512);
                    nr.mb = pin_s(pin_s(mb) + 512);
                }
            }
        });
    rg = nr;
    if constexpr (kDtype == kMx && kB == 8)
        sc = MxScales{{nsc_a0, next_a[1]}, {nsc_b0, next_b[1]}};
    if constexpr (kDtype == kMx && kB == 4)
        sc = MxScales{{next_a[0], 0u}, {next_b[0], 0u}};
}

// kT: output tile edge, 256 (one workgroup per CU, the 160 KiB LDS ring) or
// 128 (a quarter of the work per tile and an 80 KiB ring, so that two
// workgroups can share a CU: for grids with too few 256 x 256 tiles to fill
// the chip).  The wave layout, swizzles, schedule and K order are the same;
// each wave owns a (kT/2) x (kT/2) quarter, kB = kT/32 blocks a side.
template <int kDtype, int kT>
__global__ __launch_bounds__(256, kT == 128 ? 2 : 1) void gemm4_kernel(const GemmParams p)
{
    constexpr int kB = kT / 32;
    constexpr int kP = kT * kRowBytes;   // one panel: kT rows x one K step
    constexpr int kRing = 2 * kP;        // B ring after the 2 A panels
    __shared__ __attribute__((aligned(1024))) char smem[5 * kP];

    const int lane = threadIdx.x & 63;
    QuadCtx c;
    c.smem = smem;
    c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.a_rows = (kT / 2) * (c.wave >> 1) * kRowBytes;           // tile rows kT/2 (w >> 1) ..
    c.b_rows = kRing + (kT / 2) * (c.wave & 1) * kRowBytes;    // tile columns kT/2 (w & 1) ..
    const Stamp s0 = stamp();

    int tm, tn;
    remap_tile(blockIdx.x, p.Gm, p.Gn, p.W, p.Cc, tm, tn);

    constexpr int kElem = kDtype == kBf16 ? 2 : 1;
    const int kb = p.K * kElem;   // bytes of K per operand row
    c.pitch_a = p.lda * kElem;
    c.pitch_b = p.ldb * kElem;
    const int rows_a = min(kT, p.M - tm * kT);
    const int rows_b = min(kT, p.N - tn * kT);
    c.ra = make_rsrc(static_cast<const char *>(p.A) + (int64_t)tm * kT * c.pitch_a,
                     panel_bytes(rows_a, c.pitch_a, kb));
    c.rb = make_rsrc(static_cast<const char *>(p.B) + (int64_t)tn * kT * c.pitch_b,
                     panel_bytes(rows_b, c.pitch_b, kb));

    // Each wave loads row groups u = wave + 4 v (v < kB) of every panel, so
    // row bits 3,4 equal the wave index for all its loads.
    const int r8 = lane >> 3;
    c.cb_a = ((lane & 7) ^ slot_xor_a(r8 | (c.wave << 3))) << 4;
    c.cb_b = ((lane & 7) ^ slot_xor_b(r8 | (c.wave << 3))) << 4;
    c.voff_a = r8 * c.pitch_a + c.cb_a;
    c.voff_b = r8 * c.pitch_b + c.cb_b;
    c.l = quad_lane(lane);
    // MXFP8's scales are packed per whole K step, so it keeps a partial step
    // last (masked); the others take it first.
    constexpr bool kMasked = kDtype == kMx;
    c.shift = kMasked ? 0 : __builtin_amdgcn_readfirstlane(p.nk * kRowBytes - kb);
    MxScales sc = {{0u, 0u}, {0u, 0u}};
    if constexpr (kDtype == kMx) {
        // Each 128-row group holds nk K steps of 64 lanes x 8 bytes.  256 x 256
        // tiles: the wave's 128-row quarter is group 2 tm + (w >> 1) of A and
        // 2 tn + (w & 1) of B.  128 x 128 tiles: the tile is group tm of A
        // and tn of B, and the wave's 64-row half of it is bytes 0..3 or 4..7
        // of each lane's 8 (fragment rows 16 e + x of A, 32 (e >> 1) + ... of
        // B lie in rows 0..63 for e < 4).
        c.rsa = make_rsrc(p.SA, p.sa_bytes);
        c.rsb = make_rsrc(p.SB, p.sb_bytes);
        const int ga = kT == 256 ? 2 * tm + (c.wave >> 1) : tm;
        const int gb = kT == 256 ? 2 * tn + (c.wave & 1) : tn;
        c.sa_group = __builtin_amdgcn_readfirstlane(ga * p.nk * 512);
        c.sb_group = __builtin_amdgcn_readfirstlane(gb * p.nk * 512);
        c.s_off_a = lane * 8 + (kT == 256 ? 0 : 4 * (c.wave >> 1));
        c.s_off_b = lane * 8 + (kT == 256 ? 0 : 4 * (c.wave & 1));
    }

    f32x4 acc[kB][kB];
#pragma unroll
    for (int i = 0; i < kB; ++i)
#pragma unroll
        for (int j = 0; j < kB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    using Q = Quad<kDtype, kB>;
    const int nk = p.nk;
    if (nk > 0) {
        if constexpr (kDtype == kMx)
            sc = mx_load_scales<kB>(c, 0);         // issued first: covered by the wait below
        // K steps 0 and 1.  Masked: either may be partial or (step 1, for
        // nk == 1) absent, and lanes past K load zeros.  Otherwise step 0
        // covers row bytes [-shift, 128 - shift): lanes whose chunk starts
        // below 0 load zeros, the rest read `shift` bytes earlier; step 1 is
        // whole, or absent for nk == 1 (then no MFMA reads its panel).
        int va0, vb0;
        if constexpr (kMasked) {
            va0 = kstep_voff(c.voff_a, c.cb_a, 0, kb);
            vb0 = kstep_voff(c.voff_b, c.cb_b, 0, kb);
        } else {
            va0 = c.cb_a >= c.shift ? c.voff_a - c.shift : kOutOfRange;
            vb0 = c.cb_b >= c.shift ? c.voff_b - c.shift : kOutOfRange;
        }
        const int va1 = kMasked ? kstep_voff(c.voff_a, c.cb_a, 1, kb) : c.voff_a;
        const int vb1 = kMasked ? kstep_voff(c.voff_b, c.cb_b, 1, kb) : c.voff_b;
        const int so1 = kRowBytes - c.shift;
        dma_panel_part<kB>(c.ra, smem, 0, c.wave, va0, 0, c.pitch_a);
        dma_panel_part<kB>(c.rb, smem + kRing, 0, c.wave, vb0, 0, c.pitch_b);
        dma_panel_part<kB>(c.ra, smem + kP, 0, c.wave, va1, so1, c.pitch_a);
        dma_panel_part<kB>(c.rb, smem + kRing + kP, 0, c.wave, vb1, so1, c.pitch_b);
        wait_vmcnt<2 * kB>();                      // step 0 landed
        block_barrier();
        typename Q::Frags f;
        Q::read_first(f, smem, c.l, c.a_rows, c.b_rows);
        Ring rg = {0, 0, kP, 2 * kP, 2 * kRowBytes - c.shift, 0, 0, 0, 0};
        if constexpr (kMasked) {
            rg.ma = c.sa_group + 512;
            rg.mb = c.sb_group + 512;
            rg.rem = kb - 2 * kRowBytes;
            rg.vb = kstep_voff(c.voff_b, c.cb_b, 2, kb);
        }
        Bases bs0 = {{0, 0}, {0, 0}};
        Q::template base<0, 0>(bs0, c.l, c.a_rows);
        Q::template base<0, 1>(bs0, c.l, c.a_rows);
        Q::template base<0, 2>(bs0, c.l, c.b_rows);
        Q::template base<0, 3>(bs0, c.l, c.b_rows);
        for (int t = 0; t < nk; ++t)
            quad_step<kDtype, kMasked, kB>(f, acc, sc, c, t, lane, rg, bs0);
        wait_vmcnt<0>();
    }
    const Stamp s1 = stamp();
    if constexpr (kB >= 6)   // accumulators in AGPRs (the 128 x 128 tile keeps them in VGPRs)
        pin_acc(acc);
    store_tile<kB, kB, kT, kDtype == kFp8, (kB >= 6)>(p, tm, tn, c.a_rows / kRowBytes,
                                                      (c.b_rows - kRing) / kRowBytes, lane, acc);
    write_trace(p, s0, s1, tm, tn);
}

// MXFP8 scale packing: entry e (0..7) of lane l at K step t of 128-row group
// g is the E8M0 scale of row 128 g + rowmap(e, l) and k block 4 t + l / 16,
// where rowmap is the row the 4-wave kernel's fragment e gives lane l:
// A: 16 e + x; B: 32 (e >> 1) + 4 (e & 1) + (x & 3) + 8 (x >> 2), x = l % 16.
// Rows past `rows` and blocks past `nblk` get 127 (scale 1; their elements
// are zeros).  One workgroup handles one group g and kPackSteps K steps: it
// reads the 128 x 4 kPackSteps source bytes row by row (coalesced) into LDS,
// then writes the kPackSteps x 512 packed bytes in order.
constexpr int kPackSteps = 16;
constexpr int kPackCols = 4 * kPackSteps;   // source blocks per workgroup

__global__ __launch_bounds__(256) void mx_pack_kernel(int operand, int rows, int nblk, int nk,
                                                      const uint8_t *src, uint64_t *dst)
{
    __shared__ uint8_t tile[128][kPackCols];
    const int64_t g = blockIdx.x;
    const int t0 = blockIdx.y * kPackSteps;
    const int b0 = 4 * t0;
    // all loads first (a fixed trip count, unrolled), then the LDS stores, so
    // the loads overlap instead of each store waiting for its own load
    constexpr int kPer = 128 * kPackCols / 256;
    uint8_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + 256 * k;
        const int64_t row = 128 * g + i / kPackCols;
        const int blk = b0 + i % kPackCols;
        v[k] = (row < rows && blk < nblk) ? src[row * nblk + blk] : uint8_t(127);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + 256 * k;
        tile[i / kPackCols][i % kPackCols] = v[k];
    }
    __syncthreads();
    const int steps = min(kPackSteps, nk - t0);
    for (int i = threadIdx.x; i < steps * 64; i += 256) {
        const int tt = i >> 6, l = i & 63;
        const int x = l & 15, cblk = 4 * tt + (l >> 4);
        uint64_t v = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r_in = operand == 0 ? 16 * e + x
                                          : 32 * (e >> 1) + 4 * (e & 1) + (x & 3) + 8 * (x >> 2);
            v |= (uint64_t)tile[r_in][cblk] << (8 * e);
        }
        dst[(g * nk + t0 + tt) * 64 + l] = v;
    }
}

__global__ void remap_tiles_kernel(int Gm, int Gn, int W, int C, int32_t *out)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < Gm * Gn) {
        int tm, tn;
        remap_tile(b, Gm, Gn, W, C, tm, tn);
        out[2 * b] = tm;
        out[2 * b + 1] = tn;
    }
}

// Which XCD (accelerator complex die) and which compute unit each workgroup
// of a launch runs on: out[2 b] = the XCC_ID hardware register (bits 3:0 the
// die), out[2 b + 1] = the HW_ID register (wave slot, SIMD, CU, shader array
// and engine ids).  kFull: the workgroup declares the whole 160 KiB of LDS,
// as the 256 x 256 GEMM kernels do, so at most one runs per CU.  Workgroup b
// first waits ((b * 37) % 64) * spin / 64 shader cycles (a bounded wait on the
// cycle counter), so that workgroups finish out of order.
template <bool kFull>
__global__ __launch_bounds__(256) void xcd_probe_kernel(int spin, int32_t *out)
{
    __shared__ char lds[kFull ? kLdsBytes : 256];
    lds[threadIdx.x] = (char)threadIdx.x;
    __syncthreads();
    if (threadIdx.x != 0)
        return;
    const uint64_t wait = (uint64_t)((blockIdx.x * 37u) % 64u) * (uint64_t)spin / 64u;
    const uint64_t t0 = __builtin_readcyclecounter();
    while (__builtin_readcyclecounter() - t0 < wait) {
    }
    uint32_t xcc, hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    out[2 * blockIdx.x] = (int32_t)xcc + (lds[1] - 1);    // lds[1] == 1: keeps the array live
    out[2 * blockIdx.x + 1] = (int32_t)hw;
}

}  // namespace

hipError_t launch_gemm(Dtype dt, Schedule s, const GemmParams &p, hipStream_t stream)
{
    const dim3 grid(p.Gm * p.Gn), block(512);
    if (dt == kMx) {
        // only the 4-wave kernel has the block-scaled MFMA path
        if (s == kInterleave)
            hipLaunchKernelGGL((gemm4_kernel<kMx, 256>), grid, dim3(256), 0, stream, p);
        else if (s == kInterleave128)
            hipLaunchKernelGGL((gemm4_kernel<kMx, 128>), grid, dim3(256), 0, stream, p);
        else
            return hipErrorInvalidValue;
    } else if (s == kInterleave) {
        if (dt == kBf16)
            hipLaunchKernelGGL((gemm4_kernel<kBf16, 256>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((gemm4_kernel<kFp8, 256>), grid, dim3(256), 0, stream, p);
    } else if (s == kInterleave128) {
        if (dt == kBf16)
            hipLaunchKernelGGL((gemm4_kernel<kBf16, 128>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((gemm4_kernel<kFp8, 128>), grid, dim3(256), 0, stream, p);
    } else if (s == kInterleave192) {
        if (dt == kBf16)
            hipLaunchKernelGGL((gemm4_kernel<kBf16, 192>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((gemm4_kernel<kFp8, 192>), grid, dim3(256), 0, stream, p);
    } else if (dt == kBf16) {
        if (s == kPingPong)
            hipLaunchKernelGGL((gemm_kernel<kBf16, kPingPong>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<kBf16, kLockstep>), grid, block, 0, stream, p);
    } else {
        if (s == kPingPong)
            hipLaunchKernelGGL((gemm_kernel<kFp8, kPingPong>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<kFp8, kLockstep>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_mx_pack(int operand, int rows, int nblk, int nk, int groups,
                          const uint8_t *src, uint8_t *dst, hipStream_t stream)
{
    if (groups == 0 || nk == 0)
        return hipSuccess;
    const dim3 grid((unsigned)groups, (unsigned)((nk + kPackSteps - 1) / kPackSteps));
    hipLaunchKernelGGL(mx_pack_kernel, grid, dim3(256), 0, stream, operand, rows, nblk, nk, src,
                       reinterpret_cast<uint64_t *>(dst));
    return hipGetLastError();
}

hipError_t launch_xcd_probe(int workgroups, bool full_lds, int spin, int32_t *out,
                            hipStream_t stream)
{
    if (full_lds)
        hipLaunchKernelGGL(xcd_probe_kernel<true>, dim3(workgroups), dim3(256), 0, stream, spin, out);
    else
        hipLaunchKernelGGL(xcd_probe_kernel<false>, dim3(workgroups), dim3(256), 0, stream, spin, out);
    return hipGetLastError();
}

hipError_t launch_remap_tiles(int Gm, int Gn, int W, int C, int32_t *out, hipStream_t stream)
{
    const int G = Gm * Gn;
    hipLaunchKernelGGL(remap_tiles_kernel, dim3((G + 255) / 256), dim3(256), 0, stream, Gm, Gn,
                       W, C, out);
    return hipGetLastError();
}

}  // namespace hkg
