// remap.h -- chiplet-aware workgroup -> output-tile remap for the GEMM kernels.
//
// HipKittens L2 note: section 2 (Pillar 3, non-programmable cache), section 7
// (code citation 5, Algorithm 1 "XCD swizzle"), section 5 (Table 4: window W,
// chunk C).  The hardware hands workgroup b of a launch to XCD b mod 8, so
// neighbouring ids land on different L2 caches.  The remap
//   1. takes the flat id b of the Gm x Gn grid;
//   2. splits [0, G) at multiples of one cycle of 8*C ids;
//   3. inside full cycles gives the j-th workgroup an XCD receives the id
//      cycle_start + xcd*C + j, so each XCD works on C consecutive ids; after
//      the last full cycle the same is done with the chunk shrunk to the ids
//      left (per XCD), and the last (G - full) mod 8 ids keep their place;
//   4. walks the Gm x Gn tile grid in windows of W tile rows, column-major
//      inside a window, so an XCD's C consecutive ids form a W-tall patch.
// Integer-only; W = 1 and C = 1 give row-major order.  The host clamps
// 1 <= W <= Gm and 1 <= C <= G/8 + 1 (larger values give the same order)
// so that W*Gn and 8*C stay within 32 bits for G < 2^30.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#define HKG_HD inline
#else
#define HKG_HD __host__ __device__ __forceinline__
#endif

namespace hkg {

constexpr int kNumXcd = 8;

// W beyond the grid height, and any chunk with 8*C > G (no full cycle: the
// whole grid is handled by the tail rule), give the same order; clamping keeps
// the kernel's 32-bit products W*Gn and 8*C in range for G < 2^30.
inline void clamp_order(int64_t Gm, int64_t Gn, int64_t &W, int64_t &C)
{
    const int64_t G = Gm * Gn;
    if (W > Gm)
        W = Gm;
    if (C > G / kNumXcd + 1)
        C = G / kNumXcd + 1;
    if (W < 1)
        W = 1;
    if (C < 1)
        C = 1;
}

HKG_HD void remap_tile(int b, int Gm, int Gn, int W, int C, int &tile_m, int &tile_n)
{
    const int G = Gm * Gn;
    const int cycle = kNumXcd * C;
    const int full = (G / cycle) * cycle;
    int id = b;
    if (b < full) {
        const int xcd = b % kNumXcd;
        const int j = b / kNumXcd;
        id = (j / C) * cycle + xcd * C + (j % C);
    } else {
        const int left = G - full;
        const int chunk = left / kNumXcd;
        const int r = b - full;
        if (r < kNumXcd * chunk)
            id = full + (r % kNumXcd) * chunk + r / kNumXcd;
    }
    const int per_window = W * Gn;
    const int win = id / per_window;
    const int rem = id - win * per_window;
    const int rows_left = Gm - win * W;
    const int h = rows_left < W ? rows_left : W;
    tile_m = win * W + rem % h;
    tile_n = rem / h;
}

}  // namespace hkg
