// remap_model.h -- a cache model of the grid orders (host only).
//
// HipKittens L2 note, section 4 (the paper's single equation) and section 5
// (Table 4): effective operand bandwidth is
//     BW = LLC_BW * LLC_hit + L2_BW * L2_hit,
// and the window height W and per-XCD chunk C of the grid remap are tuned to
// maximise it.  The pages print the equation and measured hit rates but no
// way to predict the hit rates of an order before running it; this model
// predicts them from the launch itself:
//  - dispatch: workgroup b runs on XCD b mod 8 (checked on the GPU); each XCD
//    runs `per_xcd` workgroups at a time (32 CUs x workgroups per CU), so
//    round r of XCD x holds workgroups x + 8 (per_xcd r + j), j < per_xcd;
//  - L2 (one per XCD): the tiles an XCD holds at once stream the same K
//    steps together, so each distinct operand panel (a tile row of A or a
//    tile column of B) misses once per round and every other request for it
//    hits: L2_hit = 1 - distinct panels / (2 x tiles);
//  - LLC (shared by the XCDs): an L2 miss hits the LLC when another XCD
//    fetches the same panel in the same round, or when the panel was used in
//    the previous round and that round's panels (whole panels: tile rows x
//    K x element bytes each) fit the LLC; a cyclic stream larger than the
//    cache keeps nothing between rounds.
// Constants: L2_BW 17.05 and LLC_BW 5.99 TB/s reproduce every "Mem BW" entry
// of Table 4 by least squares; the LLC holds 256 MiB.
#pragma once

#include <stdint.h>

namespace hkg {

constexpr double kEq1L2BwTBs = 17.05;
constexpr double kEq1LlcBwTBs = 5.99;
constexpr int64_t kLlcBytes = int64_t(256) << 20;
constexpr int kCusPerXcd = 32;
constexpr int kModelRounds = 8;   // rounds simulated (the pattern repeats)

struct RemapModel {
    double l2_hit;    // fraction of operand-panel requests that hit an XCD's L2
    double llc_hit;   // fraction of L2 misses that hit the LLC
    double bw_tbs;    // Eq. 1
};

// The model for a Gm x Gn tile grid in order (W, C) (both already clamped to
// the grid), operand panels of panel_bytes, per_xcd workgroups in flight per XCD.
RemapModel model_remap(int Gm, int Gn, int W, int C, int64_t panel_bytes, int per_xcd);

}  // namespace hkg
