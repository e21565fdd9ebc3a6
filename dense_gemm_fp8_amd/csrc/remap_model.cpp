// remap_model.cpp -- Eq. 1 cache model of the grid orders (host only).
#include <hip/hip_runtime.h>

#include <vector>

#include "remap.h"
#include "remap_model.h"

namespace hkg {

RemapModel model_remap(int Gm, int Gn, int W, int C, int64_t panel_bytes, int per_xcd)
{
    const int64_t G = int64_t(Gm) * Gn;
    const int64_t per_round = int64_t(kNumXcd) * per_xcd;
    int64_t rounds = (G + per_round - 1) / per_round;
    if (rounds > kModelRounds)
        rounds = kModelRounds;
    // *_x: (round, XCD) that last requested a panel; *_r: round that last used
    // it anywhere on the chip (-2: never, so that round 0 finds nothing cached)
    std::vector<int> row_x(Gm, -1), col_x(Gn, -1), row_r(Gm, -2), col_r(Gn, -2);
    int64_t requests = 0, misses = 0, prev_union = 0;
    double llc_requests = 0.0, llc_hits = 0.0;
    for (int r = 0; r < rounds; ++r) {
        int64_t fetched = 0, uni = 0, from_prev = 0;
        auto use = [&](std::vector<int> &sx, std::vector<int> &sr, int p, int stamp) {
            if (sx[p] == stamp)
                return;                      // this XCD's L2 already has it this round
            sx[p] = stamp;
            ++misses;
            ++fetched;
            if (sr[p] != r) {                // first request on the chip this round
                if (sr[p] == r - 1)
                    ++from_prev;
                sr[p] = r;
                ++uni;
            }
        };
        for (int x = 0; x < kNumXcd; ++x) {
            for (int j = 0; j < per_xcd; ++j) {
                const int64_t b = x + int64_t(kNumXcd) * (int64_t(per_xcd) * r + j);
                if (b >= G)
                    break;
                int tm, tn;
                remap_tile(static_cast<int>(b), Gm, Gn, W, C, tm, tn);
                requests += 2;
                use(row_x, row_r, tm, r * kNumXcd + x);
                use(col_x, col_r, tn, r * kNumXcd + x);
            }
        }
        llc_requests += fetched;
        llc_hits += fetched - uni;                       // another XCD fetched it this round
        // still cached from the last round (prev_union x panel_bytes <= the
        // LLC, compared as a quotient so that no panel size can wrap it)
        if (panel_bytes == 0 || prev_union <= kLlcBytes / panel_bytes)
            llc_hits += from_prev;
        prev_union = uni;
    }
    RemapModel m;
    m.l2_hit = requests ? 1.0 - double(misses) / double(requests) : 0.0;
    m.llc_hit = llc_requests > 0 ? llc_hits / llc_requests : 0.0;
    m.bw_tbs = kEq1LlcBwTBs * m.llc_hit + kEq1L2BwTBs * m.l2_hit;
    return m;
}

}  // namespace hkg
