"""Chiplet-aware grid remap, written from the pages -- TEST INFRASTRUCTURE ONLY.

Source: HipKittens L2 note, section 2 (Q2, "Pillar 3 -- Non-programmable
cache"), section 7 (code citation 5, "XCD swizzle (Algorithm 1, section 3.4)")
and section 5 (Table 4 parameters W, C).  The pages describe the steps but do
not print the pseudocode, so this is the plainest reading of their steps:

  1. flatten the launch grid to a linear block id b in [0, G), G = Gm * Gn;
  2. cycle-aligned boundaries: a cycle is nXCD * C consecutive ids; the
     largest multiple of the cycle that fits in G is handled as full cycles;
  3. de-interleave the round-robin dispatch: the hardware hands block b to
     XCD b mod nXCD, so the j-th block an XCD receives inside a cycle is given
     the id  cycle_start + xcd * C + j, i.e. each XCD owns C consecutive ids;
     the ids after the last full cycle use the same rule with the chunk
     shrunk to what is left (t // nXCD per XCD); any final t mod nXCD ids are
     left in place;
  4. windowed traversal: the remapped id walks the Gm x Gn tile grid in
     windows of W tile rows, column-major inside each window (the last window
     is shorter when W does not divide Gm);
  5. the result is the output tile (tile_m, tile_n).

Integer arithmetic only; W = 1 and C = 1 reproduce row-major order.
"""
from __future__ import annotations

NXCD = 8


def deinterleave(b: int, G: int, C: int, nxcd: int = NXCD) -> int:
    """Step 2-3: linear id b -> id after grouping C consecutive ids per XCD."""
    if not (0 <= b < G) or C < 1:
        raise ValueError("bad block id or chunk")
    cycle = nxcd * C
    full = (G // cycle) * cycle
    if b < full:
        xcd = b % nxcd                  # which XCD the hardware sent b to
        j = b // nxcd                   # how many blocks that XCD received before b
        return (j // C) * cycle + xcd * C + (j % C)
    t = G - full                        # ids after the last full cycle
    ct = t // nxcd                      # shrunken chunk for the tail
    lim = full + nxcd * ct
    if b < lim:
        r = b - full
        return full + (r % nxcd) * ct + r // nxcd
    return b


def window(bp: int, Gm: int, Gn: int, W: int) -> tuple[int, int]:
    """Step 4: remapped id -> (tile_m, tile_n), windows of W tile rows."""
    if W < 1:
        raise ValueError("bad window")
    per_window = W * Gn
    win = bp // per_window
    rem = bp % per_window
    h = min(W, Gm - win * W)            # the last window may be shorter
    return win * W + rem % h, rem // h


def remap(b: int, Gm: int, Gn: int, W: int, C: int, nxcd: int = NXCD) -> tuple[int, int]:
    """Block id b of a flat launch of Gm*Gn blocks -> output tile (tile_m, tile_n)."""
    G = Gm * Gn
    return window(deinterleave(b, G, C, nxcd), Gm, Gn, W)


def remap_table(Gm: int, Gn: int, W: int, C: int, nxcd: int = NXCD):
    """[(tile_m, tile_n) for b in 0..G-1]."""
    return [remap(b, Gm, Gn, W, C, nxcd) for b in range(Gm * Gn)]
