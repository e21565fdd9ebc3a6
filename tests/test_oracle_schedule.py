"""Pins of the grid remap reading and of the Eq. 1 fit against the pages."""
import itertools

import pytest

from oracle import eq1, remap


CASES = [(1, 1), (1, 7), (3, 5), (4, 4), (8, 8), (32, 32), (57, 57), (64, 56), (36, 36)]


@pytest.mark.parametrize("Gm,Gn", CASES)
def test_remap_is_a_bijection(Gm, Gn):
    for W, C in itertools.product([1, 2, 5, 7, 8, 16, 64], [1, 4, 25, 32, 64, 216, 542]):
        tiles = remap.remap_table(Gm, Gn, W, C)
        assert len(set(tiles)) == Gm * Gn
        assert all(0 <= tm < Gm and 0 <= tn < Gn for tm, tn in tiles)


@pytest.mark.parametrize("Gm,Gn", CASES)
def test_w1_c1_is_row_major(Gm, Gn):
    assert remap.remap_table(Gm, Gn, 1, 1) == [(b // Gn, b % Gn) for b in range(Gm * Gn)]


def test_each_xcd_gets_chunks_of_C_consecutive_ids():
    G, C = 1024, 16
    ids = [remap.deinterleave(b, G, C) for b in range(G)]
    for x in range(8):
        mine = [ids[b] for b in range(x, G, 8)]          # dispatch order on XCD x
        for start in range(0, len(mine), C):
            chunk = mine[start:start + C]
            assert chunk == list(range(chunk[0], chunk[0] + C))
            assert (chunk[0] // C) % 8 == x


def test_chunk_of_an_eighth_gives_each_xcd_one_contiguous_range():
    # the "L2-only" extreme of Table 4 (C216 at 36x36 tiles = 1296 = 8 * 162 ... + tail)
    G = 32 * 32
    C = G // 8
    ids = [remap.deinterleave(b, G, C) for b in range(G)]
    for x in range(8):
        assert sorted(ids[b] for b in range(x, G, 8)) == list(range(x * C, (x + 1) * C))


def test_window_walks_columns_inside_a_window():
    # W = 8 over 32 x 32 tiles: ids 0..31 form an 8 x 4 patch
    tiles = [remap.window(b, 32, 32, 8) for b in range(32)]
    assert sorted(tiles) == [(m, n) for m in range(8) for n in range(4)]
    assert tiles[:9] == [(m, 0) for m in range(8)] + [(0, 1)]


def test_tail_is_deinterleaved_when_cycle_does_not_divide():
    # 36x36 = 1296 tiles with C = 216: no full cycle (8*216 = 1728 > 1296), so the
    # tail rule must still give each XCD one contiguous run (162 ids each)
    G, C = 1296, 216
    ids = [remap.deinterleave(b, G, C) for b in range(G)]
    assert sorted(ids) == list(range(G))
    for x in range(8):
        mine = sorted(ids[b] for b in range(x, G, 8))
        assert mine == list(range(mine[0], mine[0] + len(mine)))


def test_eq1_fit_reproduces_table4():
    rows = eq1.load_table4(eq1.default_table4_path())
    assert len(rows) == 6
    l2_bw, llc_bw = eq1.fit(rows)
    # the table prints BW to 0.1 TB/s and hit rates to whole percent, so a row
    # can sit up to 0.05 + 0.005 * (L2_BW + LLC_BW) from the exact model value
    slack = 0.05 + 0.005 * (l2_bw + llc_bw)
    for r in rows:
        pred = eq1.model_bw(r["l2_pct"] / 100, r["llc_pct"] / 100, l2_bw, llc_bw)
        assert abs(pred - r["bw_tbs"]) <= slack
    # the pages: L2 bandwidth is about 3x LLC bandwidth
    assert 2.5 <= l2_bw / llc_bw <= 3.5
    assert abs(l2_bw - 17.05) < 0.05 and abs(llc_bw - 5.99) < 0.05


def test_eq1_orders_table4_like_tflops():
    rows = eq1.load_table4(eq1.default_table4_path())
    l2_bw, llc_bw = eq1.fit(rows)
    for size in (9216, 14592):
        rs = [r for r in rows if r["size"] == size]
        by_bw = sorted(rs, key=lambda r: eq1.model_bw(r["l2_pct"] / 100, r["llc_pct"] / 100, l2_bw, llc_bw))
        by_tf = sorted(rs, key=lambda r: r["tflops"])
        assert [r["tflops"] for r in by_bw] == [r["tflops"] for r in by_tf]
