"""The C ABI library on the CPU: it loads, exports every declared symbol, and
its host-side logic (validation before any HIP call, the grid remap, the
default remap choice) behaves as documented.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_gemm_fp8_amd as hkg
from oracle import remap as oracle_remap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "hkg.h")).read()
    return sorted(set(re.findall(r"\b(hkg_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = hkg.load()
    names = _declared()
    assert len(names) == 18
    assert sorted(hkg.EXPORTS) == names
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    for s in range(0, -9, -1):
        assert hkg.hkg_status_string(s) != "unknown status"
    assert hkg.hkg_status_string(5) == "unknown status"


FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation
FB, FC = FAKE + (64 << 20), FAKE + (128 << 20)   # distinct fake B and C (no overlap)


@pytest.mark.parametrize("M,N,K", [(-256, 256, 64), (256, -1, 64), (256, 256, -8), (256, 256, 63),
                                   (300, 100, 4), (1, 1, 12)])
def test_bad_shapes_rejected(M, N, K):
    # any M, N >= 0 is accepted; K must be a multiple of 8 (16-byte operand rows)
    assert hkg.hkg_gemm_bf16(M, N, K, FAKE, FAKE, FAKE, None, None) == hkg.HKG_ERR_SHAPE


def test_fp8_needs_k_multiple_of_16():
    for K in (8, 72, 100):
        assert hkg.hkg_gemm_fp8(256, 256, K, FAKE, FAKE, 1.0, 1.0, FAKE, None, None) == hkg.HKG_ERR_SHAPE


def test_null_and_alignment_rejected():
    assert hkg.hkg_gemm_bf16(256, 256, 64, None, FAKE, FAKE, None, None) == hkg.HKG_ERR_NULL
    assert hkg.hkg_gemm_bf16(256, 256, 64, FAKE, FAKE, None, None, None) == hkg.HKG_ERR_NULL
    assert hkg.hkg_gemm_bf16(256, 256, 64, FAKE + 8, FAKE, FAKE, None, None) == hkg.HKG_ERR_ALIGN
    assert hkg.hkg_gemm_bf16(256, 256, 64, FAKE, FAKE, FAKE, FAKE + 4, None) == hkg.HKG_ERR_ALIGN
    assert hkg.hkg_gemm_fp8(256, 256, 128, FAKE, FAKE + 2, 1.0, 1.0, FAKE, None, None) == hkg.HKG_ERR_ALIGN


def test_size_limit_rejected():
    # one 256-row bf16 panel of K = 2^22 is 2 GiB: beyond the 32-bit buffer range
    assert hkg.hkg_gemm_bf16(256, 256, 1 << 22, FAKE, FAKE, FAKE, None, None) == hkg.HKG_ERR_SIZE


def test_launch_plan_sizes_like_the_entry_points():
    # a 256-row bf16 panel of K = 2^22 is 2 GiB; an empty output launches nothing
    # and is accepted whatever its other extents, by the plan as by the GEMM
    assert hkg.launch_plan(256, 256, 1 << 22, 0)[0] == hkg.HKG_ERR_SIZE
    assert hkg.launch_plan(256, 1 << 31, 64, 0)[0] == hkg.HKG_ERR_SIZE
    assert hkg.launch_plan(0, 256, 1 << 22, 0)[0] == hkg.HKG_OK
    assert hkg.hkg_gemm_bf16(0, 256, 1 << 22, FAKE, FAKE, FAKE, None, None) == hkg.HKG_OK


def test_overlapping_outputs_rejected():
    # an output sharing a byte with an input (or with the other output) is refused
    # before any launch; inputs may alias each other
    M, N, K = 256, 256, 64
    a, b = FAKE, FAKE + (64 << 20)
    c = FAKE + (128 << 20)
    assert hkg.hkg_gemm_bf16(M, N, K, a, b, a, None, None) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_bf16(M, N, K, a, b, a + M * K * 2 - 16, None, None) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_bf16(M, N, K, a, b, b - M * N * 2 + 16, None, None) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_bf16(M, N, K, a, b, c, c + M * N * 2 - 16, None) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_bf16(M, N, K, a, b, c, b, None) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_fp8(M, N, 128, a, b, 1.0, 1.0, b + 4096, None, None) == hkg.HKG_ERR_OVERLAP
    sa, sb = FAKE + (192 << 20), FAKE + (200 << 20)
    assert hkg.hkg_gemm_mxfp8(M, N, 128, a, b, sa, sb, sa, None, None) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_mx_pack_scales(0, M, 128, FAKE, FAKE + 16, None) == hkg.HKG_ERR_OVERLAP
    # adjacent (touching, not sharing) buffers and A == B pass validation: any
    # other status (no device here) is not an overlap
    assert hkg.hkg_gemm_bf16(M, N, K, a, b, a + M * K * 2, None, None) != hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_bf16(M, N, K, a, a, c, None, None) != hkg.HKG_ERR_OVERLAP
    assert "overlap" in hkg.hkg_status_string(hkg.HKG_ERR_OVERLAP)


def test_bad_opts_rejected():
    bad = [hkg.make_opts(remap=7), hkg.make_opts(schedule=9), hkg.make_opts(remap=hkg.HKG_REMAP_XCD, W=0, C=4),
           hkg.make_opts(remap=hkg.HKG_REMAP_XCD, W=4, C=0)]
    for o in bad:
        assert hkg.hkg_gemm_bf16_ex(256, 256, 64, FAKE, FB, FC, None, None, o) == hkg.HKG_ERR_OPTS


def test_empty_output_is_a_noop():
    # M == 0 or N == 0: nothing to compute, nothing launched, pointers unused
    assert hkg.hkg_gemm_bf16(0, 256, 64, None, None, None, None, None) == hkg.HKG_OK
    assert hkg.hkg_gemm_fp8(256, 0, 128, None, None, 1.0, 1.0, None, None, None) == hkg.HKG_OK


@pytest.mark.parametrize("Gm,Gn", [(1, 1), (3, 5), (32, 32), (64, 56), (36, 36), (57, 57)])
def test_host_remap_matches_oracle(Gm, Gn):
    for W, C in [(1, 1), (8, 32), (5, 25), (7, 216), (8, 64), (8, 542), (3, 7)]:
        want = oracle_remap.remap_table(Gm, Gn, min(W, Gm), min(C, Gm * Gn // 8 + 1))
        got = []
        for b in range(Gm * Gn):
            rc, tm, tn = hkg.hkg_remap_tile(Gm, Gn, W, C, b)
            assert rc == hkg.HKG_OK
            got.append((tm, tn))
        assert got == want


def test_remap_clamping_does_not_change_order():
    # W beyond the grid height and chunks with 8*C > G give the same order
    Gm, Gn = 6, 10
    assert oracle_remap.remap_table(Gm, Gn, 6, 8) == oracle_remap.remap_table(Gm, Gn, 6, 1000)
    assert oracle_remap.remap_table(Gm, Gn, 6, 8) == oracle_remap.remap_table(Gm, Gn, 99, 8)


def test_remap_rejects_bad_arguments():
    assert hkg.hkg_remap_tile(4, 4, 1, 1, 16)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_remap_tile(4, 4, 0, 1, 0)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_remap_tiles_device(4, 4, 1, 1, None, None) == hkg.HKG_ERR_NULL


def test_default_remap():
    rc, W, C = hkg.hkg_default_remap(8192, 8192, 8192, 0)
    assert rc == hkg.HKG_OK and (W, C) == (8, 32)
    assert hkg.hkg_default_remap(8192, 8192, 8192, 3)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_default_remap(8192, 8192, 8192, 2)[0] == hkg.HKG_OK       # MXFP8
    assert hkg.hkg_default_remap(8192, 8192, 8176, 2)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_default_remap(8192, 8192, 8190, 0)[0] == hkg.HKG_ERR_SHAPE
    # small grids run on 128 x 128 tiles by default, and the order is for that grid
    rc, W, C = hkg.hkg_default_remap(256, 256, 256, 1)     # 2 x 2 tiles of 128
    assert rc == hkg.HKG_OK and (W, C) == (2, 1)
    rc, W, C = hkg.hkg_default_remap(256, 256, 256, 2)     # MXFP8 as well: 2 x 2 tiles of 128
    assert rc == hkg.HKG_OK and (W, C) == (2, 1)
    rc, W, C = hkg.hkg_default_remap(300, 9000, 64, 0)     # ragged: 3 x 71 tiles of 128
    assert rc == hkg.HKG_OK and (W, C) == (3, 27)
    rc, W, C = hkg.hkg_default_remap(1000, 9000, 64, 0)    # ragged: 4 x 36 tiles of 256
    assert rc == hkg.HKG_OK and (W, C) == (4, 19)


@pytest.mark.parametrize("M,N,K,dtype,want", [
    (9216, 9216, 9216, 0, (8, 32)),         # 40 panels x 4.5 MiB fit the last-level cache
    (16384, 14336, 4096, 0, (8, 32)),
    (12288, 12288, 12288, 1, (8, 32)),      # e4m3: 3 MiB panels
    (10000, 10000, 10000, 0, (16, 4)),      # bf16 rows past 18944 bytes
    (12288, 12288, 12288, 0, (16, 4)),
    (16384, 16384, 16384, 0, (16, 4)),
    (16384, 16384, 20480, 1, (16, 4)),
    (2048, 2048, 16384, 0, (16, 4)),        # 16 x 16 tiles of 128: (16, 4) fits
    (2048, 2048, 32768, 2, (16, 4)),        # MXFP8, 16 x 16 tiles of 128
    (2560, 2560, 32768, 2, (16, 4)),        # 100 tiles of 256 -> 20 x 20 of 128: W = 16 fits
    (3072, 3072, 32768, 2, (12, 4)),        # 144 tiles of 256: (16, 4) with W clamped to 12
])
def test_default_remap_follows_panel_bytes(M, N, K, dtype, want):
    """Rows longer than 18944 bytes switch the default from an 8 x 32 strip of
    concurrent tiles to a 16 x 16 block (fewer panels in the last-level
    cache); both keep 12 panels per XCD's L2."""
    rc, W, C = hkg.hkg_default_remap(M, N, K, dtype)
    assert rc == hkg.HKG_OK and (W, C) == want


# ---------------------------------------------------------------- MXFP8 -------------

def test_mx_packed_scale_bytes():
    # ceil(rows/128) groups x ceil(K/128) K steps x 64 lanes x 8 bytes
    assert hkg.hkg_mx_packed_scale_bytes(8192, 8192) == 64 * 64 * 512
    assert hkg.hkg_mx_packed_scale_bytes(129, 160) == 2 * 2 * 512
    assert hkg.hkg_mx_packed_scale_bytes(1, 32) == 512
    assert hkg.hkg_mx_packed_scale_bytes(0, 64) == 0
    assert hkg.hkg_mx_packed_scale_bytes(100, 0) == 0
    for rows, K in ((-1, 64), (10, -32), (10, 48)):
        assert hkg.hkg_mx_packed_scale_bytes(rows, K) == hkg.HKG_ERR_SHAPE
    # sizes the pack refuses, including ones whose products would wrap 64 bits
    assert hkg.hkg_mx_packed_scale_bytes(1 << 20, 1 << 15) == 1 << 30   # 2^13 x 2^8 x 512
    for rows, K in ((1 << 31, 64), (1, 1 << 23), (1 << 62, 1 << 40), (1, (1 << 63) - 32)):
        assert hkg.hkg_mx_packed_scale_bytes(rows, K) == hkg.HKG_ERR_SIZE, (rows, K)


def test_mx_pack_rejects_bad_arguments():
    A, B = hkg.HKG_MX_OPERAND_A, hkg.HKG_MX_OPERAND_B
    assert hkg.hkg_mx_pack_scales(2, 10, 64, FAKE, FAKE, None) == hkg.HKG_ERR_OPTS
    assert hkg.hkg_mx_pack_scales(A, 10, 48, FAKE, FAKE, None) == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_mx_pack_scales(B, -1, 64, FAKE, FAKE, None) == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_mx_pack_scales(A, 10, 64, None, FAKE, None) == hkg.HKG_ERR_NULL
    assert hkg.hkg_mx_pack_scales(A, 10, 64, FAKE, FAKE + 8, None) == hkg.HKG_ERR_ALIGN
    assert hkg.hkg_mx_pack_scales(A, 0, 64, None, None, None) == hkg.HKG_OK      # nothing to do
    assert hkg.hkg_mx_pack_scales(A, 1, 1 << 23, FAKE, FAKE, None) == hkg.HKG_ERR_SIZE
    # K near 2^63 would wrap 256 x K and ceil(K / 128) negative: refused, never
    # launched with truncated sizes
    for rows, K in ((1, (1 << 63) - 32), (1 << 40, 64), ((1 << 62) + 128, 1 << 40)):
        assert hkg.hkg_mx_pack_scales(A, rows, K, FAKE, FB, None) == hkg.HKG_ERR_SIZE, (rows, K)


def test_mxfp8_validation():
    g = hkg.hkg_gemm_mxfp8
    for K in (16, 48, 100):
        assert g(256, 256, K, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == hkg.HKG_ERR_SHAPE
    SA, SB = FAKE + (192 << 20), FAKE + (200 << 20)
    assert g(256, 256, 64, FAKE, FB, None, SB, FC, None, None) == hkg.HKG_ERR_NULL
    assert g(256, 256, 64, FAKE, FB, SA, SB + 8, FC, None, None) == hkg.HKG_ERR_ALIGN
    assert g(0, 256, 64, None, None, None, None, None, None, None) == hkg.HKG_OK
    for sched in (hkg.HKG_SCHED_PINGPONG, hkg.HKG_SCHED_LOCKSTEP):
        o = hkg.make_opts(schedule=sched)
        assert hkg.hkg_gemm_mxfp8_ex(256, 256, 64, FAKE, FB, SA, SB, FC, None, None,
                                     o) == hkg.HKG_ERR_OPTS


# ---------------------------------------------------------------- launch plan ------

def _plan(M, N, K, dtype=0, opts=None):
    rc, launches = hkg.launch_plan(M, N, K, dtype, opts)
    assert rc == hkg.HKG_OK
    return [(d["schedule"], d["tile"], d["rows"], d["grid"], d["W"], d["C"]) for d in launches]


def test_launch_plan_whole_rounds_one_launch():
    S4, S128 = hkg.HKG_SCHED_INTERLEAVE, hkg.HKG_SCHED_INTERLEAVE_128
    assert _plan(8192, 8192, 8192) == [(S4, 256, 8192, 1024, 8, 32)]
    assert _plan(16384, 16384, 16384) == [(S4, 256, 16384, 4096, 16, 4)]
    assert _plan(16384, 14336, 4096) == [(S4, 256, 16384, 3584, 8, 32)]
    assert _plan(8192, 8192, 8192, 1) == [(S4, 256, 8192, 1024, 8, 32)]


def test_launch_plan_small_grid_uses_128_tiles():
    S4, S128 = hkg.HKG_SCHED_INTERLEAVE, hkg.HKG_SCHED_INTERLEAVE_128
    assert _plan(2048, 2048, 2048) == [(S128, 128, 2048, 256, 8, 32)]
    assert _plan(256, 256, 256) == [(S128, 128, 256, 4, 2, 1)]
    assert _plan(2048, 2048, 2048, 2) == [(S128, 128, 2048, 256, 8, 32)]    # MXFP8 too
    assert _plan(3072, 3072, 3072, 2) == [(S4, 256, 3072, 144, 8, 19)]      # MXFP8: 144 > 128 tiles


def test_launch_plan_192_tiles_when_they_fill_one_round():
    S4, S128, S192 = (hkg.HKG_SCHED_INTERLEAVE, hkg.HKG_SCHED_INTERLEAVE_128,
                      hkg.HKG_SCHED_INTERLEAVE_192)
    # 192-tiles fit one round (<= 256) while 128-tiles would not (> 256)
    assert _plan(3072, 3072, 3072) == [(S192, 192, 3072, 256, 8, 32)]
    assert _plan(2304, 2304, 2304) == [(S192, 192, 2304, 144, 8, 19)]
    assert _plan(2816, 2816, 2816)[0][:4] == (S192, 192, 2816, 225)
    assert _plan(1536, 6144, 1024)[0][:4] == (S192, 192, 1536, 256)
    # 128-tiles fit one round: they stay; 192-tiles need two rounds: 256-tiles
    assert _plan(2048, 2048, 2048)[0][:2] == (S128, 128)
    assert _plan(3328, 3328, 3328)[0][:2] == (S4, 256)
    assert _plan(8192, 8192, 8192)[0][:2] == (S4, 256)
    # whole rounds of 192-tiles against a 256 x 256 grid ending a quarter full
    assert _plan(6144, 6144, 6144) == [(S192, 192, 6144, 1024, 8, 32)]     # 576 = 2 x 256 + 64
    assert _plan(3072, 12288, 4096)[0][:4] == (S192, 192, 3072, 1024)
    assert len(_plan(9216, 9216, 9216)) == 2                               # 1296 = 5 x 256 + 16: split
    assert _plan(12288, 12288, 12288)[0][:2] == (S4, 256)                  # 2304 = 9 x 256
    # e4m3 alike; MXFP8 (scales packed per 128 rows) keeps its tiles
    assert _plan(2304, 2304, 2304, 1)[0][:2] == (S192, 192)
    assert _plan(2304, 2304, 2304, 2)[0][:2] == (S128, 128)


def test_launch_plan_invariants_over_random_shapes():
    # whatever the shape, the launches cover the M rows exactly, each grid is its
    # row block in tiles of its edge, and a split keeps whole 256-rows first
    rng = np.random.default_rng(4242)
    edge = {hkg.HKG_SCHED_INTERLEAVE: 256, hkg.HKG_SCHED_INTERLEAVE_128: 128,
            hkg.HKG_SCHED_INTERLEAVE_192: 192}
    for _ in range(400):
        M, N = (int(v) for v in rng.integers(1, 20000, 2))
        dt = int(rng.integers(0, 3))
        K = 32 * int(rng.integers(1, 200))
        rc, L = hkg.launch_plan(M, N, K, dt)
        assert rc == hkg.HKG_OK, (M, N, K, dt)
        assert 1 <= len(L) <= 2
        assert sum(d["rows"] for d in L) == M
        for d in L:
            t = edge[d["schedule"]]
            assert d["tile"] == t
            gm, gn = -(-d["rows"] // t), -(-N // t)
            assert d["grid"] == gm * gn
            assert 1 <= d["W"] <= gm and d["C"] >= 1
            if dt == 2:
                assert t != 192                      # MXFP8 has no 192 x 192 kernel
        if len(L) == 2:
            assert L[0]["tile"] == 256 and L[0]["rows"] % 256 == 0
            assert L[1]["tile"] == 128 and L[1]["grid"] <= 512
            G = -(-M // 256) * -(-N // 256)          # the single-launch 256 x 256 grid
            assert L[0]["grid"] <= 256 * (G // 256)  # the first launch fits its whole rounds


def test_launch_plan_splits_partial_last_round():
    S4, S128 = hkg.HKG_SCHED_INTERLEAVE, hkg.HKG_SCHED_INTERLEAVE_128
    # 6144^3 MXFP8 (no 192 tile): 24 x 24 = 576 tiles = 2 rounds + 64; 21 tile rows
    # (504 tiles) stay on 256, the last 768 rows run as 6 x 48 tiles of 128
    assert _plan(6144, 6144, 6144, 2) == [(S4, 256, 5376, 504, 8, 32), (S128, 128, 768, 288, 6, 32)]
    p = _plan(4500, 4400, 136)
    assert len(p) == 2 and p[0][2] + p[1][2] == 4500 and p[0][2] % 256 == 0
    assert len(_plan(16448, 16448, 16448)) == 1        # 3 % idle: not worth a second launch
    # an explicit schedule or order is one launch of what was asked for
    one = _plan(6144, 6144, 6144, 0, hkg.make_opts(schedule=hkg.HKG_SCHED_INTERLEAVE))
    assert one == [(S4, 256, 6144, 576, 8, 32)]
    assert len(_plan(6144, 6144, 6144, 0, hkg.make_opts(remap=hkg.HKG_REMAP_ROW_MAJOR))) == 1
    pp = _plan(6144, 6144, 6144, 0, hkg.make_opts(schedule=hkg.HKG_SCHED_PINGPONG))
    assert pp == [(hkg.HKG_SCHED_PINGPONG, 256, 6144, 576, 8, 32)]


def test_launch_plan_192_tiles_on_request():
    S192 = hkg.HKG_SCHED_INTERLEAVE_192
    o = hkg.make_opts(schedule=S192)
    # 3072 / 192 = 16: 256 tiles, one whole round of 256 CUs
    assert _plan(3072, 3072, 3072, 0, o) == [(S192, 192, 3072, 256, 8, 32)]
    assert _plan(1000, 700, 64, 0, o)[0][1:4] == (192, 1000, 6 * 4)          # ragged edges
    assert _plan(3072, 3072, 3072, 1, o) == [(S192, 192, 3072, 256, 8, 32)]  # e4m3 too
    assert hkg.launch_plan(3072, 3072, 3072, 2, o)[0] == hkg.HKG_ERR_OPTS     # not MXFP8
    assert hkg.launch_plan(0, 3072, 3072, 2, o)[0] == hkg.HKG_ERR_OPTS


def test_launch_plan_errors_match_entry_points():
    assert hkg.launch_plan(0, 256, 64, 0)[0] == hkg.HKG_OK
    assert hkg.launch_plan(0, 256, 64, 0)[1] == []
    assert hkg.launch_plan(256, 256, 60, 0)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.launch_plan(256, 256, 64, 3)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.launch_plan(256, 256, 1 << 23, 0)[0] == hkg.HKG_ERR_SIZE
    bad = hkg.make_opts(schedule=hkg.HKG_SCHED_PINGPONG)
    assert hkg.launch_plan(256, 256, 64, 2, bad)[0] == hkg.HKG_ERR_OPTS      # MXFP8
    assert hkg.launch_plan(0, 256, 64, 2, bad)[0] == hkg.HKG_ERR_OPTS
    assert hkg.launch_plan(256, 256, 64, 0, hkg.make_opts(schedule=9))[0] == hkg.HKG_ERR_OPTS


def test_probe_xcd_rejects_bad_arguments():
    assert hkg.hkg_probe_xcd(8, 1, 0, None, None) == hkg.HKG_ERR_NULL
    assert hkg.hkg_probe_xcd(0, 1, 0, FAKE, None) == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_probe_xcd((1 << 24) + 1, 1, 0, FAKE, None) == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_probe_xcd(8, 2, 0, FAKE, None) == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_probe_xcd(8, 1, -1, FAKE, None) == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_probe_xcd(8, 0, 0, FAKE + 2, None) == hkg.HKG_ERR_ALIGN


def test_valid_call_without_a_gfx950_is_a_device_error():
    """A call that passes validation checks the stream's device before its
    first launch; on a host without a gfx950 (this CPU-only run) every entry
    point returns HKG_ERR_DEVICE and launches nothing."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    M, N, K = 256, 256, 64
    assert hkg.hkg_gemm_bf16(M, N, K, FAKE, FB, FC, None, None) == hkg.HKG_ERR_DEVICE
    assert hkg.hkg_gemm_fp8(M, N, 128, FAKE, FB, 1.0, 1.0, FC, None, None) == hkg.HKG_ERR_DEVICE
    assert hkg.hkg_probe_xcd(8, 1, 0, FAKE, None) == hkg.HKG_ERR_DEVICE
    assert hkg.hkg_remap_tiles_device(4, 4, 1, 1, FAKE, None) == hkg.HKG_ERR_DEVICE


def test_trace_buffer_validated_before_launch():
    M, N, K = 256, 256, 64
    o = hkg.make_opts(trace=FC + (64 << 20) + 4)            # not 8-byte aligned
    assert hkg.hkg_gemm_bf16_ex(M, N, K, FAKE, FB, FC, None, None, o) == hkg.HKG_ERR_ALIGN
    o = hkg.make_opts(trace=FC + 64)                         # inside C
    assert hkg.hkg_gemm_bf16_ex(M, N, K, FAKE, FB, FC, None, None, o) == hkg.HKG_ERR_OVERLAP
    o = hkg.make_opts(trace=FAKE)                            # over A
    assert hkg.hkg_gemm_fp8_ex(M, N, 128, FAKE, FB, 1.0, 1.0, FC, None, None, o) == hkg.HKG_ERR_OVERLAP
    assert ctypes.sizeof(hkg.hkg_gemm_opts) == 48
    assert [hkg.hkg_gemm_opts.__dict__[f].offset for f in ("remap", "W", "C", "schedule", "trace",
                                                           "lda", "ldb", "ldc")] == \
        [0, 4, 8, 12, 16, 24, 32, 40]


def _table4():
    import csv
    path = os.path.join(ROOT, "tests", "golden", "table4_chiplet_schedule.csv")
    return list(csv.DictReader(line for line in open(path) if not line.startswith("#")))


def test_remap_model_l2_term_tracks_table4():
    """The cache model's L2 hit rate for the pages' Table 4 orders (HipKittens L2
    note, section 5): within 6.5 points of the printed value on every row but the
    9216 row-major one (printed 55 %, modelled 73 %), and the rows of each size in
    the printed order of Eq. 1 bandwidth (TFLOPS order) at 14592."""
    got = {}
    for r in _table4():
        n = int(r["size"])
        g = -(-n // 256)
        rc, l2, llc, bw = hkg.hkg_remap_model(g, g, int(r["W"]), int(r["C"]), 256 * n * 2)
        assert rc == hkg.HKG_OK and 0 <= l2 <= 1 and 0 <= llc <= 1
        assert bw == pytest.approx(17.05 * l2 + 5.99 * llc)
        got[(n, int(r["W"]), int(r["C"]))] = (l2, llc, bw, float(r["l2_pct"]), float(r["tflops"]))
    for (n, W, C), (l2, llc, bw, page_l2, tf) in got.items():
        if (n, W, C) != (9216, 1, 1):
            assert abs(100 * l2 - page_l2) <= 6.5, (n, W, C, l2, page_l2)
    rows = sorted((v for k, v in got.items() if k[0] == 14592), key=lambda v: v[4])
    assert [v[2] for v in rows] == sorted(v[2] for v in rows)


def test_remap_model_closed_forms():
    # one XCD round of a grid with a single tile column: every tile of an XCD
    # shares the one B panel, rows all differ -> L2 hit = 1 - (32 + 1) / 64
    rc, l2, llc, bw = hkg.hkg_remap_model(256, 1, 1, 1, 1 << 20)
    assert rc == hkg.HKG_OK and l2 == pytest.approx(1 - 33 / 64)
    # (8, 32) on a 32 x 32 grid: each XCD's 32 tiles form an 8 x 4 patch: 12 panels
    rc, l2, llc, bw = hkg.hkg_remap_model(32, 32, 8, 32, 4 << 20)
    assert l2 == pytest.approx(1 - 12 / 64)
    # a single tile: both panels miss
    rc, l2, llc, bw = hkg.hkg_remap_model(1, 1, 1, 1, 1 << 20)
    assert l2 == 0.0 and llc == 0.0
    assert hkg.hkg_remap_model(0, 4, 1, 1, 1, 32)[0] == hkg.HKG_ERR_SHAPE
    # grid sides whose product would wrap are refused before it is formed
    # (2^32 x 2^32 is 2^64, 0 modulo 2^64)
    for gm, gn in ((1 << 32, 1 << 32), (1 << 40, 2), (1 << 31, 1)):
        assert hkg.hkg_remap_model(gm, gn, 1, 1, 1 << 20)[0] == hkg.HKG_ERR_SHAPE
        assert hkg.hkg_remap_tile(gm, gn, 1, 1, 0)[0] == hkg.HKG_ERR_SHAPE
        assert hkg.hkg_remap_tiles_device(gm, gn, 1, 1, FAKE, None) == hkg.HKG_ERR_SHAPE
    # a panel size too large for the last-level cache term does not wrap it:
    # no panel stays cached between rounds, as for any size above the cache
    rc, l2, llc_big, bw = hkg.hkg_remap_model(32, 32, 8, 32, (1 << 62) + 1)
    rc2, l2b, llc_huge, bw2 = hkg.hkg_remap_model(32, 32, 8, 32, 1 << 30)
    assert rc == rc2 == hkg.HKG_OK and llc_big == llc_huge and l2 == l2b
    assert hkg.hkg_remap_model(4, 4, 0, 1, 1, 32)[0] == hkg.HKG_ERR_SHAPE


def test_remap_candidates_are_the_model_ranked_orders():
    """hkg_remap_candidates: every clamped, distinct (W, C) of the default
    schedule's grid, best first by the model's Eq. 1 bandwidth, each entry equal
    to hkg_remap_model for that order."""
    for M, N, K, dt, tile, per in ((14592, 14592, 14592, 0, 256, 32), (8192, 8192, 8192, 1, 256, 32),
                                   (2048, 2048, 2048, 0, 128, 64), (16384, 14336, 4096, 0, 256, 32),
                                   (3072, 3072, 1024, 0, 192, 32)):
        rc, L, n = hkg.hkg_remap_candidates(M, N, K, dt)
        assert rc == hkg.HKG_OK and n == len(L) and 0 < n <= 48
        assert len(set((w, c) for w, c, _ in L)) == n
        bws = [b for _, _, b in L]
        assert bws == sorted(bws, reverse=True)
        Gm, Gn = -(-M // tile), -(-N // tile)
        elem = 2 if dt == 0 else 1
        for w, c, b in L:
            assert 1 <= w <= Gm and 1 <= c
            rc, l2, llc, bw = hkg.hkg_remap_model(Gm, Gn, w, c, tile * K * elem, per)
            assert rc == hkg.HKG_OK and bw == pytest.approx(b)
        # every enumerated window height, clamped to the grid's tile rows, occurs
        assert set(min(w, Gm) for w in (1, 2, 4, 8, 16, 32)) == set(w for w, _, _ in L)
    # at 14592 the top order is the one the measured rule picks there
    rc, L, n = hkg.hkg_remap_candidates(14592, 14592, 14592, 0)
    assert L[0][:2] == (16, 4) and hkg.hkg_default_remap(14592, 14592, 14592, 0)[1:] == (16, 4)
    # truncation, empty shapes, bad input
    rc, L, n = hkg.hkg_remap_candidates(8192, 8192, 8192, 0, 3)
    assert rc == hkg.HKG_OK and len(L) == 3 and n > 3
    assert hkg.hkg_remap_candidates(0, 100, 64, 0)[::2] == (hkg.HKG_OK, 0)
    assert hkg.hkg_remap_candidates(100, 100, 60, 1)[0] == hkg.HKG_ERR_SHAPE
    assert hkg.hkg_remap_candidates(100, 100, 64, 3)[0] == hkg.HKG_ERR_SHAPE
    n = ctypes.c_int32()
    assert hkg.load().hkg_remap_candidates(100, 100, 64, 0, 4, None, None, None,
                                           ctypes.byref(n)) == hkg.HKG_ERR_NULL
    assert hkg.load().hkg_remap_candidates(100, 100, 64, 0, 0, None, None, None,
                                           ctypes.byref(n)) == hkg.HKG_OK and n.value > 0


def test_tune_remap_validates_before_any_hip_call():
    best = hkg.hkg_gemm_opts()
    lib = hkg.load()
    T = lambda *a: hkg.hkg_tune_remap(*a)[0]
    assert lib.hkg_tune_remap(256, 256, 256, 0, FAKE, FB, FC, 5, None, None, None, None, None,
                              None) == hkg.HKG_ERR_NULL
    ms = ctypes.c_float()
    assert lib.hkg_tune_remap(256, 256, 256, 0, FAKE, FB, FC, 5, ctypes.byref(best), None, None,
                              ctypes.byref(ms), None, None) == hkg.HKG_ERR_NULL   # partial report
    assert T(256, 256, 256, 2, FAKE, FB, FC, 5, best, None) == hkg.HKG_ERR_SHAPE   # MXFP8: tune as e4m3
    assert T(256, 256, 255, 0, FAKE, FB, FC, 5, best, None) == hkg.HKG_ERR_SHAPE
    assert T(256, 256, 256, 0, None, FB, FC, 5, best, None) == hkg.HKG_ERR_NULL
    assert T(256, 256, 256, 0, FAKE + 8, FB, FC, 5, best, None) == hkg.HKG_ERR_ALIGN
    assert T(256, 256, 256, 0, FAKE, FB, FAKE, 5, best, None) == hkg.HKG_ERR_OVERLAP
    assert T(256, 256, 256, 0, FAKE, FB, FC, 0, best, None) == hkg.HKG_ERR_OPTS
    assert T(256, 256, 256, 1, FAKE, FB, FC, 1001, best, None) == hkg.HKG_ERR_OPTS
    # an empty product launches nothing and returns the defaults
    best.remap = 7
    rc, ms, tried = hkg.hkg_tune_remap(0, 256, 256, 0, None, None, None, 5, best, None)
    assert rc == hkg.HKG_OK and ms == 0.0 and best.remap == hkg.HKG_REMAP_DEFAULT and tried == []


def test_tune_remap_without_a_gfx950_is_a_device_error():
    """Valid arguments reach the device check, which fails without a gfx950, and
    `best` stays as it was."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    best = hkg.make_opts(remap=hkg.HKG_REMAP_XCD, W=3, C=5)
    rc, ms, tried = hkg.hkg_tune_remap(256, 256, 256, 0, FAKE, FB, FC, 5, best, None)
    assert rc == hkg.HKG_ERR_DEVICE and tried == []
    assert (best.remap, best.W, best.C) == (hkg.HKG_REMAP_XCD, 3, 5)


def test_row_pitches_validated_before_launch():
    """lda / ldb / ldc: 0 = dense; below the row's extent or negative ->
    HKG_ERR_OPTS; operand rows not 16-byte aligned -> HKG_ERR_ALIGN; panels past
    the 32-bit range -> HKG_ERR_SIZE; overlap checks span first to last element.
    Valid layouts reach the device check (HKG_ERR_DEVICE without a gfx950)."""
    M, N, K = 300, 200, 64
    G = lambda **kw: hkg.hkg_gemm_bf16_ex(M, N, K, FAKE, FB, FC, None, None, hkg.make_opts(**kw))
    F = lambda **kw: hkg.hkg_gemm_fp8_ex(M, N, K, FAKE, FB, 1.0, 1.0, FC, None, None,
                                         hkg.make_opts(**kw))
    assert G(lda=63) == hkg.HKG_ERR_OPTS and G(ldb=32) == hkg.HKG_ERR_OPTS
    assert G(ldc=199) == hkg.HKG_ERR_OPTS and G(lda=-64) == hkg.HKG_ERR_OPTS
    assert G(lda=68) == hkg.HKG_ERR_ALIGN            # 136-byte rows
    assert F(ldb=72) == hkg.HKG_ERR_ALIGN and F(ldb=80) in (hkg.HKG_OK, hkg.HKG_ERR_DEVICE)
    assert G(lda=1 << 22) == hkg.HKG_ERR_SIZE          # 256 rows x 8 MiB
    # a pitched C reaches further: C at FC with ldc 4096 spans 299 * 8 KiB + 400 B
    far = FC + 299 * 8192
    assert hkg.hkg_gemm_bf16_ex(M, N, K, FAKE, far, FC, None, None,
                                hkg.make_opts(ldc=4096)) == hkg.HKG_ERR_OVERLAP
    assert hkg.hkg_gemm_bf16_ex(M, N, K, FAKE, far + 512, FC, None, None,
                                hkg.make_opts(ldc=4096)) != hkg.HKG_ERR_OVERLAP
    try:
        import torch
        gpu = torch.cuda.is_available()
    except ImportError:
        gpu = False
    if not gpu:
        for kw in (dict(lda=64), dict(lda=72, ldb=128, ldc=256), dict(ldc=201)):
            assert G(**kw) == hkg.HKG_ERR_DEVICE, kw
    # pitches whose byte size would wrap a 64-bit product are refused, not
    # wrapped into range (256 x 2^56 x 2 bytes is 2^65)
    for big in (1 << 56, 1 << 60, (1 << 63) - 16):
        assert G(lda=big) == hkg.HKG_ERR_SIZE and G(ldb=big) == hkg.HKG_ERR_SIZE, big
        assert G(ldc=big) == hkg.HKG_ERR_SIZE and F(ldb=big) == hkg.HKG_ERR_SIZE, big
        assert hkg.launch_plan(M, N, K, 0, hkg.make_opts(lda=big))[0] == hkg.HKG_ERR_SIZE
    assert G(lda=(1 << 63) - 1) == hkg.HKG_ERR_ALIGN
    # the plan takes the pitches into its size check too
    assert hkg.launch_plan(M, N, K, 0, hkg.make_opts(lda=1 << 22))[0] == hkg.HKG_ERR_SIZE
    assert hkg.launch_plan(M, N, K, 0, hkg.make_opts(lda=63))[0] == hkg.HKG_ERR_OPTS
    assert hkg.launch_plan(M, N, K, 0, hkg.make_opts(lda=128))[0] == hkg.HKG_OK


def test_header_is_c99_and_a_c_caller_links(tmp_path):
    """include/hkg.h compiles as C99 with -Wall -Wextra -Werror, and a plain C
    program using it (tests/c/gemm_c_api.c) links against libhkg.so."""
    import importlib.util
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    spec = importlib.util.spec_from_file_location("c_api_build", os.path.join(ROOT, "tests", "c",
                                                                               "build.py"))
    c_api = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(c_api)
    out = str(tmp_path / "gemm_c_api")
    res = subprocess.run(c_api.command(out), capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert os.path.exists(out)
