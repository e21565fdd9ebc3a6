"""GPU parity of the MXFP8 path (hkg_mx_pack_scales + hkg_gemm_mxfp8) against
the oracle, through the C ABI (needs a gfx950 GPU).

MXFP8 follows the OCP Microscaling Formats v1.0 encoding: e4m3 elements and one
E8M0 scale per 32 consecutive elements along K.  The packed scale layout is
checked against its definition in include/hkg.h; small-integer cases are exact
in fp32 and compared bit for bit; N(0,1) cases use the (i)-(iii) acceptance of
tests/_parity.py."""
import sys

import numpy as np
import pytest

import oracle
from dense_gemm_fp8_amd import synth

from _parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("no GPU", allow_module_level=True)

import dense_gemm_fp8_amd as hkg  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def packed_layout(S, operand, K):
    """The packed scale bytes as include/hkg.h defines them (numpy, host)."""
    rows = S.shape[0]
    groups, nk = -(-rows // 128), -(-K // 128)
    out = np.full((groups, nk, 64, 8), 127, dtype=np.uint8)
    for l in range(64):
        x, q = l & 15, l >> 4
        for e in range(8):
            if operand == hkg.HKG_MX_OPERAND_A:
                rho = 16 * e + x
            else:
                rho = 32 * (e >> 1) + 4 * (e & 1) + (x & 3) + 8 * (x >> 2)
            r = 128 * np.arange(groups)[:, None] + rho                 # [g, 1]
            blk = 4 * np.arange(nk)[None, :] + q                       # [1, t]
            ok = (r < rows) & (blk < K // 32)
            vals = S[np.minimum(r, rows - 1), np.minimum(blk, K // 32 - 1)]
            out[:, :, l, e] = np.where(ok, vals, 127)
    return out.reshape(-1)


def run_mx(A, SA, B, SB, opts=None, want_f32=True):
    M, K = A.shape
    N = B.shape[0]
    pa = hkg.mx_pack_scales(_dev(SA), hkg.HKG_MX_OPERAND_A)
    pb = hkg.mx_pack_scales(_dev(SB), hkg.HKG_MX_OPERAND_B)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Cf = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") if want_f32 else None
    hkg.gemm_mxfp8(_dev(A), _dev(B), pa, pb, C, Cf, opts=opts)
    torch.cuda.synchronize()
    cb = C.view(torch.int16).cpu().numpy().view(np.uint16)
    return cb, (Cf.cpu().numpy() if want_f32 else None)


@pytest.mark.parametrize("rows,K", [(1, 32), (128, 128), (130, 160), (256, 1024), (300, 96),
                                    (1000, 544)])
@pytest.mark.parametrize("operand", [0, 1])
def test_pack_layout(rows, K, operand):
    _say("mx pack rows=%d K=%d operand=%d" % (rows, K, operand))
    g = np.random.Generator(np.random.PCG64(9300 + rows + K + operand))
    S = g.integers(0, 255, size=(rows, K // 32), dtype=np.uint8)
    packed = hkg.mx_pack_scales(_dev(S), operand)
    torch.cuda.synchronize()
    n = hkg.hkg_mx_packed_scale_bytes(rows, K)
    np.testing.assert_array_equal(packed[:n].cpu().numpy(), packed_layout(S, operand, K))


SHAPES_EXACT = [(256, 256, 128), (512, 768, 384), (256, 256, 32), (256, 256, 64), (256, 256, 96),
                (300, 260, 96), (257, 1, 32), (1, 513, 160), (1000, 777, 544), (640, 384, 2048)]


# both tiles of the 4-wave kernel (the default picks 128 x 128 for these small grids)
TILES = [hkg.HKG_SCHED_INTERLEAVE, hkg.HKG_SCHED_INTERLEAVE_128]
TILE_IDS = ["tile256", "tile128"]


@pytest.mark.parametrize("sched", TILES, ids=TILE_IDS)
@pytest.mark.parametrize("M,N,K", SHAPES_EXACT)
def test_small_integer_blocks_bit_exact(M, N, K, sched):
    # elements in [-2, 2], scales 2^-2..2^2: every product and partial sum is exact in fp32
    _say("mx ints %dx%dx%d sched=%d" % (M, N, K, sched))
    A, SA = synth.small_int_mx(9310 + K, M, K)
    B, SB = synth.small_int_mx(9320 + K, N, K)
    cb, cf = run_mx(A, SA, B, SB, opts=hkg.make_opts(schedule=sched))
    want = oracle.gemm_mxfp8(A, B, SA, SB)
    np.testing.assert_array_equal(cf.astype(np.float64), want)
    np.testing.assert_array_equal(cb, oracle.bf16_round(want))


def test_long_k_exact():
    """K of about 2^20 (8193 K steps, the last one partial and masked): scale
    and element offsets reach megabytes.  Elements in {-1, 0, 1} with unit
    block scales keep every partial sum an integer below 2^24, so the fp32
    copy is exact in any order; both tile kernels, sampled outputs."""
    M, N, K = 300, 260, (1 << 20) + 32
    _say("mx long K %dx%dx%d" % (M, N, K))
    A, SA = synth.small_int_mx(9397, M, K, -1, 1, 0, 0)
    B, SB = synth.small_int_mx(9398, N, K, -1, 1, 0, 0)
    pm, pn = synth.sample_pairs(9399, M, N, 300)
    want = oracle.gemm_mxfp8_pairs(A, B, SA, SB, pm, pn)
    assert np.all(want == np.round(want)) and np.abs(want).max() < 1 << 24
    for opts in (None, hkg.make_opts(schedule=hkg.HKG_SCHED_INTERLEAVE)):
        cb, cf = run_mx(A, SA, B, SB, opts=opts)
        np.testing.assert_array_equal(cf[pm, pn].astype(np.float64), want)
        np.testing.assert_array_equal(cb[pm, pn], oracle.bf16_round(want))


def test_max_k_exact():
    """The largest MXFP8 K the entry point accepts, 2^23 - 32 (a 256-row e4m3
    panel just under 2 GiB; one more block is refused), at 257 x 257.
    Elements in {-1, 0, 1} with block scales 2^-1, 2^0 or 2^1 make every
    product one of +-1/4 ... +-4, inside one MFMA's exact window, and every
    partial sum a multiple of 1/4 far below 2^22: the fp32 copy is exact and
    is compared bit for bit on sampled outputs of both tile kernels."""
    import time
    M = N = 257
    K = (1 << 23) - 32
    assert hkg.launch_plan(M, N, K + 32, 2)[0] == hkg.HKG_ERR_SIZE
    assert hkg.launch_plan(M, N, K, 2)[0] == hkg.HKG_OK
    _say("mx max K %dx%dx%d" % (M, N, K))
    t0 = time.time()
    A, B = synth.ternary_long(9391, M, K, "fp8"), synth.ternary_long(9392, N, K, "fp8")
    SA, SB = synth.e8m0_near_one(9393, M, K // 32), synth.e8m0_near_one(9394, N, K // 32)
    pm, pn = synth.sample_pairs(9395, M, N, 150)
    want = oracle.gemm_mxfp8_pairs(A, B, SA, SB, pm, pn)
    assert np.all(want * 4 == np.round(want * 4)) and np.abs(want).max() < 1 << 22
    pa = hkg.mx_pack_scales(_dev(SA), hkg.HKG_MX_OPERAND_A)
    pb = hkg.mx_pack_scales(_dev(SB), hkg.HKG_MX_OPERAND_B)
    dA, dB = _dev(A), _dev(B)
    del A, B
    _say("  inputs and oracle: %.1f s" % (time.time() - t0))
    for opts in (None, hkg.make_opts(schedule=hkg.HKG_SCHED_INTERLEAVE)):
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        Cf = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        hkg.gemm_mxfp8(dA, dB, pa, pb, C, Cf, opts=opts)
        torch.cuda.synchronize()
        cb = C.view(torch.int16).cpu().numpy().view(np.uint16)
        cf = Cf.cpu().numpy()
        np.testing.assert_array_equal(cf[pm, pn].astype(np.float64), want)
        np.testing.assert_array_equal(cb[pm, pn], oracle.bf16_round(want))
    _say("  done: %.1f s" % (time.time() - t0))


def test_unit_scales_equal_per_tensor_fp8():
    _say("mx unit scales vs fp8")
    M, N, K = 512, 512, 512
    A = synth.small_int_e4m3(9330, M, K)
    B = synth.small_int_e4m3(9331, N, K)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    cb, cf = run_mx(A, ones_a, B, ones_b)
    C8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Cf8 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    hkg.gemm_fp8(_dev(A), _dev(B), 1.0, 1.0, C8, Cf8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cf, Cf8.cpu().numpy())
    np.testing.assert_array_equal(cb, C8.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("sched", TILES, ids=TILE_IDS)
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (512, 768, 640), (1024, 512, 1536),
                                   (700, 900, 1056)])
def test_random_matches_oracle(M, N, K, sched):
    _say("mx random %dx%dx%d sched=%d" % (M, N, K, sched))
    A, SA = synth.mx_quantize(synth.normal_f32(9340 + K, M, K))
    B, SB = synth.mx_quantize(synth.normal_f32(9350 + K, N, K))
    cb, cf = run_mx(A, SA, B, SB, opts=hkg.make_opts(schedule=sched))
    check(oracle.gemm_mxfp8(A, B, SA, SB), cf, cb, K, "mxfp8 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("d", [-60, -13, 1, 29, 50])
def test_uniform_scale_shift_is_exact(d):
    # every scale + d multiplies every product by 2^(2d): exact while fp32 holds the sums
    # (|C| < 2^15 here, so 2^(2d) stays within 2^-120..2^100)
    _say("mx scale shift %d" % d)
    M, N, K = 256, 512, 384
    A, SA = synth.small_int_mx(9395, M, K)
    B, SB = synth.small_int_mx(9396, N, K)
    _, base = run_mx(A, SA, B, SB)
    SA2 = (SA.astype(np.int32) + d).astype(np.uint8)
    SB2 = (SB.astype(np.int32) + d).astype(np.uint8)
    cb, cf = run_mx(A, SA2, B, SB2)
    np.testing.assert_array_equal(cf.astype(np.float64), base.astype(np.float64) * 2.0 ** (2 * d))
    np.testing.assert_array_equal(cb, oracle.bf16_round(oracle.gemm_mxfp8(A, B, SA2, SB2)))


def test_wide_scale_range_matches_oracle():
    # block scales spread over 2^-40..2^40, so products inside one MFMA can be
    # far apart: the hardware aligns them to the largest and keeps ~13 bits
    # below it, so the bound is relative to the sum of magnitudes
    _say("mx wide scales")
    M, N, K = 256, 256, 512
    g = np.random.Generator(np.random.PCG64(9360))
    A, _ = synth.mx_quantize(synth.normal_f32(9361, M, K))
    B, _ = synth.mx_quantize(synth.normal_f32(9362, N, K))
    SA = g.integers(127 - 40, 127 + 41, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(127 - 40, 127 + 41, size=(N, K // 32)).astype(np.uint8)
    cb, cf = run_mx(A, SA, B, SB)
    ref = oracle.gemm_mxfp8(A, B, SA, SB)
    # magnitude scale of each output: sum over k of |a||b| (fp64, via the oracle on |codes|)
    mag = oracle.gemm_mxfp8(A & 0x7F, B & 0x7F, SA, SB)
    assert np.all(np.abs(cf.astype(np.float64) - ref) <= 2.0 ** -6 * mag + 1e-30)


def test_full_size_every_entry():
    """MXFP8 8192^3 (N(0,1) quantised per 32-element block), EVERY output
    entry, against the oracle's full-grid route (exact MXFP8 decoding, BLAS
    fp64 product, row blocks); (i)-(iii) of tests/_parity.py on each entry.
    The bench's launch (no fp32 copy) and the validation launch agree bit for
    bit, and (ii) holds on every entry on the device."""
    from oracle import dense
    w = synth.MX_WORKLOAD
    _say("mx full-size %s: inputs" % w.name)
    A, B, SA, SB = synth.make_inputs(w)
    dA, dB = _dev(A), _dev(B)
    pa = hkg.mx_pack_scales(_dev(SA), hkg.HKG_MX_OPERAND_A)
    pb = hkg.mx_pack_scales(_dev(SB), hkg.HKG_MX_OPERAND_B)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    Cf = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    _say("mx full-size: launch")
    hkg.gemm_mxfp8(dA, dB, pa, pb, C)
    hkg.gemm_mxfp8(dA, dB, pa, pb, C2, Cf)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    assert torch.equal(Cf.to(torch.bfloat16).view(torch.int16), C.view(torch.int16))
    cb = C.view(torch.int16).cpu().numpy().view(np.uint16)
    cf = Cf.cpu().numpy()
    del dA, dB, C, C2, Cf
    torch.cuda.empty_cache()
    ref = dense.DenseReference("mxfp8", A, B, SA, SB)
    worst, checked = 0.0, 0
    for r0, r1 in ref.row_blocks():
        d = check(ref.rows(r0, r1), cf[r0:r1], cb[r0:r1], w.K, "%s rows %d..%d" % (w.name, r0, r1))
        worst, checked = max(worst, d["max_abs_err"]), checked + d["checked"]
    assert checked == w.M * w.N
    _say("mx full-size: every entry, max|d| %.3g (tol %.3g)" % (worst, d["tol"]))


@pytest.mark.parametrize("M,N,K", [(300, 260, 96), (257, 1, 32)])
@pytest.mark.parametrize("sched", TILES, ids=TILE_IDS)
def test_no_stray_writes(M, N, K, sched):
    _say("mx canary %dx%dx%d sched=%d" % (M, N, K, sched))
    A, SA = synth.small_int_mx(9380, M, K)
    B, SB = synth.small_int_mx(9381, N, K)
    pa = hkg.mx_pack_scales(_dev(SA), hkg.HKG_MX_OPERAND_A)
    pb = hkg.mx_pack_scales(_dev(SB), hkg.HKG_MX_OPERAND_B)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), 12345, dtype=torch.int16, device="cuda")
    C = buf[pad:pad + M * N].view(torch.bfloat16).view(M, N)
    hkg.gemm_mxfp8(_dev(A), _dev(B), pa, pb, C, opts=hkg.make_opts(schedule=sched))
    torch.cuda.synchronize()
    assert (buf[:pad] == 12345).all() and (buf[pad + M * N:] == 12345).all()


@pytest.mark.parametrize("sched", [hkg.HKG_SCHED_PINGPONG, hkg.HKG_SCHED_LOCKSTEP,
                                   hkg.HKG_SCHED_INTERLEAVE_192],
                         ids=["pingpong", "lockstep", "interleave192"])
def test_unsupported_schedules_rejected(sched):
    """Only the 4-wave kernel on 256 x 256 or 128 x 128 tiles has the
    block-scaled path."""
    _say("mx rejected schedule %d" % sched)
    A, SA = synth.small_int_mx(9390, 256, 64)
    pa = hkg.mx_pack_scales(_dev(SA), hkg.HKG_MX_OPERAND_A)
    pb = hkg.mx_pack_scales(_dev(SA), hkg.HKG_MX_OPERAND_B)
    C = torch.full((256, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hkg.HkgError):
        hkg.gemm_mxfp8(_dev(A), _dev(A), pa, pb, C, opts=hkg.make_opts(schedule=sched))
    torch.cuda.synchronize()
    assert (C.float() == 3.0).all()


def test_split_default_launch_identical_to_single_launch():
    """MXFP8's default launch splits a partial last round like the other
    dtypes (whole rounds on 256 x 256 tiles, the rest on 128 x 128 reading
    the same packed scales); the result equals one 256 x 256 launch."""
    M, N, K = 4352, 4352, 288
    _say("mx split launch %dx%dx%d" % (M, N, K))
    rc, plan = hkg.launch_plan(M, N, K, 2)
    assert rc == hkg.HKG_OK and [d["tile"] for d in plan] == [256, 128]
    A, SA = synth.mx_quantize(synth.normal_f32(9420, M, K))
    B, SB = synth.mx_quantize(synth.normal_f32(9421, N, K))
    split = run_mx(A, SA, B, SB)
    one = run_mx(A, SA, B, SB, opts=hkg.make_opts(schedule=hkg.HKG_SCHED_INTERLEAVE))
    np.testing.assert_array_equal(split[1].view(np.uint32), one[1].view(np.uint32))
    np.testing.assert_array_equal(split[0], one[0])


def test_random_shapes_default_launch_exact():
    """10 seeded ragged shapes (M, N up to 4700, K = 32, 64 or 96)
    through the default MXFP8 launch, which among them takes both tile edges and
    a split launch; small-integer blocks make every sum exact."""
    rng = np.random.default_rng(7879)
    tiles, splits = set(), 0
    for i in range(10):
        M, N = (int(v) for v in rng.integers(1, 4700, 2))
        K = 32 * int(rng.integers(1, 4))
        rc, plan = hkg.launch_plan(M, N, K, 2)
        assert rc == hkg.HKG_OK
        tiles |= {d["tile"] for d in plan}
        splits += len(plan) == 2
        _say("mx random shape %d: %dx%dx%d plan %s" % (i, M, N, K,
                                                     [(d["tile"], d["rows"]) for d in plan]))
        A, SA = synth.small_int_mx(7200 + i, M, K)
        B, SB = synth.small_int_mx(7300 + i, N, K)
        cb, cf = run_mx(A, SA, B, SB)
        want = oracle.gemm_mxfp8(A, B, SA, SB)
        np.testing.assert_array_equal(cf.astype(np.float64), want)
        np.testing.assert_array_equal(cb, oracle.bf16_round(want))
    assert tiles == {128, 256} and splits >= 1
