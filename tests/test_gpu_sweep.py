"""Seeded random sweep of every launch option against the oracle (needs a gfx950
GPU): shapes with ragged edges, every schedule a dtype accepts, default /
row-major / explicit grid orders, row pitches on A, B and C, A and B in one
buffer, K = 0.  With small-integer operands (block scales powers of two) the
oracle's fp64 product is exact in fp32: C_f32 must equal it bit for bit, C
must be its round-to-nearest-even bf16, and the bytes between C's rows must
keep their canary.  With N(0,1) operands (quantised per tensor or per block
for e4m3) every entry must meet the acceptance rule (i)-(iii)."""
import sys

import numpy as np
import pytest

from dense_gemm_fp8_amd import synth
from oracle import dense
from oracle.parity import f32_to_bf16_rne

from _parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("no GPU", allow_module_level=True)

import dense_gemm_fp8_amd as hkg  # noqa: E402

CASES = 60
K_ALIGN = {"bf16": 8, "fp8": 16, "mxfp8": 32}
SCHEDULES = {"bf16": [0, 1, 2, 3, 4, 5], "fp8": [0, 1, 2, 3, 4, 5], "mxfp8": [0, 3, 4]}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dim(rng):
    """Small, near a multiple of the 256 tile, or anywhere up to 2600."""
    r = rng.random()
    if r < 0.3:
        return int(rng.integers(1, 300))
    if r < 0.6:
        return max(1, int(256 * rng.integers(1, 10) + rng.integers(-3, 4)))
    return int(rng.integers(1, 2600))


def _case(rng, dt):
    M, N = _dim(rng), _dim(rng)
    al = K_ALIGN[dt]
    K = 0 if rng.random() < 0.05 else al * int(rng.integers(1, 2048 // al + 1))
    sched = int(rng.choice(SCHEDULES[dt]))
    r = rng.random()
    if r < 0.5:
        o = dict(schedule=sched)
    elif r < 0.7:
        o = dict(schedule=sched, remap=hkg.HKG_REMAP_ROW_MAJOR)
    else:
        o = dict(schedule=sched, remap=hkg.HKG_REMAP_XCD, W=int(rng.integers(1, 65)),
                 C=int(rng.integers(1, 600)))
    step = 16 // (2 if dt == "bf16" else 1)          # pitches keep rows 16-byte aligned
    pa = step * int(rng.integers(1, 5)) if rng.random() < 0.4 else 0
    pb = step * int(rng.integers(1, 5)) if rng.random() < 0.4 else 0
    pc = int(rng.integers(1, 40)) if rng.random() < 0.3 else 0
    alias = dt != "mxfp8" and rng.random() < 0.15
    if alias:
        N = M
    return M, N, K, o, pa, pb, pc, alias, int(rng.integers(1, 1 << 30))


def _pitched(t, ld, fill):
    rows, cols = t.shape
    big = torch.full((rows, ld), fill, dtype=t.dtype, device="cuda")
    big[:, :cols] = t
    return big[:, :cols]


@pytest.mark.parametrize("dt", ["bf16", "fp8", "mxfp8"])
def test_random_launch_options_exact(dt):
    rng = np.random.default_rng({"bf16": 8101, "fp8": 8102, "mxfp8": 8103}[dt])
    for i in range(CASES):
        M, N, K, o, pa, pb, pc, alias, s = _case(rng, dt)
        _say("sweep %s %d: %dx%dx%d opts %s pads %d/%d/%d alias %s" % (dt, i, M, N, K, o, pa, pb,
                                                                      pc, alias))
        opts = hkg.make_opts(**o)
        if dt == "bf16":
            A = synth.small_int_bf16(s, M, K)
            B = A if alias else synth.small_int_bf16(s + 1, N, K)
            want = dense.gemm_bf16(A, B)
            dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).cuda()
            dB = None if alias else torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).cuda()
            fill = float("nan")
        elif dt == "fp8":
            A = synth.small_int_e4m3(s, M, K)
            B = A if alias else synth.small_int_e4m3(s + 1, N, K)
            sa, sb = (float(2.0 ** int(v)) for v in rng.integers(-3, 3, 2))
            want = dense.gemm_fp8(A, B, sa, sb)
            dA = torch.from_numpy(A).cuda()
            dB = None if alias else torch.from_numpy(B).cuda()
            fill = 0x7F                                  # an e4m3 NaN code
        else:
            A, SA = synth.small_int_mx(s, M, K)
            B, SB = synth.small_int_mx(s + 1, N, K)
            want = dense.gemm_mxfp8(A, B, SA, SB)
            dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
            pA = hkg.mx_pack_scales(torch.from_numpy(SA).cuda(), hkg.HKG_MX_OPERAND_A)
            pB = hkg.mx_pack_scales(torch.from_numpy(SB).cuda(), hkg.HKG_MX_OPERAND_B)
            fill = 0x7F
        assert np.all(np.abs(want) < 2.0 ** 24)          # exact in fp32
        if pa:
            dA = _pitched(dA, K + pa, fill)
        if alias:
            dB = dA
        elif pb:
            dB = _pitched(dB, K + pb, fill)
        canary = -1234.5
        bigC = torch.full((M, N + pc), canary, dtype=torch.bfloat16, device="cuda")
        bigF = torch.full((M, N + pc), canary, dtype=torch.float32, device="cuda")
        C, F = bigC[:, :N], bigF[:, :N]
        if dt == "bf16":
            hkg.gemm_bf16(dA, dB, C, F, opts=opts)
        elif dt == "fp8":
            hkg.gemm_fp8(dA, dB, sa, sb, C, F, opts=opts)
        else:
            hkg.gemm_mxfp8(dA, dB, pA, pB, C, F, opts=opts)
        torch.cuda.synchronize()
        w32 = want.astype(np.float32)
        np.testing.assert_array_equal(F.cpu().numpy().view(np.uint32), w32.view(np.uint32))
        got = C.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, f32_to_bf16_rne(w32))
        if pc:
            assert torch.all(bigC[:, N:] == canary) and torch.all(bigF[:, N:] == canary)


@pytest.mark.parametrize("dt", ["bf16", "fp8", "mxfp8"])
def test_random_launch_options_normal_inputs(dt):
    rng = np.random.default_rng({"bf16": 8201, "fp8": 8202, "mxfp8": 8203}[dt])
    for i in range(20):
        M, N, K, o, pa, pb, pc, alias, s = _case(rng, dt)
        M, N, K = min(M, 1500), (M if alias else min(N, 1500)), max(K_ALIGN[dt], min(K, 1024))
        _say("sweep N(0,1) %s %d: %dx%dx%d opts %s pads %d/%d/%d alias %s" % (
            dt, i, M, N, K, o, pa, pb, pc, alias))
        opts = hkg.make_opts(**o)
        x = synth.normal_f32(s, M, K)
        y = x if alias else synth.normal_f32(s + 1, N, K)
        if dt == "bf16":
            A, B = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(y)
            ref = dense.gemm_bf16(A, B)
            dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).cuda()
            dB = None if alias else torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).cuda()
            fill = float("nan")
        elif dt == "fp8":
            (A, sa), (B, sb) = synth.e4m3_quantize(x), synth.e4m3_quantize(y)
            sa, sb = float(sa), float(sb)
            ref = dense.gemm_fp8(A, B, sa, sb)
            dA = torch.from_numpy(A).cuda()
            dB = None if alias else torch.from_numpy(B).cuda()
            fill = 0x7F
        else:
            (A, SA), (B, SB) = synth.mx_quantize(x), synth.mx_quantize(y)
            ref = dense.gemm_mxfp8(A, B, SA, SB)
            dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
            pA = hkg.mx_pack_scales(torch.from_numpy(SA).cuda(), hkg.HKG_MX_OPERAND_A)
            pB = hkg.mx_pack_scales(torch.from_numpy(SB).cuda(), hkg.HKG_MX_OPERAND_B)
            fill = 0x7F
        if pa:
            dA = _pitched(dA, K + pa, fill)
        if alias:
            dB = dA
        elif pb:
            dB = _pitched(dB, K + pb, fill)
        C = torch.empty((M, N + pc), dtype=torch.bfloat16, device="cuda")[:, :N]
        F = torch.empty((M, N + pc), dtype=torch.float32, device="cuda")[:, :N]
        if dt == "bf16":
            hkg.gemm_bf16(dA, dB, C, F, opts=opts)
        elif dt == "fp8":
            hkg.gemm_fp8(dA, dB, sa, sb, C, F, opts=opts)
        else:
            hkg.gemm_mxfp8(dA, dB, pA, pB, C, F, opts=opts)
        torch.cuda.synchronize()
        check(ref, F.contiguous().cpu().numpy(),
              C.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), K,
              "%s case %d" % (dt, i))
