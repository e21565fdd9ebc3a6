"""Pins of the MXFP8 oracle and of the MX quantiser (CPU only).

The reference follows the OCP Microscaling Formats specification v1.0: e4m3
elements with one E8M0 scale 2^(E-127) per 32 consecutive elements along K.
Each pin reaches the expected value by a route that does not go through the
oracle's C loop: torch's e4m3 decoding and numpy's matmul, exact rational
arithmetic, the per-tensor e4m3 oracle (pinned elsewhere) at unit scales, and
the effect of changing one block scale."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_fp8_amd import synth

torch = pytest.importorskip("torch")


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    """e4m3 codes -> float64 via torch's float8_e4m3fn dtype (independent decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return torch_e4m3(codes) * np.exp2(np.repeat(scales.astype(np.float64), 32, axis=1) - 127.0)


def test_e8m0_landmarks():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0_value(255))
    for e in range(255):
        assert oracle.e8m0_value(e) == 2.0 ** (e - 127)


def test_unit_scales_reduce_to_per_tensor_e4m3():
    A, _ = synth.mx_quantize(synth.normal_f32(9101, 7, 96))
    B, _ = synth.mx_quantize(synth.normal_f32(9102, 5, 96))
    ones_a = np.full((7, 3), 127, np.uint8)
    ones_b = np.full((5, 3), 127, np.uint8)
    np.testing.assert_array_equal(oracle.gemm_mxfp8(A, B, ones_a, ones_b),
                                  oracle.gemm_fp8(A, B, 1.0, 1.0))


def test_small_integer_blocks_equal_numpy_dequant_matmul():
    # integers in [-4, 4] times 2^-3..2^3: every product and sum is exact in fp64
    A, SA = synth.small_int_mx(9103, 33, 256, -4, 4, -3, 3)
    B, SB = synth.small_int_mx(9104, 17, 256, -4, 4, -3, 3)
    want = dequant(A, SA) @ dequant(B, SB).T
    np.testing.assert_array_equal(oracle.gemm_mxfp8(A, B, SA, SB), want)


def test_tiny_case_exact_rational():
    A, SA = synth.mx_quantize(synth.normal_f32(9105, 2, 64))
    B, SB = synth.mx_quantize(synth.normal_f32(9106, 3, 64))
    dec = {c: Fraction(float(v)) for c, v in enumerate(torch_e4m3(np.arange(256, dtype=np.uint8)))
           if not math.isnan(v)}
    got = oracle.gemm_mxfp8(A, B, SA, SB)
    for m in range(2):
        for n in range(3):
            s = Fraction(0)
            for k in range(64):
                sa = Fraction(2) ** (int(SA[m, k // 32]) - 127)
                sb = Fraction(2) ** (int(SB[n, k // 32]) - 127)
                s += dec[A[m, k]] * sa * dec[B[n, k]] * sb
            assert abs(Fraction(got[m, n]) - s) <= abs(s) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_one_block_scale_changes_one_block_of_one_row():
    A, SA = synth.small_int_mx(9107, 6, 128, -3, 3, -2, 2)
    B, SB = synth.small_int_mx(9108, 4, 128, -3, 3, -2, 2)
    base = oracle.gemm_mxfp8(A, B, SA, SB)
    m, b = 3, 2
    SA2 = SA.copy()
    SA2[m, b] += 1                                   # doubles block b of row m
    got = oracle.gemm_mxfp8(A, B, SA2, SB)
    part = dequant(A, SA)[m, 32 * b:32 * b + 32] @ dequant(B, SB)[:, 32 * b:32 * b + 32].T
    np.testing.assert_array_equal(got[m], base[m] + part)
    rows = [r for r in range(6) if r != m]
    np.testing.assert_array_equal(got[rows], base[rows])


def test_pairs_match_full_grid():
    A, SA = synth.mx_quantize(synth.normal_f32(9109, 40, 160))
    B, SB = synth.mx_quantize(synth.normal_f32(9110, 30, 160))
    full = oracle.gemm_mxfp8(A, B, SA, SB)
    pm, pn = synth.sample_pairs(9111, 40, 30, 50, tile=16)
    np.testing.assert_array_equal(oracle.gemm_mxfp8_pairs(A, B, SA, SB, pm, pn), full[pm, pn])


def test_rejects_k_not_multiple_of_32():
    A = np.zeros((2, 48), np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_mxfp8(A, A, np.zeros((2, 1), np.uint8), np.zeros((2, 1), np.uint8))


# ---------------------------------------------------------------- quantiser ----

def test_mx_scale_is_floor_log2_amax_minus_8():
    x = synth.normal_f32(9112, 16, 256) * np.float32(3.7)
    _, S = synth.mx_quantize(x)
    for r in range(16):
        for b in range(8):
            amax = float(np.max(np.abs(x[r, 32 * b:32 * b + 32])))
            assert int(S[r, b]) == math.floor(math.log2(amax)) - 8 + 127


def test_mx_block_maximum_lands_in_top_binade_or_saturates():
    x = synth.normal_f32(9113, 32, 512)
    C, S = synth.mx_quantize(x)
    dec = np.abs(torch_e4m3(C)).reshape(32, 16, 32)
    top = dec.max(axis=2)
    assert np.all(top >= 256.0) and np.all(top <= 448.0)


def test_mx_dequantised_error_within_half_ulp():
    x = synth.normal_f32(9114, 64, 256).astype(np.float64)
    C, S = synth.mx_quantize(x.astype(np.float32))
    d = dequant(C, S)
    scale = np.exp2(np.repeat(S.astype(np.float64), 32, axis=1) - 127.0)
    y = np.abs(x) / scale                            # magnitude in element units
    normal = (y >= 2.0 ** -6) & (y <= 448.0)
    # e4m3 normals carry 3 fraction bits: rounding error <= 2^-4 relative
    assert np.all(np.abs(d - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4 + 1e-300)
    sub = y < 2.0 ** -6                               # subnormal step 2^-9
    assert np.all(np.abs(d - x)[sub] <= scale[sub] * 2.0 ** -10)
    sat = y > 448.0
    np.testing.assert_array_equal(np.abs(d[sat]), 448.0 * scale[sat])
    assert np.all(np.sign(d[x != 0]) * np.sign(x[x != 0]) >= 0)


def test_mx_zero_and_extreme_blocks():
    x = np.zeros((3, 64), np.float32)
    x[1, :32] = np.float32(2.0 ** 100)
    x[2, 32:] = np.float32(2.0 ** -140)              # shared exponent clamps at -127
    C, S = synth.mx_quantize(x)
    assert S[0, 0] == 127 and S[0, 1] == 127 and not C[0].any()
    assert S[1, 0] == 100 - 8 + 127
    assert S[2, 1] == 0
    np.testing.assert_array_equal(dequant(C, S)[1, :32], x[1, :32].astype(np.float64))
