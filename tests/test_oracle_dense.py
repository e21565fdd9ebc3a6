"""Pins of the oracle's full-grid route (oracle/dense.py) against things other
than itself.

The route decodes inputs exactly into fp64 and lets the BLAS fp64 matrix
product form the sums.  The checks are chosen so that a plausible mistake in
it (a wrong decode, an untransposed or swapped operand, a dropped scale, a
wrong row block) fails at least one of them:

* brute force over exact rationals on tiny shapes (bf16: within the fp64
  summation bound; e4m3: exactly, since e4m3 sums are exact in fp64);
* small-integer inputs against an int64 matrix product;
* closed forms: all-ones gives K, identity operands give the other operand;
* decoders against torch's own bfloat16 / float8_e4m3fn conversions;
* the plain k-ascending oracle (oracle.c, itself pinned in test_oracle_gemm):
  e4m3 results equal bit for bit, bf16 results within the summation bound;
* row blocks reassemble the whole grid bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import dense
from dense_gemm_fp8_amd import synth


def _exact(av, bv):
    M, K = av.shape
    N = bv.shape[0]
    return [[sum((Fraction(float(av[m, k])) * Fraction(float(bv[n, k])) for k in range(K)),
                 Fraction(0)) for n in range(N)] for m in range(M)]


def test_decoders_match_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = dense.decode_bf16(bits)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    codes = np.arange(256, dtype=np.uint8)
    want8 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got8 = dense.decode_e4m3(codes)
    same8 = (got8 == want8) | (np.isnan(got8) & np.isnan(want8))
    assert same8.all()


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (9, 4, 33), (5, 6, 64)])
def test_bf16_brute_force(M, N, K):
    A = synth.f32_to_bf16_bits(synth.normal_f32(9031 + M, M, K))
    B = synth.f32_to_bf16_bits(synth.normal_f32(9032 + N, N, K))
    got = dense.gemm_bf16(A, B)
    av, bv = synth.bf16_bits_to_f32(A).astype(np.float64), synth.bf16_bits_to_f32(B).astype(np.float64)
    ex = _exact(av, bv)
    bound = np.abs(av) @ np.abs(bv).T * (K * 2.0 ** -52)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(got[m, n])) - ex[m][n]) <= Fraction(float(bound[m, n])) + Fraction(1, 10 ** 300)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (4, 3, 17), (7, 9, 128)])
def test_fp8_brute_force_exact(M, N, K):
    torch = pytest.importorskip("torch")
    A, sa = synth.e4m3_quantize(synth.normal_f32(9041 + M, M, K))
    B, sb = synth.e4m3_quantize(synth.normal_f32(9042 + N, N, K))
    dec = lambda q: torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ex = _exact(dec(A), dec(B))
    unscaled = dense.gemm_fp8(A, B, 1.0, 1.0)
    scaled = dense.gemm_fp8(A, B, sa, sb)
    s = float(sa) * float(sb)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(unscaled[m, n])) == ex[m][n]        # the sum is exact
            assert scaled[m, n] == float(unscaled[m, n]) * s            # one fp64 scale multiply


def test_small_integers_exact():
    M, N, K = 70, 90, 300
    A = synth.small_int_bf16(9051, M, K)
    B = synth.small_int_bf16(9052, N, K)
    ai = synth.bf16_bits_to_f32(A).astype(np.int64)
    bi = synth.bf16_bits_to_f32(B).astype(np.int64)
    np.testing.assert_array_equal(dense.gemm_bf16(A, B), (ai @ bi.T).astype(np.float64))
    A8 = synth.small_int_e4m3(9053, M, K)
    B8 = synth.small_int_e4m3(9054, N, K)
    torch = pytest.importorskip("torch")
    dec = lambda q: torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = (dec(A8).astype(np.int64) @ dec(B8).astype(np.int64).T).astype(np.float64)
    np.testing.assert_array_equal(dense.gemm_fp8(A8, B8, 1.0, 1.0), want)


def test_closed_forms():
    K = 4096
    one = np.full((3, K), 0x3F80, dtype=np.uint16)
    np.testing.assert_array_equal(dense.gemm_bf16(one, one[:2]), np.full((3, 2), float(K)))
    one8 = np.full((2, K), 0x38, dtype=np.uint8)
    np.testing.assert_array_equal(dense.gemm_fp8(one8, one8, 1.0, 1.0), np.full((2, 2), float(K)))
    k = 40
    eye = synth.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    B = synth.f32_to_bf16_bits(synth.normal_f32(9055, 11, k))
    np.testing.assert_array_equal(dense.gemm_bf16(eye, B), synth.bf16_bits_to_f32(B).T)
    np.testing.assert_array_equal(dense.gemm_bf16(B, eye), synth.bf16_bits_to_f32(B))


def test_matches_plain_oracle():
    M, N, K = 200, 150, 1040
    A8, sa = synth.e4m3_quantize(synth.normal_f32(9061, M, K))
    B8, sb = synth.e4m3_quantize(synth.normal_f32(9062, N, K))
    # e4m3: both routes are exact sums, then the same fp64 scale multiply
    np.testing.assert_array_equal(dense.gemm_fp8(A8, B8, sa, sb), oracle.gemm_fp8(A8, B8, sa, sb))
    A = synth.f32_to_bf16_bits(synth.normal_f32(9063, M, K))
    B = synth.f32_to_bf16_bits(synth.normal_f32(9064, N, K))
    av, bv = synth.bf16_bits_to_f32(A).astype(np.float64), synth.bf16_bits_to_f32(B).astype(np.float64)
    bound = np.abs(av) @ np.abs(bv).T * (2 * K * 2.0 ** -53)
    assert np.all(np.abs(dense.gemm_bf16(A, B) - oracle.gemm_bf16(A, B)) <= bound)


def test_row_blocks_reassemble():
    M, N, K = 97, 64, 72
    A = synth.f32_to_bf16_bits(synth.normal_f32(9071, M, K))
    B = synth.f32_to_bf16_bits(synth.normal_f32(9072, N, K))
    ref = dense.DenseReference("bf16", A, B)
    blocks = ref.row_blocks(max_flops=2.0 * N * K * 10)
    assert blocks[0] == (0, 10) and blocks[-1] == (90, 97)
    whole = ref.rows(0, M)
    np.testing.assert_array_equal(np.concatenate([ref.rows(a, b) for a, b in blocks]), whole)


def test_rejects_bad_inputs():
    with pytest.raises(TypeError):
        dense.DenseReference("bf16", np.zeros((2, 4), np.uint8), np.zeros((2, 4), np.uint8))
    with pytest.raises(ValueError):
        dense.DenseReference("fp8", np.zeros((2, 4), np.uint8), np.zeros((2, 5), np.uint8))
    with pytest.raises(ValueError):
        dense.DenseReference("fp16", np.zeros((2, 4), np.uint16), np.zeros((2, 4), np.uint16))


# ---- MXFP8 (e4m3 elements, one E8M0 scale per 32 along K) -------------------

def test_mxfp8_decoder_matches_torch_and_ldexp():
    torch = pytest.importorskip("torch")
    codes = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(8, 128)      # every code, 4 blocks a row
    scales = np.array([[0, 100, 127, 254], [1, 126, 128, 255]] * 4, dtype=np.uint8)
    got = dense.decode_mxfp8(codes, scales)
    e4 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.ldexp(e4, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    want[np.repeat(scales == 255, 32, axis=1)] = np.nan                      # E8M0 0xFF is NaN
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 5, 64), (4, 2, 96)])
def test_mxfp8_brute_force_exact(M, N, K):
    A, SA = synth.mx_quantize(synth.normal_f32(9081 + M, M, K))
    B, SB = synth.mx_quantize(synth.normal_f32(9082 + N, N, K))
    got = dense.gemm_mxfp8(A, B, SA, SB)
    tab = oracle.e4m3_table()
    for m in range(M):
        for n in range(N):
            ex = sum((Fraction(float(tab[A[m, k]])) * Fraction(2) ** (int(SA[m, k // 32]) - 127) *
                      Fraction(float(tab[B[n, k]])) * Fraction(2) ** (int(SB[n, k // 32]) - 127)
                      for k in range(K)), Fraction(0))
            assert Fraction(float(got[m, n])) == ex        # exact: K small, power-of-two scales


def test_mxfp8_matches_plain_oracle():
    M, N, K = 200, 150, 1024
    A, SA = synth.mx_quantize(synth.normal_f32(9091, M, K))
    B, SB = synth.mx_quantize(synth.normal_f32(9092, N, K))
    got, want = dense.gemm_mxfp8(A, B, SA, SB), oracle.gemm_mxfp8(A, B, SA, SB)
    av, bv = np.abs(dense.decode_mxfp8(A, SA)), np.abs(dense.decode_mxfp8(B, SB))
    assert np.all(np.abs(got - want) <= av @ bv.T * (2 * K * 2.0 ** -53))
    ref = dense.DenseReference("mxfp8", A, B, SA, SB)
    np.testing.assert_array_equal(np.concatenate([ref.rows(a, b) for a, b in
                                                  ref.row_blocks(max_flops=2.0 * N * K * 64)]), got)


def test_mxfp8_rejects_mismatched_scales():
    with pytest.raises(ValueError):
        dense.DenseReference("mxfp8", np.zeros((2, 64), np.uint8), np.zeros((3, 64), np.uint8),
                             np.zeros((2, 2), np.uint8), np.zeros((3, 1), np.uint8))
