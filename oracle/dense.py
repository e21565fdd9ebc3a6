"""Full-grid route to the oracle's GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and bench.py's CPU-baseline leg may use this
module; the GPU library never does, and nothing here imports it.

It evaluates the same definition as oracle.c -- the plain GEMM of the
HipKittens L2 note, section 3 "Target operation" table (B used transposed, as
the mma_ABt calls of the section 7 / 9.2 listing descriptions show):

    ref[m][n] = sum_k a[m][k] * b[n][k]        (fp64; fp8: times sa * sb)

in two steps:
  1. decode every input element exactly into an fp64 matrix (bf16: the 16 bits
     are the upper half of an IEEE binary32 value; OCP e4m3: the oracle's own
     256-entry table, oracle_e4m3_value; MXFP8: that e4m3 value times the
     E8M0 scale 2^(E-127) of its 32-element block along K, oracle_e8m0_value,
     as the OCP Microscaling Formats v1.0 define the element's value);
  2. form the sums with the BLAS fp64 matrix product, a library primitive.

The BLAS adds the products in a blocked order, not k ascending.  That changes
nothing for e4m3: every product is a multiple of 2^-18 below 2^18 in
magnitude, so every partial sum over K < 2^17 terms is a multiple of 2^-18
below 2^35 and is exact in fp64 in any order -- the result equals oracle.c's
bit for bit.  For bf16 the products are exact and the two summation orders
differ by at most about K * 2^-53 * sum_k |a b|, many orders of magnitude below
the 1e-3 * sqrt(K) parity tolerance; MXFP8 products are exact too (a power of
two times an e4m3 product), and the same bound holds.  The pins in tests/test_oracle_dense.py
check both statements, and the closed forms, against things other than this
module.

It exists because the plain k-ascending loop of oracle.c takes minutes per
full-size workload, while every output entry of those workloads is to be
compared.  Rows are evaluated in blocks so that memory stays bounded.
"""
from __future__ import annotations

import numpy as np

from . import e4m3_table, e8m0_value


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: the upper half of a binary32)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 codes -> float64 through the oracle's decoder table (NaN codes -> NaN)."""
    return e4m3_table()[np.ascontiguousarray(codes, dtype=np.uint8)]


def decode_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 elements -> float64: e4m3(code) * 2^(E-127) with E the E8M0 scale
    of the element's 32-element block along K (0xFF -> NaN); exact."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if codes.shape[1] != 32 * scales.shape[1] or codes.shape[0] != scales.shape[0]:
        raise ValueError("scales must be [rows, K/32] for codes [rows, K]")
    table = np.array([e8m0_value(e) for e in range(256)], dtype=np.float64)
    return decode_e4m3(codes) * np.repeat(table[scales], 32, axis=1)


class DenseReference:
    """ref = (scale_a * scale_b) * decode(A) @ decode(B)^T in fp64, by row blocks.

    kind: "bf16" (A, B uint16 bit arrays), "fp8" (A, B uint8 e4m3 codes with
    fp32 per-tensor scales) or "mxfp8" (A, B uint8 e4m3 codes with E8M0 block
    scales scale_a [M, K/32], scale_b [N, K/32]).  B is decoded once;
    rows(r0, r1) decodes that row range of A and returns ref[r0:r1, :]."""

    def __init__(self, kind: str, A: np.ndarray, B: np.ndarray, scale_a=1.0, scale_b=1.0):
        if kind not in ("bf16", "fp8", "mxfp8"):
            raise ValueError("kind must be bf16, fp8 or mxfp8")
        want = np.uint16 if kind == "bf16" else np.uint8
        if A.dtype != want or B.dtype != want:
            raise TypeError("expected %s inputs" % np.dtype(want).name)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
            raise ValueError("A must be [M,K] and B [N,K]")
        self.kind = kind
        self.A = A
        self.M, self.K = A.shape
        self.N = B.shape[0]
        if kind == "mxfp8":
            self._sa = np.ascontiguousarray(scale_a, dtype=np.uint8)
            self._b = decode_mxfp8(B, scale_b)                      # [N, K]
            self.scale = 1.0
            self._decode = None
        else:
            self._decode = decode_bf16 if kind == "bf16" else decode_e4m3
            self._b = self._decode(B)                               # [N, K]
            # the product of the two scales, formed in fp64 as oracle.c does
            self.scale = 1.0 if kind == "bf16" else float(scale_a) * float(scale_b)

    def rows(self, r0: int, r1: int) -> np.ndarray:
        r0, r1 = max(0, r0), min(self.M, r1)
        if self.kind == "mxfp8":
            a = decode_mxfp8(self.A[r0:r1], self._sa[r0:r1])
        else:
            a = self._decode(self.A[r0:r1])
        out = a @ self._b.T
        if self.scale != 1.0:
            out *= self.scale
        return out

    def row_blocks(self, max_flops: float = 1.2e12):
        """(r0, r1) ranges whose product costs at most max_flops each."""
        per_row = max(1.0, 2.0 * self.N * self.K)
        step = max(1, int(max_flops // per_row))
        return [(r, min(self.M, r + step)) for r in range(0, self.M, step)]


def gemm_bf16(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Whole fp64 reference of A·Bᵀ for bf16 bit arrays (small and mid sizes)."""
    ref = DenseReference("bf16", A, B)
    return ref.rows(0, ref.M)


def gemm_fp8(A: np.ndarray, B: np.ndarray, scale_a: float, scale_b: float) -> np.ndarray:
    """Whole fp64 reference of (sa·sb)·(A·Bᵀ) for e4m3 code arrays."""
    ref = DenseReference("fp8", A, B, scale_a, scale_b)
    return ref.rows(0, ref.M)


def gemm_mxfp8(A: np.ndarray, B: np.ndarray, SA: np.ndarray, SB: np.ndarray) -> np.ndarray:
    """Whole fp64 reference of the MXFP8 product (e4m3 codes, E8M0 block scales)."""
    ref = DenseReference("mxfp8", A, B, SA, SB)
    return ref.rows(0, ref.M)
