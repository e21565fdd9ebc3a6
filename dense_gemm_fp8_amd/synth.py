"""Seeded synthetic inputs for the tiled GEMM C = A·Bᵀ.

This module is shared by the GPU tests, the bench and the oracle's tests.  It
holds no GEMM arithmetic: it only draws seeded normal matrices and encodes them
into the two input formats the path consumes.

* bf16: float32 N(0, sigma^2) draws rounded to bfloat16 (round to nearest even).
* fp8 (OCP e4m3): float32 N(0, 1) draws divided by a per-tensor scale
  s = amax / 448 (448 is the largest finite e4m3 value) and rounded to the
  nearest e4m3 code with ties to even; magnitudes above 448 saturate to +-448.

* MXFP8 (OCP Microscaling Formats specification v1.0): e4m3 elements with one
  E8M0 scale (2^(E-127)) per block of 32 consecutive elements along K; the
  block's shared exponent is floor(log2(amax)) - 8 (8 = exponent of the
  largest power of two in e4m3) as in the specification's conversion, and the
  elements are x / 2^shared rounded to e4m3 (nearest even, saturating).

The HipKittens L2 note (section 3, "Target operation" table) gives the GEMM shapes and
dtypes but no RNG, quantiser or rounding rule; the plainest readings are used
here and listed in the design notes.

Only numpy is imported, so loading this module never touches the GPU library.
"""
from __future__ import annotations

import dataclasses

import numpy as np

E4M3_MAX = 448.0


def normal_f32(seed: int, rows: int, cols: int, sigma: float = 1.0) -> np.ndarray:
    """rows x cols float32 draws from N(0, sigma^2), PCG64(seed), row-major."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(rows * cols, dtype=np.float32).reshape(rows, cols)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Finite inputs only (the generators never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3 codes (uint8), round to nearest even, saturating.

    Layout S.EEEE.MMM with exponent bias 7; exponent field 0 is subnormal
    (M/8 * 2^-6); S.1111.111 is NaN and never produced here."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    sign = (np.signbit(x)).astype(np.uint8) << np.uint8(7)
    a_in = np.abs(x).astype(np.float32)
    a = np.minimum(a_in, np.float32(E4M3_MAX))   # keeps the integer casts in range
    # normal range [2^-6, 448): a = f * 2^E with f in [0.5, 1); unbiased exponent e = E - 1
    f, E = np.frexp(a)
    e = E.astype(np.int32) - 1
    normal = a >= np.float32(2.0 ** -6)
    # significand in [1, 2) scaled to 3 fraction bits; exact power-of-two scaling
    mq = np.rint(np.ldexp(a, -e) * np.float32(8.0)).astype(np.int32) - 8  # 0..8
    carry = mq == 8
    e_n = np.where(carry, e + 1, e)
    mq = np.where(carry, 0, mq)
    code_n = ((e_n + 7) << 3) | mq
    # subnormal range: multiples of 2^-9; a code of 8 is the smallest normal
    code_s = np.rint(a * np.float32(2.0 ** 9)).astype(np.int32)
    code = np.where(normal, code_n, code_s)
    code = np.where(a_in >= np.float32(E4M3_MAX), 0x7E, code)
    code = np.minimum(code, 0x7E)
    return (code.astype(np.uint8) | sign)


def e4m3_quantize(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Per-tensor quantisation: s = amax/448 (s = 1 if amax == 0), codes = e4m3(x / s)."""
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    q = e4m3_encode((x / s).astype(np.float32))
    return q, s


MX_BLOCK = 32          # elements per E8M0 scale (along K)
E8M0_BIAS = 127
E4M3_EMAX = 8          # exponent of the largest power of two that e4m3 holds (256)


def mx_quantize(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 quantisation of a float32 [R, K] matrix (K % 32 == 0).

    Returns (codes uint8 [R, K], scales uint8 [R, K/32]).  Per block of 32:
    shared = floor(log2(amax)) - 8, clamped to the E8M0 range [-127, 127];
    codes = e4m3(x / 2^shared).  An all-zero block gets scale byte 127 (1.0)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, E = np.frexp(amax)                       # amax = f * 2^E, f in [0.5, 1)
    shared = np.where(amax > 0, E.astype(np.int32) - 1 - E4M3_EMAX, 0)
    shared = np.clip(shared, -E8M0_BIAS, E8M0_BIAS)
    scaled = np.ldexp(blocks, -shared[:, :, None]).astype(np.float32)   # exact power-of-two scaling
    codes = e4m3_encode(scaled).reshape(R, K)
    return codes, (shared + E8M0_BIAS).astype(np.uint8)


def small_int_mx(seed: int, rows: int, cols: int, lo: int = -2, hi: int = 2,
                 elo: int = -2, ehi: int = 2) -> tuple[np.ndarray, np.ndarray]:
    """Integer-valued e4m3 codes in [lo, hi] with E8M0 block scales 2^e,
    e uniform in [elo, ehi] (every product and partial sum exact in fp32 for
    small K)."""
    g = np.random.Generator(np.random.PCG64(seed))
    codes = e4m3_encode(g.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32))
    scales = (g.integers(elo, ehi + 1, size=(rows, cols // MX_BLOCK)) + E8M0_BIAS).astype(np.uint8)
    return codes, scales


# --- workloads -------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMM workload: C[M,N] = A[M,K] · B[N,K]ᵀ."""
    name: str
    dtype: str          # "bf16", "fp8" (per-tensor scales) or "mxfp8" (block scales)
    M: int
    N: int
    K: int
    seed_a: int
    seed_b: int
    sigma_a: float = 1.0
    sigma_b: float = 1.0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def tol(self) -> float:
        """Absolute fp32 tolerance 1e-3 * sqrt(K) on the pre-round result."""
        return 1e-3 * float(np.sqrt(self.K))


def workload(idx: int) -> Workload:
    """The five seeded workloads (1-based index, seeds 1000*i + 1 / + 2)."""
    table = {
        1: ("bf16_256", "bf16", 256, 256, 256, 1.0, 1.0),
        2: ("bf16_8192", "bf16", 8192, 8192, 8192, 1.0, 1.0),
        3: ("bf16_mlp_16384x14336x4096", "bf16", 16384, 14336, 4096, 1.0, 0.02),
        4: ("bf16_16384", "bf16", 16384, 16384, 16384, 1.0, 1.0),
        5: ("fp8_e4m3_8192", "fp8", 8192, 8192, 8192, 1.0, 1.0),
        6: ("mxfp8_8192", "mxfp8", 8192, 8192, 8192, 1.0, 1.0),
    }
    name, dt, M, N, K, sa, sb = table[idx]
    return Workload(name, dt, M, N, K, 1000 * idx + 1, 1000 * idx + 2, sa, sb)


ALL_WORKLOADS = tuple(workload(i) for i in range(1, 6))   # the five configurations
MX_WORKLOAD = workload(6)                                  # block-scaled e4m3 at 8192^3


def make_inputs(w: Workload):
    """Host inputs for a workload.

    bf16:  (A_bits uint16 [M,K], B_bits uint16 [N,K], None, None)
    fp8:   (A_codes uint8 [M,K], B_codes uint8 [N,K], scale_a, scale_b)
    mxfp8: (A_codes uint8 [M,K], B_codes uint8 [N,K], SA uint8 [M,K/32], SB uint8 [N,K/32])"""
    a = normal_f32(w.seed_a, w.M, w.K, w.sigma_a)
    if w.dtype == "bf16":
        A = f32_to_bf16_bits(a)
        del a
        B = f32_to_bf16_bits(normal_f32(w.seed_b, w.N, w.K, w.sigma_b))
        return A, B, None, None
    quant = mx_quantize if w.dtype == "mxfp8" else e4m3_quantize
    qa, sa = quant(a)
    del a
    qb, sb = quant(normal_f32(w.seed_b, w.N, w.K, w.sigma_b))
    return qa, qb, sa, sb


def small_int_bf16(seed: int, rows: int, cols: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer-valued bf16 bits with entries uniform in [lo, hi] (exact in bf16)."""
    g = np.random.Generator(np.random.PCG64(seed))
    v = g.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)
    return f32_to_bf16_bits(v)


def small_int_e4m3(seed: int, rows: int, cols: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer-valued e4m3 codes with entries uniform in [lo, hi] (exact in e4m3)."""
    g = np.random.Generator(np.random.PCG64(seed))
    v = g.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)
    return e4m3_encode(v)


def ternary(seed: int, rows: int, cols: int, dtype: str) -> np.ndarray:
    """Entries in {-1, 0, 1} as bf16 bits (uint16) or e4m3 codes (uint8), one
    random byte each (bytes 0-84 give -1, 85-169 and 255 give 0, 170-254 give
    1), so that operands of gigabytes take seconds to make."""
    g = np.random.Generator(np.random.PCG64(seed))
    n = rows * cols
    words = g.integers(0, 1 << 64, size=-(-n // 8), dtype=np.uint64, endpoint=False)
    raw = words.view(np.uint8)[:n].reshape(rows, cols)
    code = (np.uint16 if dtype == "bf16" else np.uint8)
    neg, one = (0xBF80, 0x3F80) if dtype == "bf16" else (0xB8, 0x38)   # -1.0, 1.0
    table = np.zeros(256, dtype=code)
    table[:85], table[170:255] = neg, one
    return table[raw]


def ternary_long(seed: int, rows: int, cols: int, dtype: str, chunk: int = 1 << 16) -> np.ndarray:
    """Rows of gigabytes with entries in {-1, 0, 1}, made in one write pass:
    each row is a run of `chunk`-element pieces, piece j of row r being row r
    of one random ternary() block with its sign flipped by a random bit per
    (r, j) (sign-bit XOR; a flipped 0 is -0).  An offset error of whole pieces
    therefore meets the opposite sign half the time, and any other offset
    meets different random entries."""
    g = np.random.Generator(np.random.PCG64(seed))
    w = min(chunk, cols)
    block = ternary(int(g.integers(1 << 62)), rows, w, dtype)
    pieces = -(-cols // w)
    bit = 0x8000 if dtype == "bf16" else 0x80
    masks = g.integers(0, 2, size=(rows, pieces)).astype(block.dtype) * block.dtype.type(bit)
    out = np.empty((rows, cols), dtype=block.dtype)
    for j in range(pieces):
        lo, hi = j * w, min(cols, (j + 1) * w)
        np.bitwise_xor(block[:, :hi - lo], masks[:, j:j + 1], out=out[:, lo:hi])
    return out


def e8m0_near_one(seed: int, rows: int, blocks: int) -> np.ndarray:
    """E8M0 block scales uniform in {126, 127, 128} (x0.5, x1, x2), one random
    byte each as in ternary(), for MXFP8 operands of gigabytes."""
    g = np.random.Generator(np.random.PCG64(seed))
    n = rows * blocks
    words = g.integers(0, 1 << 64, size=-(-n // 8), dtype=np.uint64, endpoint=False)
    raw = words.view(np.uint8)[:n].reshape(rows, blocks)
    table = np.full(256, 127, dtype=np.uint8)
    table[:85], table[170:255] = 126, 128
    return table[raw]


def sample_pairs(seed: int, M: int, N: int, count: int, tile: int = 256) -> tuple[np.ndarray, np.ndarray]:
    """Sampled output coordinates (m, n) that touch every output tile.

    One row per tile row and one column per tile column are always included
    (offset inside the tile varies per tile), then `count` further uniform pairs."""
    g = np.random.Generator(np.random.PCG64(seed))
    gm, gn = -(-M // tile), -(-N // tile)
    ms, ns = [], []
    for tm in range(gm):
        for tn in range(gn):
            ms.append(min(M - 1, tm * tile + int(g.integers(0, tile))))
            ns.append(min(N - 1, tn * tile + int(g.integers(0, tile))))
    ms = np.array(ms, dtype=np.int64)
    ns = np.array(ns, dtype=np.int64)
    extra_m = g.integers(0, M, size=count, dtype=np.int64)
    extra_n = g.integers(0, N, size=count, dtype=np.int64)
    return np.concatenate([ms, extra_m]), np.concatenate([ns, extra_n])
