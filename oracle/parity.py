"""Acceptance statistics of a GEMM output against the oracle -- TEST
INFRASTRUCTURE, like the rest of this package: the GPU tests assert on them,
bench.py's CPU-baseline leg reports them for the rows it computes.

For checked entries with fp64 oracle value ref and tol = 1e-3 * sqrt(K):
  (i)   |C_f32 - ref| <= tol;
  (ii)  C_bf16 == RNE_bf16(C_f32) bit for bit (the epilogue rounds once);
  (iii) where one bf16 ulp of the oracle's rounded value exceeds tol, C_bf16 is
        within 1 ulp of that value; elsewhere (near zero, where the permitted
        fp32 error is larger than a bf16 ulp) C_bf16 is within tol + ulp/2 of
        ref.
The ulp histogram counts how many bf16 codes C_bf16 lies from the oracle's
rounded value (0, 1, 2 or more), whatever its magnitude.
"""
from __future__ import annotations

import numpy as np

from . import bf16_round


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_ulp(v) -> np.ndarray:
    """Spacing of bf16 at |v| (v already a bf16 value, as float64)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def _ordered(bits) -> np.ndarray:
    """bf16 codes as integers in value order (+0 and -0 both 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def stats(ref, c_f32, c_bf16, K: int) -> dict:
    """Counts of (i)-(iii) and the ulp histogram over the given entries."""
    tol = 1e-3 * np.sqrt(max(K, 1))
    ref = np.asarray(ref, dtype=np.float64)
    c32 = np.asarray(c_f32, dtype=np.float32)
    cb = np.asarray(c_bf16, dtype=np.uint16)
    err = np.abs(c32.astype(np.float64) - ref)
    max_err = float(err.max()) if err.size else 0.0
    ref_b = bf16_round(ref)
    rv, cv = bf16_to_f64(ref_b), bf16_to_f64(cb)
    ulp = bf16_ulp(rv)
    far = ulp > tol
    codes = np.abs(_ordered(cb) - _ordered(ref_b))
    out = {
        "checked": int(ref.size),
        "tol": tol,
        "max_abs_err": max_err,
        "max_err_over_sqrtK": max_err / np.sqrt(max(K, 1)),
        "fail_i": int(np.count_nonzero(err > tol)),
        "fail_ii": int(np.count_nonzero(f32_to_bf16_rne(c32) != cb)),
        "fail_iii_far": int(np.count_nonzero(far & (np.abs(cv - rv) > ulp))),
        "fail_iii_near": int(np.count_nonzero(~far & (np.abs(cv - ref) > tol + ulp / 2))),
        "literal_1ulp_violations": int(np.count_nonzero(np.abs(cv - rv) > ulp)),
        "ulp_hist": {"0": int(np.count_nonzero(codes == 0)), "1": int(np.count_nonzero(codes == 1)),
                     ">=2": int(np.count_nonzero(codes >= 2))},
    }
    out["pass"] = not (out["fail_i"] or out["fail_ii"] or out["fail_iii_far"] or out["fail_iii_near"])
    return out
