"""Parity checks of GPU results against the oracle (helpers for the GPU tests).

Acceptance for a floating-point GEMM output (tol = 1e-3 * sqrt(K)):
  (i)   |C_f32 - ref| <= tol for every checked entry (ref = fp64 oracle);
  (ii)  C_bf16 == RNE_bf16(C_f32) bit for bit (the epilogue rounds once);
  (iii) where one bf16 ulp of the rounded reference exceeds tol, C_bf16 is
        within 1 ulp of the oracle's rounded value; elsewhere (near zero, where
        the permitted fp32 error is larger than a bf16 ulp) C_bf16 is within
        tol + ulp/2 of ref.
"""
import numpy as np

import oracle


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_ulp(v):
    """Spacing of bf16 at |v| (v already a bf16 value, as float64)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def check(ref, c_f32, c_bf16, K, what=""):
    """Apply (i)-(iii); returns a dict of diagnostics; raises AssertionError on failure."""
    tol = 1e-3 * np.sqrt(max(K, 1))
    ref = np.asarray(ref, dtype=np.float64)
    c32 = np.asarray(c_f32, dtype=np.float32)
    cb = np.asarray(c_bf16, dtype=np.uint16)
    err = np.abs(c32.astype(np.float64) - ref)
    max_err = float(err.max()) if err.size else 0.0
    assert max_err <= tol, "%s (i): max|C_f32 - ref| = %g > tol %g" % (what, max_err, tol)
    rne = f32_to_bf16_rne(c32)
    nbad = int(np.count_nonzero(rne != cb))
    assert nbad == 0, "%s (ii): %d bf16 outputs differ from RNE(C_f32)" % (what, nbad)
    ref_b = oracle.bf16_round(ref)
    rv = bf16_to_f64(ref_b)
    cv = bf16_to_f64(cb)
    ulp = bf16_ulp(rv)
    far = ulp > tol
    bad_far = far & (np.abs(cv - rv) > ulp)
    bad_near = (~far) & (np.abs(cv - ref) > tol + ulp / 2)
    assert not bad_far.any(), "%s (iii): %d outputs off by more than 1 bf16 ulp" % (what, int(bad_far.sum()))
    assert not bad_near.any(), "%s (iii): %d near-zero outputs off by more than tol+ulp/2" % (what, int(bad_near.sum()))
    return {"max_abs_err": max_err, "tol": tol, "max_err_over_sqrtK": max_err / np.sqrt(max(K, 1)),
            "literal_1ulp_violations": int(np.count_nonzero(np.abs(cv - rv) > ulp)),
            "checked": int(ref.size)}
