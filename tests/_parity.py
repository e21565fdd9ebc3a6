"""Parity checks of GPU results against the oracle (helpers for the GPU tests).

The acceptance rule (i)-(iii) and its statistics live in oracle/parity.py;
check() asserts that an output meets it.
"""
from oracle.parity import bf16_to_f64, bf16_ulp, f32_to_bf16_rne, stats   # noqa: F401


def check(ref, c_f32, c_bf16, K, what=""):
    """Apply (i)-(iii); returns the statistics; raises AssertionError on failure."""
    s = stats(ref, c_f32, c_bf16, K)
    assert s["fail_i"] == 0, "%s (i): max|C_f32 - ref| = %g > tol %g (%d entries)" % (
        what, s["max_abs_err"], s["tol"], s["fail_i"])
    assert s["fail_ii"] == 0, "%s (ii): %d bf16 outputs differ from RNE(C_f32)" % (what, s["fail_ii"])
    assert s["fail_iii_far"] == 0, "%s (iii): %d outputs off by more than 1 bf16 ulp" % (
        what, s["fail_iii_far"])
    assert s["fail_iii_near"] == 0, "%s (iii): %d near-zero outputs off by more than tol+ulp/2" % (
        what, s["fail_iii_near"])
    return s
