"""The acceptance statistics of oracle/parity.py on hand-built outputs: each
rule (i)-(iii) and the ulp histogram count exactly the entries built to
break them."""
import numpy as np

from oracle import parity

BF16_TWO = 0x4000          # 2.0; the next code up is 2 + 2^-6


def _case(values, K=64):
    """Outputs that equal the reference exactly (fp32 and bf16 codes)."""
    ref = np.asarray(values, dtype=np.float64)
    c32 = ref.astype(np.float32)
    cb = parity.f32_to_bf16_rne(c32)
    return ref, c32, cb, K


def test_exact_output_passes_with_every_count_zero():
    ref, c32, cb, K = _case([1.0, -2.5, 0.0, 300.0, -0.0078125])
    s = parity.stats(ref, c32, cb, K)
    assert s["pass"] and s["checked"] == 5 and s["max_abs_err"] == 0.0
    assert s["ulp_hist"] == {"0": 5, "1": 0, ">=2": 0}
    assert s["fail_i"] == s["fail_ii"] == s["fail_iii_far"] == s["fail_iii_near"] == 0
    assert abs(s["tol"] - 1e-3 * 8.0) < 1e-15 and s["max_err_over_sqrtK"] == 0.0


def test_one_and_two_ulp_away_in_the_far_range():
    # K = 64: tol = 0.008 < ulp(2.0) = 2^-6, so 2.0 is in the 1-ulp range
    # (1.0 is not: its ulp 2^-7 = 0.0078 is below tol)
    ref, c32, cb, K = _case([2.0, 2.0, 2.0])
    cb = cb.copy()
    cb[1] = BF16_TWO + 1                       # one code up
    cb[2] = BF16_TWO + 2                       # two codes up
    c32 = parity.bf16_to_f64(cb).astype(np.float32)   # keep (ii) satisfied
    s = parity.stats(ref, c32, cb, K)
    assert s["ulp_hist"] == {"0": 1, "1": 1, ">=2": 1}
    assert s["fail_iii_far"] == 1 and s["literal_1ulp_violations"] == 1
    assert s["fail_i"] == 2                    # fp32 values 2^-6 and 2^-5 off, tol 0.008
    assert not s["pass"]


def test_bf16_not_the_rounding_of_fp32_is_rule_ii():
    ref, c32, cb, K = _case([3.0, 5.0])
    cb = cb.copy()
    cb[0] ^= 1                                 # bf16 code one off, fp32 untouched
    s = parity.stats(ref, c32, cb, K)
    assert s["fail_ii"] == 1 and s["fail_i"] == 0 and s["ulp_hist"]["1"] == 1


def test_near_zero_uses_tol_plus_half_ulp():
    # K = 1 << 20: tol = 1.024, larger than ulp(ref) for |ref| < 128
    K = 1 << 20
    ref = np.array([0.5, 0.5, 0.5])
    c32 = np.array([0.5 + 1.0, 0.5 + 1.2, 0.5 - 0.9], dtype=np.float32)
    cb = parity.f32_to_bf16_rne(c32)
    s = parity.stats(ref, c32, cb, K)
    # 1.5 and -0.4 are within tol (1.024) + ulp/2 of 0.5; 1.7 is not
    assert s["fail_iii_near"] == 1 and s["fail_iii_far"] == 0
    assert s["fail_i"] == 1                    # |1.7 - 0.5| > 1.024
    assert s["ulp_hist"][">=2"] == 3          # many codes away, yet two entries pass (iii)


def test_signed_zero_and_sign_crossing_in_the_histogram():
    ref = np.array([0.0, 0.0, 2.0 ** -133])
    cb = np.array([0x8000, 0x0000, 0x8001], dtype=np.uint16)   # -0, +0, -(smallest subnormal)
    c32 = parity.bf16_to_f64(cb).astype(np.float32)
    s = parity.stats(ref, c32, cb, 64)
    # -0 and +0 are the same value; +min to -min is two codes (through zero)
    assert s["ulp_hist"] == {"0": 2, "1": 0, ">=2": 1}
