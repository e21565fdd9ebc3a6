"""Pins of the oracle's decoders and its one-step bf16 rounding, and of the
input encoders in dense_gemm_fp8_amd.synth, against library conversions
(torch) and the published format landmarks."""
import math

import numpy as np
import pytest

import oracle
from dense_gemm_fp8_amd import synth

torch = pytest.importorskip("torch")


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(np.isnan(tab), nan)
    np.testing.assert_array_equal(tab[~nan], ref[~nan])
    # signed zeros
    assert math.copysign(1.0, tab[0x80]) == -1.0 and math.copysign(1.0, tab[0x00]) == 1.0


def test_e4m3_landmarks():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0
    assert v(0x01) == 2.0 ** -9
    assert v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6
    assert v(0x38) == 1.0
    assert v(0x7E) == 448.0
    assert v(0xFE) == -448.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))


def test_e4m3_encoder_roundtrip_all_codes():
    tab = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = tab[codes].astype(np.float32)
    np.testing.assert_array_equal(synth.e4m3_encode(vals), codes)


def test_e4m3_encoder_rne_and_saturation():
    enc = lambda x: int(synth.e4m3_encode(np.array([x], dtype=np.float32))[0])
    assert enc(1.0625) == 0x38           # tie between 1.0 and 1.125 -> even (1.0)
    assert enc(1.1875) == 0x3A           # tie between 1.125 and 1.25 -> even (1.25)
    assert enc(500.0) == 0x7E and enc(-1e9) == 0xFE
    assert enc(2.0 ** -10) == 0x00       # tie between 0 and 2^-9 -> 0
    assert enc(3 * 2.0 ** -10) == 0x02   # tie between 2^-9 and 2^-8 -> even (2*2^-9)
    assert enc(15.5 * 2.0 ** -10) == 0x08  # rounds up into the smallest normal


def test_e4m3_encoder_matches_torch_in_range():
    x = synth.normal_f32(9990, 1, 200000).ravel() * np.float32(60.0)
    x = x[np.abs(x) < 440.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(synth.e4m3_encode(x), ref)


def test_e4m3_quantize_scale():
    x = synth.normal_f32(9991, 64, 64)
    q, s = synth.e4m3_quantize(x)
    assert s == np.float32(np.float32(np.max(np.abs(x))) / np.float32(448.0))
    assert np.max(q & 0x7F) == 0x7E      # the amax element maps to 448
    q0, s0 = synth.e4m3_quantize(np.zeros((3, 3), dtype=np.float32))
    assert s0 == 1.0 and not q0.any()


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_bf16_round_landmarks():
    f = lambda u: float(np.array([u], dtype=np.uint32).view(np.float32)[0])
    r = lambda x: int(oracle.bf16_round(np.array([x]))[0])
    assert r(f(0x3F808000)) == 0x3F80          # tie -> even (down)
    assert r(f(0x3F818000)) == 0x3F82          # tie -> even (up)
    assert r(-f(0x3F818000)) == 0xBF82
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81   # single rounding from fp64
    assert r(0.0) == 0x0000 and r(-0.0) == 0x8000
    assert r(2.0 ** -133) == 0x0001            # smallest bf16 subnormal
    assert r(2.0 ** -134) == 0x0000            # tie with zero -> even
    assert r(3.5e38) == 0x7F80                 # overflow -> inf
    assert r(float("inf")) == 0x7F80 and r(float("-inf")) == 0xFF80


def test_bf16_round_matches_torch_for_float32_values():
    x = synth.normal_f32(9992, 1, 100000).ravel() * np.float32(1000.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_round(x.astype(np.float64)), ref)
    # the input generator's bit rule agrees with it too
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), ref)
