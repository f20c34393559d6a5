"""Pins for the oracle's format decoders: hand tables, torch's independent dtype casts, the
zero-exponent equivalence of the Humming announcement ("Results: quantization support"),
and bf16 round-to-nearest-even tie cases."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def test_e2m1_hand_table():
    # OCP MX v1.0 e2m1 magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.decode_e2m1(np.arange(16))
    assert list(got[:8]) == expect
    assert list(got[8:]) == [-v for v in expect]
    assert got[0x1] == 0.5 and got[0x7] == 6.0 and got[0xA] == -1.0 and got[0xF] == -6.0
    assert np.signbit(got[0x8])  # negative zero


def test_e8m0_hand_and_torch():
    assert oracle.decode_e8m0(np.array([127]))[0] == 1.0
    assert oracle.decode_e8m0(np.array([128]))[0] == 2.0
    assert oracle.decode_e8m0(np.array([0]))[0] == 2.0 ** -127
    assert np.isnan(oracle.decode_e8m0(np.array([255]))[0])
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(oracle.decode_e8m0(b), ref)


def test_e4m3_hand_table():
    d = lambda c: oracle.decode_e4m3(np.array([c]))[0]  # noqa: E731
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0xC0) == -2.0 and d(0x3C) == 1.5
    assert d(0x7E) == 448.0 and d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x00) == 0.0 and np.signbit(d(0x80))


def test_e4m3_matches_torch_all_codes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(b)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(got))


def test_int_codecs():
    assert list(oracle.decode_int4_sym(np.arange(16))) == list(range(8)) + list(range(-8, 0))
    assert list(oracle.decode_uint4(np.arange(16))) == list(range(16))
    assert list(oracle.decode_int8(np.array([0, 127, 128, 129, 255], dtype=np.uint8))) == \
        [0, 127, -128, -127, -1]


def test_unpack_nibbles_low_first():
    got = oracle.unpack_nibbles(np.array([[0xF1, 0x78]], dtype=np.uint8))
    assert got.tolist() == [[0x1, 0xF, 0x8, 0x7]]


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, 4096).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_rne_ties_golden():
    case = GOLD["bf16_rne_ties"]
    f = np.array(case["f32_bits"], dtype=np.uint32).view(np.float32).astype(np.float64)
    assert oracle.round_to_bf16(f).tolist() == case["bf16_bits"]


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    # For inputs that are exactly fp32, one RNE from fp64 equals torch's fp32 -> bf16 RNE.
    x = np.random.default_rng(1).standard_normal(1 << 14).astype(np.float32)
    x = np.concatenate([x, x * 1e-38, x * 1e30, np.array([0.0, -0.0, 1e-45], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), ref)


def test_round_to_bf16_single_rounding():
    # A float64 value just above a bf16 midpoint must round up; a detour through fp32 would
    # first round it onto the midpoint and then to even (down).
    lo = 1.0
    ulp = 2.0 ** -7
    x = lo + ulp / 2 + 2.0 ** -40            # above the midpoint between 1.0 and 1.0078125
    assert oracle.round_to_bf16(np.array([x]))[0] == 0x3F81
    assert oracle.round_to_bf16(np.array([lo + ulp / 2]))[0] == 0x3F80   # exact tie -> even


def test_round_to_bf16_overflow_and_specials():
    big = 3.4e38
    assert oracle.round_to_bf16(np.array([big]))[0] == 0x7F80
    assert oracle.round_to_bf16(np.array([-big]))[0] == 0xFF80
    assert oracle.round_to_bf16(np.array([np.inf]))[0] == 0x7F80
    assert (oracle.round_to_bf16(np.array([np.nan]))[0] & 0x7FC0) == 0x7FC0


@pytest.mark.parametrize("bits", [8, 4])
def test_zero_exponent_equals_symmetric_int(bits):
    """Section 'Results: quantization support': a float format with zero exponent bits holds
    exactly the symmetric integers of the same width (INT8 without -128 <-> float8e0m7)."""
    lim = (1 << (bits - 1)) - 1
    vals = np.arange(-lim, lim + 1)
    # encode v as sign-magnitude by hand, decode with the oracle
    codes = np.where(vals < 0, (1 << (bits - 1)) | (-vals), vals)
    assert np.array_equal(codecs.decode_sign_magnitude(codes, bits), vals)
    # every code of the format lands in the symmetric-integer range; +-0 both decode to 0
    all_vals = codecs.decode_sign_magnitude(np.arange(1 << bits), bits)
    assert set(all_vals.tolist()) == set(vals.tolist())
    # and the two's-complement decoder agrees on the shared range
    if bits == 8:
        tc = oracle.decode_int8((vals & 0xFF).astype(np.uint8))
    else:
        tc = oracle.decode_int4_sym(vals & 0xF)
    assert np.array_equal(tc, vals)
