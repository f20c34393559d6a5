"""Pins of the oracle's per-token activation quantization (oracle/actquant.py), CPU only.

The e4m3 encoder is checked against torch's own float8_e4m3fn cast (an independent library
routine) on every midpoint and code value plus random values; the per-token quantizer against
hand cases whose scales are powers of two, so every quotient and tie is exact and checkable by
hand."""
import numpy as np
import torch

import oracle.actquant as aq
from oracle.codecs import decode_e4m3

import synth


def _bf16(vals):
    return synth.bf16_bits(np.asarray(vals, dtype=np.float32))


def test_e4m3_encoder_matches_torch_cast():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = decode_e4m3(codes)
    pos = np.unique(np.abs(vals))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    rand = rng.uniform(-448, 448, 20000)
    tiny = rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)
    v = np.concatenate([vals, mids, -mids, rand, tiny, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = aq.encode_e4m3(v)
    assert np.array_equal(got, ref)


def test_e4m3_encoder_saturates():
    assert aq.encode_e4m3(np.array([1000.0, -449.0, 448.0])).tolist() == [0x7E, 0xFE, 0x7E]


def test_int8_hand_case():
    # amax = 15.875 = 127 * 2^-3 -> s = 0.125 exactly; quotients 127, -127, 0.5, 1.5, -2.5, 8
    x = _bf16([[15.875, -15.875, 0.0625, 0.1875, -0.3125, 1.0]])
    q, s = aq.quantize_per_token(x, "int8")
    assert s.tolist() == [0.125]
    assert q.tolist() == [[127, -127, 0, 2, -2, 8]]


def test_e4m3_hand_case():
    # amax = 112 = 448 * 2^-2 -> s = 0.25 exactly; quotients 448, 1, 1.125, 1.0625 (tie -> 1.0),
    # 1.1875 (tie -> 1.25), -2^-9 (smallest subnormal), 3*2^-10 (tie -> 2^-8), tiny negative -> -0
    x = _bf16([[112.0, 0.25, 0.28125, 0.265625, 0.296875, -2.0 ** -11, 3 * 2.0 ** -12, -2.0 ** -16]])
    q, s = aq.quantize_per_token(x, "e4m3")
    assert s.tolist() == [0.25]
    assert q.tolist() == [[0x7E, 0x38, 0x39, 0x38, 0x3A, 0x81, 0x02, 0x80]]


def test_zero_row_and_scale_rule():
    x = np.zeros((2, 16), dtype=np.uint16)
    x[1, 3] = _bf16([-3.0])[0]
    for act, qmax in (("int8", 127.0), ("e4m3", 448.0)):
        q, s = aq.quantize_per_token(x, act)
        assert s[0] == 1.0 and not q[0].any()
        assert s[1] == np.float32(np.float32(3.0) / np.float32(qmax))


def test_int8_error_bound_and_range():
    g = np.random.default_rng(1)
    x = synth.normal_bf16(g, (64, 512))
    q, s = aq.quantize_per_token(x, "int8")
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    assert (np.abs(q).max(axis=1) == 127).all()           # the absmax element reaches the range end
    err = np.abs(xf - q.astype(np.float64) * s[:, None].astype(np.float64))
    # the binary32 quotient is within 127 * 2^-24 of the exact one
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -23)).all()
