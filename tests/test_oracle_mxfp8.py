"""Pins of the oracle's MXFP8 activations (W4A8 with MX-scaled FP8 activations), CPU only: hand
cases of the OCP MX scale rule with the e4m3 element (saturation, ties, zero block), torch's own
e4m3 cast on the scaled values, and the GEMM against a scalar loop and the W4A8 oracle."""
import numpy as np
import torch

import oracle
import synth


def _bf16(v):
    return synth.bf16_bits(np.asarray(v, dtype=np.float32))


def test_mxfp8_scale_rule_hand_cases():
    blocks = [
        [448.0, 1.0, -17.0, 19.0] + [0.0] * 28,   # floor(log2 448) = 8 -> e = 0; 17 ties 16/18 -> 16
        [500.0, -500.0] + [0.0] * 30,             # e = 0: 500 saturates to 448
        [1.0, 0.5] + [0.0] * 30,                  # e = -8: v = 256x
        [0.0] * 32,                               # zero block: byte 0
    ]
    codes, scales = oracle.quantize_mxfp8_act(_bf16([sum(blocks, [])]))
    assert scales.tolist() == [[127, 127, 119, 0]]
    c = codes[0].reshape(4, 32)
    # e4m3 (sign, 4-bit exponent field = exponent + 7, 3 mantissa bits): 448 = 0x7E, 1 = 0x38;
    # between 16 and 32 the step is 2: -17 ties -16 (mantissa 000, even) and -18 -> -16 = 0xD8;
    # 19 ties 18 (001) and 20 (010, even) -> 20 = 0x5A
    assert c[0, :4].tolist() == [0x7E, 0x38, 0xD8, 0x5A]
    assert c[1, :2].tolist() == [0x7E, 0xFE]
    assert c[2, :2].tolist() == [0x78, 0x70]   # 256 = 2^8, 128 = 2^7
    assert (c[3] == 0).all()


def test_mxfp8_codes_match_torch_cast_of_scaled_values():
    g = synth.rng(31)
    x = np.concatenate([synth.normal_bf16(g, (32, 256), std=s) for s in (1.0, 1e-3, 300.0)])
    codes, scales = oracle.quantize_mxfp8_act(x)
    e = scales.astype(np.int64) - 127
    xv = oracle.decode_bf16(x).reshape(x.shape[0], -1, 32)
    v = xv * np.ldexp(1.0, -e)[:, :, None]
    assert np.abs(v).max() < 512
    want = torch.from_numpy(np.clip(v, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(codes.reshape(v.shape), want.view(torch.uint8).numpy())


def test_w4a8_mx_brute_force_and_unit_scales():
    M, N, K = 3, 4, 64
    g = synth.rng(32)
    xq = g.integers(0, 0x7F, (M, K)).astype(np.uint8) | (g.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    xs = g.integers(118, 136, (M, K // 32)).astype(np.uint8)
    wq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = g.integers(120, 134, (N, K // 32)).astype(np.uint8)
    y, _ = oracle.ref_w4a8_mx(xq, xs, wq, ws)
    wc = np.stack([wq & 0xF, wq >> 4], axis=-1).reshape(N, K)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                a = float(oracle.decode_e4m3(xq[m, k])) * 2.0 ** (int(xs[m, k // 32]) - 127)
                b = float(oracle.decode_e2m1(wc[n, k])) * 2.0 ** (int(ws[n, k // 32]) - 127)
                acc += a * b
            assert y[m, n] == acc
    y1, b1 = oracle.ref_w4a8_mx(xq, np.full_like(xs, 127), wq, ws)
    y8, b8 = oracle.ref_w4a8(xq, np.ones(M, np.float32), wq, ws)
    assert np.array_equal(y1, y8) and np.array_equal(b1, b8)
