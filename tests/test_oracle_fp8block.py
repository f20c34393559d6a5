"""Pins of the oracle's block-scaled FP8 W8A8 (CPU only): a scalar loop with distinct block
scales, unit scales reducing to a plain matmul of decoded e4m3 values, and the block activation
quantizer equal to the pinned per-token rule on every 128-column slice."""
import numpy as np
import torch

import oracle
import synth


def _e4m3_codes(g, shape):
    c = g.integers(0, 0x7F, shape).astype(np.uint8) | (g.integers(0, 2, shape).astype(np.uint8) << 7)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # no NaN codes


def test_fp8_block_brute_force():
    M, N, K = 3, 256, 256
    g = synth.rng(51)
    xq, wq = _e4m3_codes(g, (M, K)), _e4m3_codes(g, (N, K))
    xs = np.exp2(g.integers(-4, 5, (M, K // 128))).astype(np.float32) * np.float32(1.25)
    ws = np.exp2(g.integers(-4, 5, (N // 128, K // 128))).astype(np.float32) * np.float32(0.75)
    y, bits = oracle.ref_w8a8_fp8_block(xq, xs, wq, ws)
    xv, wv = oracle.decode_e4m3(xq), oracle.decode_e4m3(wq)
    for m in range(M):
        for n in (0, 1, 127, 128, 200, 255):
            acc = 0.0
            for k in range(K):
                acc += float(xv[m, k]) * float(xs[m, k // 128]) * float(wv[n, k]) * float(ws[n // 128, k // 128])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(bits, oracle.round_to_bf16(y))


def test_fp8_block_unit_scales_is_a_decoded_matmul():
    M, N, K = 5, 128, 384
    g = synth.rng(52)
    xq, wq = _e4m3_codes(g, (M, K)), _e4m3_codes(g, (N, K))
    y, _ = oracle.ref_w8a8_fp8_block(xq, np.ones((M, 3), np.float32), wq, np.ones((1, 3), np.float32))
    xt = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64)
    wt = torch.from_numpy(wq).view(torch.float8_e4m3fn).to(torch.float64)
    assert np.array_equal(y, (xt @ wt.T).numpy())


def test_fp8_block_activation_quantizer_is_per_token_per_slice():
    x = synth.normal_bf16(synth.rng(53), (7, 384), std=3.0)
    x[2, 128:256] = 0
    codes, scales = oracle.quantize_fp8_block_act(x)
    assert scales[2, 1] == 1.0 and (codes[2, 128:256] == 0).all()
    for gi in range(3):
        q, s = oracle.quantize_per_token(x[:, 128 * gi:128 * (gi + 1)], "e4m3")
        assert np.array_equal(codes[:, 128 * gi:128 * (gi + 1)], q) and np.array_equal(scales[:, gi], s)
