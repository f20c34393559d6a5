"""Pins of the oracle's 8-bit-weight paths with bf16 activations (INT8 and FP8 e4m3 weights with a
per-channel fp32 scale), CPU only: hand values, a scalar loop that decodes the codes itself
(two's complement by hand, e4m3 by torch's own cast), the W8A8 INT8 oracle on integer
activations, the block-scaled FP8 oracle on e4m3-exact activations with uniform scales, and
column-wise scale indexing."""
import numpy as np
import torch

import oracle
import synth


def _bf16(v):
    return synth.bf16_bits(np.asarray(v, dtype=np.float32))


def test_w8a16_hand_values():
    # INT8: x = [1.5, -2], codes [3, -4] (bytes 0x03, 0xFC), s = 0.5:
    #   (1.5*3 + (-2)*(-4)) * 0.5 = (4.5 + 8) * 0.5 = 6.25
    x = _bf16([[1.5, -2.0]])
    wq = np.array([[3, -4]], dtype=np.int8)
    y, bits = oracle.ref_w8a16(x, wq, np.array([0.5], np.float32))
    assert y[0, 0] == 6.25 and bits[0, 0] == 0x40C8          # 6.25 = 0x40C8 in bf16
    # INT8 extremes: -127 (0x81) and 127 (0x7F) with x = 1, 1: 0 after the scale
    y, _ = oracle.ref_w8a16(_bf16([[1.0, 1.0]]), np.array([[-127, 127]], np.int8), np.array([3.0], np.float32))
    assert y[0, 0] == 0.0
    # FP8 e4m3: 0x40 = 2.0 (exp field 8, bias 7), 0xB8 = -1.0, 0x01 = 2^-9 (smallest subnormal),
    # 0x7E = 448; x = [1, 3, 2^9, 1], s = 0.25:
    #   (2 - 3 + 1 + 448) * 0.25 = 112
    x = _bf16([[1.0, 3.0, 512.0, 1.0]])
    wq = np.array([[0x40, 0xB8, 0x01, 0x7E]], dtype=np.uint8)
    y, _ = oracle.ref_w8a16(x, wq, np.array([0.25], np.float32), fp8=True)
    assert y[0, 0] == 112.0


def test_w8a16_brute_force_int8_and_fp8():
    M, N, K = 3, 5, 48
    g = synth.rng(51)
    x = synth.normal_bf16(g, (M, K))
    xv = synth.bf16_bits_to_f32(x).astype(np.float64)
    s = (g.random(N) + 0.5).astype(np.float32)
    # INT8 codes over the whole byte range except -128 (decoded by hand: b - 256 for b >= 128)
    b8 = g.integers(0, 256, (N, K)).astype(np.uint8)
    b8[b8 == 0x80] = 0x81
    y, bits = oracle.ref_w8a16(x, b8.view(np.int8), s)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                q = int(b8[n, k]) - 256 if b8[n, k] >= 128 else int(b8[n, k])
                acc += xv[m, k] * (q * float(s[n]))
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(bits, oracle.round_to_bf16(y))
    # FP8 e4m3 codes (no NaN: 0x7F / 0xFF excluded), decoded by torch's float8_e4m3fn cast
    f8 = g.integers(0, 0x7F, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)).astype(np.uint8) << 7)
    dec = torch.from_numpy(f8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    y, _ = oracle.ref_w8a16(x, f8, s, fp8=True)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += xv[m, k] * (dec[n, k] * float(s[n]))
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_w8a16_int8_equals_w8a8_on_integer_activations():
    # bf16 holds every integer in [-127, 127] exactly: with those as activations and a unit token
    # scale, the bf16-activation oracle and the W8A8 integer oracle compute the same sum
    M, N, K = 4, 32, 256
    g = synth.rng(52)
    xi = g.integers(-127, 128, (M, K)).astype(np.int8)
    w = synth.quantize_int8_rows(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    y16, b16 = oracle.ref_w8a16(_bf16(xi.astype(np.float32)), w[0], w[1])
    _, y8, b8 = oracle.ref_w8a8(xi, np.ones(M, np.float32), w[0], w[1])
    np.testing.assert_allclose(y16, y8, rtol=1e-13, atol=0)
    assert np.abs(b16.astype(np.int64) - b8.astype(np.int64)).max() <= 1


def test_w8a16_fp8_equals_block_scaled_fp8_with_uniform_scales():
    # e4m3 activations are exact in bf16; with every weight scale equal (s) and unit activation
    # block scales, the block-scaled FP8 oracle reduces to the per-channel one
    M, N, K = 3, 128, 256
    g = synth.rng(53)
    xc = g.integers(0, 0x7F, (M, K)).astype(np.uint8) | (g.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    x32 = torch.from_numpy(xc).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    wc = g.integers(0, 0x7F, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)).astype(np.uint8) << 7)
    s = np.float32(0.0625)
    y16, _ = oracle.ref_w8a16(_bf16(x32), wc, np.full(N, s, np.float32), fp8=True)
    yb, _ = oracle.ref_w8a8_fp8_block(xc, np.ones((M, K // 128), np.float32), wc,
                                      np.full((N // 128, K // 128), s, np.float32))
    np.testing.assert_allclose(y16, yb, rtol=1e-13, atol=0)


def test_w8a16_scale_is_per_output_channel():
    # distinct scales per channel, M != N: column n of y must be (x . q[n]) * s[n]; a transposed
    # or per-row scale fails
    M, N, K = 3, 7, 32
    g = synth.rng(54)
    x = synth.normal_bf16(g, (M, K))
    q = g.integers(-127, 128, (N, K)).astype(np.int8)
    s = (2.0 ** g.integers(-6, 6, N)).astype(np.float32)
    y, _ = oracle.ref_w8a16(x, q, s)
    xv = synth.bf16_bits_to_f32(x).astype(np.float64)
    for n in range(N):
        np.testing.assert_allclose(y[:, n], (xv @ q[n].astype(np.float64)) * float(s[n]), rtol=1e-13)
    # and the unit-scale case is the decoded matmul
    y1, _ = oracle.ref_w8a16(x, q, np.ones(N, np.float32))
    np.testing.assert_allclose(y1, xv @ q.astype(np.float64).T, rtol=1e-13)


def test_w8a16_row_and_column_subsets():
    d = synth.make_w8a16(902, 9, 48, 256, fp8=True)
    y, bits = oracle.ref_w8a16(d["x"], d["wq"], d["s_ch"], fp8=True)
    rows, cols = [0, 4, 8], [1, 17, 47]
    ys, bs = oracle.ref_w8a16(d["x"], d["wq"], d["s_ch"], fp8=True, rows=rows, cols=cols)
    assert np.array_equal(ys, y[np.ix_(rows, cols)]) and np.array_equal(bs, bits[np.ix_(rows, cols)])


def test_moe_gemm_with_8bit_experts_equals_per_token_dense():
    T, topk, E, N, K = 4, 2, 3, 32, 256
    x = synth.normal_bf16(synth.rng(55), (T, K))
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, 1]])
    for fp8 in (False, True):
        ws = {}
        for e in range(E):
            d = synth.make_w8a16(980 + e, 1, N, K, fp8=fp8)
            ws[e] = {"wq": d["wq"], "s_ch": d["s_ch"], "fp8": fp8}
        y, _, valid = oracle.ref_moe_gemm(x, ids, lambda e: ws[e], N, E, 128)
        assert valid.all()
        for t in range(T):
            for j in range(topk):
                e = ids[t, j]
                yd, _ = oracle.ref_w8a16(x[t:t + 1], ws[e]["wq"], ws[e]["s_ch"], fp8=fp8)
                np.testing.assert_allclose(y[t * topk + j], yd[0], rtol=1e-13)
        yc, _, _ = oracle.ref_moe_gemm(x, ids, lambda e: ws[e], N, E, 128, cols=[3, 31])
        assert np.array_equal(yc, y[:, [3, 31]])
