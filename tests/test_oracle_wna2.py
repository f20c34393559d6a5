"""Pins of the oracle's 2-bit WnA16 path (UINT2 codes with a uint2 zero-point and a bf16 scale
per (channel, group of 128)), CPU only: hand values with the bit positions written out, a scalar
loop that unpacks the bytes itself, and the 4-bit oracle on the same codes (a 2-bit code and
zero are also valid 4-bit ones)."""
import numpy as np

import oracle
import synth


def test_wna2_hand_values():
    # one channel, K = 128 (one group), s = 0.5, z = 1; byte 0 = 0b11_10_01_00 holds codes 0,1,2,3
    # for k = 0..3 (lowest k in the lowest bits); every other code 1 (= z, weight 0).
    wq = np.full((1, 32), 0b01010101, np.uint8)
    wq[0, 0] = 0b11100100
    s = synth.bf16_bits(np.array([[0.5]], np.float32))
    z = np.array([[1]], np.uint8)
    w = oracle.dequant_wna2(wq, s, z, 128)
    assert w[0, :4].tolist() == [-0.5, 0.0, 0.5, 1.0] and not w[0, 4:].any()
    x = np.zeros((1, 128), np.float32)
    x[0, :4] = [2.0, 3.0, -1.0, 4.0]          # 2*(-0.5) + 0 + (-1)*0.5 + 4*1 = 2.5
    y, bits = oracle.ref_wna2(synth.bf16_bits(x), wq, s, z, 128)
    assert y[0, 0] == 2.5 and bits[0, 0] == 0x4020


def test_wna2_brute_force():
    M, N, K = 3, 5, 256
    g = synth.rng(71)
    x = synth.normal_bf16(g, (M, K))
    xv = synth.bf16_bits_to_f32(x).astype(np.float64)
    wq = g.integers(0, 256, (N, K // 4), dtype=np.uint8)
    s = synth.bf16_bits((g.random((N, K // 128)) + 0.5).astype(np.float32))
    sv = synth.bf16_bits_to_f32(s).astype(np.float64)
    z = g.integers(0, 4, (N, K // 128)).astype(np.uint8)
    y, bits = oracle.ref_wna2(x, wq, s, z, 128)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                q = (int(wq[n, k // 4]) >> (2 * (k % 4))) & 3
                acc += xv[m, k] * ((q - int(z[n, k // 128])) * sv[n, k // 128])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(bits, oracle.round_to_bf16(y))


def test_wna2_equals_4bit_oracle_on_the_same_codes():
    M, N, K = 4, 48, 384
    d = synth.make_wna2(921, M, N, K)
    codes = oracle.unpack_crumbs(d["wq"])
    wq4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    y2, b2 = oracle.ref_wna2(d["x"], d["wq"], d["scales"], d["zeros"], 128)
    y4, b4 = oracle.ref_wna16(d["x"], wq4, d["scales"], d["zeros"], 128)
    assert np.array_equal(y2, y4) and np.array_equal(b2, b4)
    ys, _ = oracle.ref_wna2(d["x"], d["wq"], d["scales"], d["zeros"], 128, rows=[1, 3], cols=[0, 47])
    assert np.array_equal(ys, y2[np.ix_([1, 3], [0, 47])])


def test_uint2_quantizer_reconstructs_within_half_a_step():
    w = synth.rng(72).standard_normal((8, 256)).astype(np.float32) * np.float32(0.02)
    d = synth.quantize_uint2_asym(w, 128)
    deq = oracle.dequant_wna2(d["wq"], d["scales"], d["zeros"], 128)
    s = synth.bf16_bits_to_f32(d["scales"]).astype(np.float64)[:, np.arange(256) // 128]
    # codes clamp to [0, 3], so the error bound holds inside the representable range only
    lo = (0 - d["zeros"].astype(np.float64)[:, np.arange(256) // 128]) * s
    hi = (3 - d["zeros"].astype(np.float64)[:, np.arange(256) // 128]) * s
    inside = (w >= lo) & (w <= hi)
    assert inside.mean() > 0.9
    assert np.all(np.abs(deq - w)[inside] <= 0.5 * s[inside] * (1 + 1e-6))


def test_moe_gemm_with_2bit_experts_equals_per_token_dense():
    T, topk, E, N, K = 4, 2, 3, 32, 256
    x = synth.normal_bf16(synth.rng(73), (T, K))
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, 1]])
    ws = {e: dict(synth.make_wna2(990 + e, 1, N, K), bits=2) for e in range(E)}
    y, _, valid = oracle.ref_moe_gemm(x, ids, lambda e: ws[e], N, E, 128)
    assert valid.all()
    for t in range(T):
        for j in range(topk):
            w = ws[ids[t, j]]
            yd, _ = oracle.ref_wna2(x[t:t + 1], w["wq"], w["scales"], w["zeros"], 128)
            assert np.array_equal(y[t * topk + j], yd[0])
