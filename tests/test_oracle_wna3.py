"""Pins of the oracle's 3-bit WnA16 path (UINT3 codes in a little-endian bit string per row, a uint3
zero-point and a bf16 scale per (channel, group of 128)), CPU only: hand values with the bit
positions written out, a scalar loop that reads the bit string itself, and the 4-bit oracle on
the same codes."""
import numpy as np

import oracle
import synth


def test_wna3_hand_values():
    # one channel, K = 128, s = 0.25, z = 3; the first 8 codes 0..7 as a bit string:
    # code k at bits 3k..3k+2 -> bytes 0b10_001_000 = 0x88, 0b1_100_011_0 = 0xC6, 0b111_110_10 = 0xFA
    codes = np.full((1, 128), 3, np.uint8)           # z -> weight 0
    codes[0, :8] = np.arange(8)
    wq = np.zeros((1, 48), np.uint8)
    bits = np.zeros(384, np.uint8)
    for k in range(128):
        for b in range(3):
            bits[3 * k + b] = (codes[0, k] >> b) & 1
    for i in range(48):
        wq[0, i] = sum(int(bits[8 * i + j]) << j for j in range(8))
    assert wq[0, :3].tolist() == [0x88, 0xC6, 0xFA]
    s = synth.bf16_bits(np.array([[0.25]], np.float32))
    z = np.array([[3]], np.uint8)
    w = oracle.dequant_wna3(wq, s, z, 128)
    assert w[0, :8].tolist() == [-0.75, -0.5, -0.25, 0.0, 0.25, 0.5, 0.75, 1.0] and not w[0, 8:].any()
    assert np.array_equal(synth._pack_triplets(codes), wq)


def test_wna3_brute_force():
    M, N, K = 3, 5, 256
    g = synth.rng(91)
    x = synth.normal_bf16(g, (M, K))
    xv = synth.bf16_bits_to_f32(x).astype(np.float64)
    wq = g.integers(0, 256, (N, 3 * K // 8), dtype=np.uint8)
    s = synth.bf16_bits((g.random((N, K // 128)) + 0.5).astype(np.float32))
    sv = synth.bf16_bits_to_f32(s).astype(np.float64)
    z = g.integers(0, 8, (N, K // 128)).astype(np.uint8)
    y, bits = oracle.ref_wna3(x, wq, s, z, 128)
    for m in range(M):
        for n in range(N):
            stream = int.from_bytes(bytes(wq[n]), "little")
            acc = 0.0
            for k in range(K):
                q = (stream >> (3 * k)) & 7
                acc += xv[m, k] * ((q - int(z[n, k // 128])) * sv[n, k // 128])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(bits, oracle.round_to_bf16(y))


def test_wna3_equals_4bit_oracle_on_the_same_codes():
    M, N, K = 4, 48, 384
    d = synth.make_wna3(931, M, N, K)
    codes = oracle.unpack_triplets(d["wq"])
    wq4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    y3, b3 = oracle.ref_wna3(d["x"], d["wq"], d["scales"], d["zeros"], 128)
    y4, b4 = oracle.ref_wna16(d["x"], wq4, d["scales"], d["zeros"], 128)
    assert np.array_equal(y3, y4) and np.array_equal(b3, b4)
    ys, _ = oracle.ref_wna3(d["x"], d["wq"], d["scales"], d["zeros"], 128, rows=[0, 3], cols=[5, 47])
    assert np.array_equal(ys, y3[np.ix_([0, 3], [5, 47])])
