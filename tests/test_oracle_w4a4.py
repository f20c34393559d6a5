"""Pins of the oracle's W4A4-MXFP4 path (CPU only): the MXFP4 activation quantizer against hand
cases of the OCP MX rule (ties, saturation, zero and subnormal blocks, the largest scale),
invariants on random data, and the GEMM against a scalar triple loop and against the W4A8 oracle
on activations that e4m3 holds exactly."""
import numpy as np
import torch

import oracle
import synth


def _bf16(v):
    return synth.bf16_bits(np.asarray(v, dtype=np.float32))


def _unpack(packed):
    return np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[0], -1)


def test_mxfp4_act_ties_and_saturation():
    # amax 6 -> floor(log2 6) - 2 = 0: scale byte 127, v = x
    row = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 6.0, -6.0, 0.5, 0.0, -0.0, 1.0, 3.0]
    row = row + [0.0] * 16
    codes, scales = oracle.quantize_mxfp4_act(_bf16([row]))
    assert scales.tolist() == [[127]]
    got = _unpack(codes)[0, :16].tolist()
    # midpoints go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0,
    # 3.5 -> 4.0, 5 -> 4.0; -0.25 rounds to +0; sign bit 8 for the negative non-zero values
    assert got == [0, 2, 2, 4, 4, 6, 6, 0, 8 | 6, 7, 8 | 7, 1, 0, 0, 2, 5]


def test_mxfp4_act_scale_rule():
    blocks = [
        [0.75] + [0.3] * 31,          # floor(log2 0.75) = -1 -> e = -3, v = 8x: 6 and 2.4 -> 2
        [3.984375] + [0.0] * 31,      # floor(log2 3.98) = 1 -> e = -1: v = 7.97 saturates to 6
        [0.0] * 32,                   # zero block: byte 0, all codes 0
        [2.0 ** -130] * 32,           # subnormal: e clamps at -127, v = 2^-3 rounds to 0
        [1.5 * 2.0 ** 127] + [2.0 ** 126] * 31,   # e = 125: v = 6 and 2
    ]
    x = _bf16([sum(blocks, [])])
    codes, scales = oracle.quantize_mxfp4_act(x)
    assert scales.tolist() == [[124, 126, 0, 0, 252]]
    c = _unpack(codes)[0].reshape(5, 32)
    assert c[0, 0] == 7 and (c[0, 1:] == 4).all()
    assert c[1, 0] == 7 and (c[1, 1:] == 0).all()
    assert (c[2] == 0).all() and (c[3] == 0).all()
    assert c[4, 0] == 7 and (c[4, 1:] == 4).all()


def test_mxfp4_act_invariants_random():
    g = synth.rng(11)
    x = synth.normal_bf16(g, (64, 256), std=3.0)
    x[5] = synth.normal_bf16(g, (1, 256), std=1e-20)[0]
    codes, scales = oracle.quantize_mxfp4_act(x)
    xv = oracle.decode_bf16(x)
    deq = oracle.dequant_mxfp4(codes, scales)
    scale = oracle.decode_e8m0(scales)[:, np.arange(256) // 32]
    v = xv / scale
    # |v| < 8 always (amax < 2^(e+3)); only values past 6 saturate
    assert np.abs(v).max() < 8
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    unsat = np.abs(v) <= 6
    assert (np.abs(deq - xv)[unsat] <= 0.5 * (step * scale)[unsat]).all()
    assert (np.abs(deq)[~unsat] == 6 * scale[~unsat]).all()
    # MX-representable values come back unchanged
    codes2, scales2 = oracle.quantize_mxfp4_act(oracle.round_to_bf16(deq))
    assert np.array_equal(oracle.dequant_mxfp4(codes2, scales2), deq)


def test_encode_e2m1_matches_torch_decode_of_all_codes():
    """Every code decodes (oracle table) to a value that encodes back to the same code, signed
    zero aside; torch's e2m1 decode agrees on the magnitudes where the dtype is available."""
    vals = oracle.decode_e2m1(np.arange(16))
    back = oracle.encode_e2m1(vals)
    assert back.tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 0, 9, 10, 11, 12, 13, 14, 15]
    assert vals.tolist()[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    if hasattr(torch, "float4_e2m1fn_x2"):
        b = torch.tensor([0x10 * ((c + 1) % 16) + c for c in range(16)], dtype=torch.uint8)
        try:
            f = b.view(torch.float4_e2m1fn_x2).to(torch.float32)
        except (RuntimeError, NotImplementedError, TypeError):
            return
        got = f.reshape(-1).numpy().astype(np.float64)
        want = np.stack([vals, oracle.decode_e2m1((np.arange(16) + 1) % 16)], axis=1).reshape(-1)
        assert np.array_equal(got, want)


def test_w4a4_brute_force():
    M, N, K = 3, 5, 64
    g = synth.rng(12)
    xq = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    xs = g.integers(120, 134, (M, K // 32), dtype=np.uint8)
    wq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = g.integers(118, 136, (N, K // 32), dtype=np.uint8)
    y, bits = oracle.ref_w4a4(xq, xs, wq, ws)
    xc, wc = _unpack(xq), _unpack(wq)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                xv = float(oracle.decode_e2m1(xc[m, k])) * 2.0 ** (int(xs[m, k // 32]) - 127)
                wv = float(oracle.decode_e2m1(wc[n, k])) * 2.0 ** (int(ws[n, k // 32]) - 127)
                acc += xv * wv
            assert y[m, n] == acc
    assert np.array_equal(bits, oracle.round_to_bf16(y))


def test_w4a4_equals_w4a8_on_e4m3_exact_activations():
    """Activation scales within 2^-6 .. 2^4 keep every MXFP4 value exact in e4m3, so the W4A4
    product equals the W4A8 oracle with those values as e4m3 codes and unit token scales."""
    M, N, K = 4, 16, 128
    g = synth.rng(13)
    xq = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    xs = g.integers(121, 132, (M, K // 32), dtype=np.uint8)
    w = synth.quantize_mxfp4(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    xv = oracle.dequant_mxfp4(xq, xs)
    x8 = torch.from_numpy(xv.astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(x8.to(torch.float64).numpy(), xv)
    y4, b4 = oracle.ref_w4a4(xq, xs, w["wq"], w["scales"])
    y8, b8 = oracle.ref_w4a8(x8.view(torch.uint8).numpy(), np.ones(M, np.float32), w["wq"], w["scales"])
    assert np.array_equal(y4, y8) and np.array_equal(b4, b8)
