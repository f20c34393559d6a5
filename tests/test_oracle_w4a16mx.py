"""Pins of the oracle's MXFP4-weight paths with bf16 activations (dense and MoE), CPU only: a
scalar loop, the W4A8 oracle on activations that e4m3 holds exactly, and per-token dense GEMMs."""
import numpy as np
import torch

import oracle
import synth


def test_w4a16_mx_brute_force():
    M, N, K = 3, 5, 64
    g = synth.rng(41)
    x = synth.normal_bf16(g, (M, K))
    wq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = g.integers(118, 136, (N, K // 32)).astype(np.uint8)
    y, bits = oracle.ref_w4a16_mx(x, wq, ws)
    xv = oracle.decode_bf16(x)
    wc = np.stack([wq & 0xF, wq >> 4], axis=-1).reshape(N, K)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(xv[m, k]) * float(oracle.decode_e2m1(wc[n, k])) * 2.0 ** (int(ws[n, k // 32]) - 127)
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(bits, oracle.round_to_bf16(y))


def test_w4a16_mx_equals_w4a8_on_e4m3_exact_activations():
    M, N, K = 4, 16, 256
    g = synth.rng(42)
    codes = g.integers(0, 0x7F, (M, K)).astype(np.uint8) | (g.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    x32 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    x_bf16 = synth.bf16_bits(x32)                       # e4m3 values are exact in bf16
    w = synth.quantize_mxfp4(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    y16, b16 = oracle.ref_w4a16_mx(x_bf16, w["wq"], w["scales"])
    y8, b8 = oracle.ref_w4a8(codes, np.ones(M, np.float32), w["wq"], w["scales"])
    assert np.array_equal(y16, y8) and np.array_equal(b16, b8)


def test_moe_gemm_with_mxfp4_experts_equals_per_token_dense():
    T, topk, E, N, K = 4, 2, 3, 16, 128
    x = synth.normal_bf16(synth.rng(43), (T, K))
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, 1]])
    ws = {e: synth.make_moe_weights_expert_mx(960, e, N, K) for e in range(E)}
    y, _, valid = oracle.ref_moe_gemm(x, ids, lambda e: ws[e], N, E, 128)
    assert valid.all()
    for t in range(T):
        for j in range(topk):
            yd, _ = oracle.ref_w4a16_mx(x[t:t + 1], ws[ids[t, j]]["wq"], ws[ids[t, j]]["scales"])
            assert np.array_equal(y[t * topk + j], yd[0])
    offs = np.array([0, 1, 3, 4])
    yg, _, vg = oracle.ref_grouped_gemm(x, offs, lambda e: ws[e], N, E, 128)
    for r, e in enumerate([0, 1, 1, 2]):
        yd, _ = oracle.ref_w4a16_mx(x[r:r + 1], ws[e]["wq"], ws[e]["scales"])
        assert np.array_equal(yg[r], yd[0])
