"""Pins of the oracle's MoE grouped GEMMs with block-scaled FP8 experts and tokens, and with MX-scaled
tokens (MXFP4, MXFP8) and MXFP4 experts, CPU only: every routed row equals the dense oracle of the
format on that token and expert, rows routed outside [0, E) stay invalid, the router weight
multiplies, and a scalar loop over the block-scaled definition on a tiny case with distinct
block scales."""
import numpy as np

import oracle
import synth


def _tokens(seed, T, K):
    x = synth.bf16_bits_to_f32(synth.normal_bf16(synth.rng(seed), (T, K)))
    return synth.quantize_fp8_blocks(x, 1, 128)


def test_moe_fp8_block_equals_per_token_dense():
    T, topk, E, N, K = 5, 2, 3, 256, 384
    xq, xs = _tokens(61, T, K)
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, 1], [0, 3]])     # 3 is outside [0, E)
    ws = {e: synth.make_moe_weights_expert_fp8b(970, e, N, K) for e in range(E)}
    tw = synth.rng(62).random((T, topk)).astype(np.float32)
    y, bits, valid = oracle.ref_moe_gemm_fp8_block(xq, xs, ids, lambda e: ws[e], N, E, topk_weights=tw)
    assert valid.tolist() == [True] * 9 + [False]
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            if e >= E:
                continue
            yd, _ = oracle.ref_w8a8_fp8_block(xq[t:t + 1], xs[t:t + 1], ws[e]["wq"], ws[e]["ws"])
            np.testing.assert_allclose(y[t * topk + j], yd[0] * np.float64(tw[t, j]), rtol=1e-12, atol=1e-300)
    assert np.array_equal(bits[valid], oracle.round_to_bf16(y[valid]))
    cols = [0, 129, 255]
    ys, _, _ = oracle.ref_moe_gemm_fp8_block(xq, xs, ids, lambda e: ws[e], N, E, topk_weights=tw,
                                             rows=[1, 4], cols=cols)
    assert np.array_equal(ys, y[np.ix_([1, 4], cols)])


def test_moe_fp8_block_scalar_loop():
    T, topk, E, N, K = 2, 2, 2, 128, 256
    g = synth.rng(63)
    codes = lambda shape: g.integers(0, 0x7F, shape).astype(np.uint8) | (g.integers(0, 2, shape).astype(np.uint8) << 7)
    xq = codes((T, K))
    xs = (2.0 ** g.integers(-4, 4, (T, K // 128))).astype(np.float32)
    ws = {e: {"wq": codes((N, K)), "ws": (2.0 ** g.integers(-6, 2, (1, K // 128))).astype(np.float32)}
          for e in range(E)}
    ids = np.array([[1, 0], [1, 1]])
    y, _, _ = oracle.ref_moe_gemm_fp8_block(xq, xs, ids, lambda e: ws[e], N, E)
    import torch
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xv = dec(xq)
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            wv = dec(ws[e]["wq"])
            for n in (0, 77, 127):
                acc = 0.0
                for k in range(K):
                    acc += float(xs[t, k // 128]) * float(ws[e]["ws"][n // 128, k // 128]) * xv[t, k] * wv[n, k]
                assert abs(y[t * topk + j, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_moe_mx_tokens_equal_per_token_dense():
    T, topk, E, N, K = 4, 2, 3, 32, 256
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, 5]])          # 5 is outside [0, E)
    ws = {e: synth.make_moe_weights_expert_mx(975, e, N, K) for e in range(E)}
    tw = synth.rng(64).random((T, topk)).astype(np.float32)
    a4 = synth.make_w4a4_activations(976, T, K)
    x8 = synth.bf16_bits_to_f32(synth.normal_bf16(synth.rng(977), (T, K)))
    xq8, xs8 = synth.quantize_mxfp8_rows(x8)
    for act, xq, xs, dense in (("mxfp4", a4["xq"], a4["xs"], oracle.ref_w4a4),
                               ("mxfp8", xq8, xs8, oracle.ref_w4a8_mx)):
        y, bits, valid = oracle.ref_moe_gemm_mx(xq, xs, ids, lambda e: ws[e], N, E, act, topk_weights=tw)
        assert valid.tolist() == [True] * 7 + [False]
        for t in range(T):
            for j in range(topk):
                e = ids[t, j]
                if e >= E:
                    continue
                yd, _ = dense(xq[t:t + 1], xs[t:t + 1], ws[e]["wq"], ws[e]["scales"])
                np.testing.assert_allclose(y[t * topk + j], yd[0] * np.float64(tw[t, j]), rtol=1e-13)
        ys, _, _ = oracle.ref_moe_gemm_mx(xq, xs, ids, lambda e: ws[e], N, E, act, topk_weights=tw,
                                          rows=[0, 5], cols=[1, 30])
        assert np.array_equal(ys, y[np.ix_([0, 5], [1, 30])])
