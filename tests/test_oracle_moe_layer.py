"""Pins of the oracle's MoE layer stages (gated activation, top-k combine, full layer), CPU only."""
import math

import numpy as np
from scipy.special import expit

import oracle
from oracle.codecs import decode_bf16, round_to_bf16

import synth


def _bf16(v):
    return synth.bf16_bits(np.asarray(v, dtype=np.float32))


def test_silu_mul_hand_values():
    # gate = [0, 1, -2, 4], up = [5, 2, 1, -0.5]
    gu = _bf16([[0.0, 1.0, -2.0, 4.0, 5.0, 2.0, 1.0, -0.5]])
    act, bits = oracle.ref_silu_mul(gu)
    want = [0.0, 2.0 / (1 + math.exp(-1.0)), -2.0 / (1 + math.exp(2.0)), -0.5 * 4.0 / (1 + math.exp(-4.0))]
    assert np.allclose(act[0], want, rtol=0, atol=1e-15)
    assert bits.tolist() == [round_to_bf16(np.array(want)).tolist()]


def test_silu_mul_against_expit():
    g = synth.normal_bf16(synth.rng(5), (16, 64), std=3.0)
    u = synth.normal_bf16(synth.rng(6), (16, 64))
    act, _ = oracle.ref_silu_mul(np.concatenate([g, u], axis=1))
    gv, uv = decode_bf16(g), decode_bf16(u)
    assert np.allclose(act, gv * expit(gv) * uv, rtol=1e-14, atol=1e-300)


def test_combine_hand_case_and_skipped_rows():
    ids = np.array([[0, 3], [7, 1]])          # E = 4: expert 7 is out of range
    y = _bf16([[1.0, 2.0], [0.5, -4.0], [100.0, 100.0], [0.25, 0.25]])
    out, bits = oracle.ref_moe_combine(y, ids, 4)
    assert out.tolist() == [[1.5, -2.0], [0.25, 0.25]]
    assert bits.tolist() == _bf16([[1.5, -2.0], [0.25, 0.25]]).tolist()


def _layer_brute(x_bits, ids, tw, gu_w, dn_w, I, H, E, rounded=True):
    """Scalar loops over one routed row at a time, straight from the layer's definition
    (rounded=False: no bf16 rounding between the stages)."""
    rnd = (lambda v: decode_bf16(round_to_bf16(np.array(v)))) if rounded else (lambda v: np.array(v))
    T, topk = ids.shape
    x = decode_bf16(x_bits)
    out = np.zeros((T, H))
    for t in range(T):
        acc = [0.0] * H
        for k in range(topk):
            e = int(ids[t, k])
            if not 0 <= e < E:
                continue
            Wgu = oracle.dequant_wna16(gu_w[e]["wq"], gu_w[e]["scales"], None, 128)
            Wd = oracle.dequant_wna16(dn_w[e]["wq"], dn_w[e]["scales"], None, 128)
            gu = [sum(float(x[t, j]) * float(Wgu[n, j]) for j in range(x.shape[1])) for n in range(2 * I)]
            gu = rnd(gu)
            a = [gu[i] / (1.0 + math.exp(-gu[i])) * gu[I + i] for i in range(I)]
            a = rnd(a)
            w = float(np.float32(tw[t, k]))
            d = [w * sum(a[i] * float(Wd[h, i]) for i in range(I)) for h in range(H)]
            d = rnd(d)
            acc = [acc[h] + d[h] for h in range(H)]
        out[t] = acc
    return round_to_bf16(out) if rounded else out


def test_layer_matches_scalar_loops():
    T, topk, E, H, I = 3, 2, 3, 128, 128
    g = synth.rng(77)
    gu_w = [synth.quantize_int4_sym(g.standard_normal((2 * I, H)).astype(np.float32) * np.float32(0.05), 128)
            for _ in range(E)]
    dn_w = [synth.quantize_int4_sym(g.standard_normal((H, I)).astype(np.float32) * np.float32(0.05), 128)
            for _ in range(E)]
    x = synth.normal_bf16(g, (T, H))
    ids = np.array([[0, 2], [1, 5], [2, 2]])  # expert 5 is out of range; token 2 routes twice to 2
    tw = np.array([[0.7, 0.3], [0.6, 0.4], [0.5, 0.5]], dtype=np.float32)
    ref = oracle.ref_moe_layer(x, ids, tw, lambda e: gu_w[e], lambda e: dn_w[e], I, H, E, 128)
    assert np.array_equal(ref["out"], _layer_brute(x, ids, tw, gu_w, dn_w, I, H, E))
    exact = oracle.ref_moe_layer(x, ids, tw, lambda e: gu_w[e], lambda e: dn_w[e], I, H, E, 128, exact=True)
    brute = _layer_brute(x, ids, tw, gu_w, dn_w, I, H, E, rounded=False)
    assert np.allclose(exact["out"], brute, rtol=1e-12, atol=1e-12 * np.abs(brute).max())
    # the bf16 boundaries move the result by rounding noise only: a few bf16 ulps at most
    assert np.abs(decode_bf16(ref["out"]) - exact["out"]).max() <= 2.0 ** -5 * np.abs(exact["out"]).max()


def test_w4a8_layer_with_one_expert_is_the_dense_chain():
    """E = 1, top-1: every stage of the W4A8 layer is the dense chain quantize -> W4A8 GEMM ->
    SiLU*mul -> quantize -> W4A8 GEMM (router weight 1) computed with the dense oracles."""
    T, H, I = 6, 256, 128
    x = synth.normal_bf16(synth.rng(81), (T, H))
    gu_w = synth.make_moe_weights_expert_mx(82, 0, 2 * I, H)
    dn_w = synth.make_moe_weights_expert_mx(83, 0, H, I)
    ids = np.zeros((T, 1), np.int64)
    tw = np.ones((T, 1), np.float32)
    r = oracle.ref_moe_layer_w4a8(x, ids, tw, lambda e: gu_w, lambda e: dn_w, I, H, 1)
    xq, xs = oracle.quantize_per_token(x, "e4m3")
    _, gu = oracle.ref_w4a8(xq, xs, gu_w["wq"], gu_w["scales"])
    _, act = oracle.ref_silu_mul(gu)
    aq, as_ = oracle.quantize_per_token(act, "e4m3")
    _, dn = oracle.ref_w4a8(aq, as_, dn_w["wq"], dn_w["scales"])
    assert np.array_equal(r["gate_up"], gu) and np.array_equal(r["act"], act)
    assert np.array_equal(r["down"], dn) and np.array_equal(r["out"], dn)
    assert np.array_equal(r["xq"], xq) and np.array_equal(r["aq"], aq)


def test_w4a8_layer_routes_each_row_to_its_expert():
    T, topk, E, H, I = 5, 2, 3, 128, 64
    x = synth.normal_bf16(synth.rng(84), (T, H))
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, 1], [0, 1]])
    tw = synth.rng(85).random((T, topk)).astype(np.float32)
    gw = {e: synth.make_moe_weights_expert_mx(86, e, 2 * I, H) for e in range(E)}
    dw = {e: synth.make_moe_weights_expert_mx(87, e, H, I) for e in range(E)}
    r = oracle.ref_moe_layer_w4a8(x, ids, tw, lambda e: gw[e], lambda e: dw[e], I, H, E)
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            _, gu = oracle.ref_w4a8(r["xq"][t:t + 1], r["xs"][t:t + 1], gw[e]["wq"], gw[e]["scales"])
            assert np.array_equal(r["gate_up"][t * topk + j], gu[0])
            y, _ = oracle.ref_w4a8(r["aq"][t * topk + j:t * topk + j + 1], r["as"][t * topk + j:t * topk + j + 1],
                                   dw[e]["wq"], dw[e]["scales"])
            assert np.array_equal(r["down"][t * topk + j], oracle.round_to_bf16(y[0] * np.float64(tw[t, j])))
