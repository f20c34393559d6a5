"""Pins for the oracle's MoE token sort and grouped GEMM: the hand case H5, invariants of the
sort, and reduction of the grouped GEMM to per-token dense GEMMs."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def test_h5_moe_align():
    c = GOLD["H5_moe_align"]
    r = oracle.ref_moe_align(np.array(c["topk_ids"]), c["E"], c["block_m"])
    assert r["counts"].tolist() == c["counts"]
    assert r["expert_offsets"].tolist() == c["expert_offsets"]
    assert r["num_padded"] == c["num_padded"]
    assert r["sorted_ids"].tolist() == c["sorted_ids"]
    assert r["block_expert"].tolist() == c["block_expert"]


@pytest.mark.parametrize("T,topk,E,bm", [(1, 8, 256, 16), (37, 8, 16, 4), (200, 2, 7, 64)])
def test_moe_align_invariants(T, topk, E, bm):
    ids = np.random.default_rng(T).integers(0, E, (T, topk)).astype(np.int32)
    r = oracle.ref_moe_align(ids, E, bm)
    flat = ids.reshape(-1)
    S = T * topk
    assert r["counts"].sum() == S
    off = r["expert_offsets"]
    assert off[0] == 0 and np.all(np.diff(off) % bm == 0) and off[-1] == r["num_padded"]
    real = r["sorted_ids"][r["sorted_ids"] != S]
    assert sorted(real.tolist()) == list(range(S))
    for e in range(E):
        seg = r["sorted_ids"][off[e]:off[e + 1]]
        members = seg[seg != S]
        assert np.all(flat[members] == e)
        assert np.all(np.diff(members) > 0)                     # stable ascending order
        assert np.all(seg[len(members):] == S)                  # padding at the end only
        assert len(seg) - len(members) < bm                      # minimal padding
    for b, e in enumerate(r["block_expert"]):
        assert off[e] <= b * bm < off[e + 1]


def test_moe_align_skips_out_of_range_ids():
    ids = np.array([[0, 5], [-1, 1]], np.int32)
    r = oracle.ref_moe_align(ids, 2, 2)
    assert r["counts"].tolist() == [1, 1]
    assert r["sorted_ids"].tolist() == [0, 4, 3, 4]


def test_moe_gemm_equals_per_token_dense():
    T, topk, E, N, K = 5, 2, 4, 8, 256
    x = synth.normal_bf16(np.random.default_rng(0), (T, K))
    ids = np.array([[0, 3], [1, 0], [3, 3], [2, 1], [0, 2]], np.int32)
    ws = {e: synth.make_moe_weights_expert(950, e, N, K) for e in range(E)}
    tw = np.random.default_rng(1).random((T, topk)).astype(np.float32)
    y, _, valid = oracle.ref_moe_gemm(x, ids, lambda e: ws[e], N, E, 128, topk_weights=tw)
    assert valid.all()
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            yd, _ = oracle.ref_wna16(x[t:t + 1], ws[e]["wq"], ws[e]["scales"], None, 128)
            assert np.array_equal(y[t * topk + j], yd[0] * float(tw[t, j]))


def test_moe_gemm_invalid_rows_masked():
    T, topk, E, N, K = 2, 2, 2, 4, 128
    x = synth.normal_bf16(np.random.default_rng(0), (T, K))
    ids = np.array([[0, 7], [1, -1]], np.int32)
    ws = {e: synth.make_moe_weights_expert(951, e, N, K) for e in range(E)}
    _, _, valid = oracle.ref_moe_gemm(x, ids, lambda e: ws[e], N, E, 128)
    assert valid.tolist() == [True, False, True, False]


def test_grouped_gemm_equals_per_row_dense_and_masks_uncovered_rows():
    """Each row equals the dense WNA16 GEMM of its own expert (a special case that reduces to the
    dense oracle); empty, decreasing and out-of-range bounds cover no rows."""
    R, E, N, K = 11, 5, 16, 256
    x = synth.normal_bf16(np.random.default_rng(2), (R, K))
    ws = {e: synth.make_moe_weights_expert(952, e, N, K) for e in range(E)}
    # expert 0: rows 0-2; 1: empty; 2: rows 3-6; 3: [7, 14) clipped to [7, 11); 4: the
    # decreasing pair [14, 9), no rows
    offs = np.array([0, 3, 3, 7, 14, 9])
    y, bits, valid = oracle.ref_grouped_gemm(x, offs, lambda e: ws[e], N, E, 128)
    owner = {r: 0 for r in range(0, 3)} | {r: 2 for r in range(3, 7)} | {r: 3 for r in range(7, 11)}
    for r in range(R):
        e = owner[r]
        yd, _ = oracle.ref_wna16(x[r:r + 1], ws[e]["wq"], ws[e]["scales"], None, 128)
        assert np.array_equal(y[r], yd[0]), r
    assert valid.all()


def test_grouped_gemm_brute_force_and_gaps():
    """Scalar triple loop on a tiny case with a gap between ranges; E = 1 is the dense GEMM."""
    R, E, N, K = 6, 3, 4, 128
    x = synth.normal_bf16(np.random.default_rng(3), (R, K))
    ws = {e: synth.make_moe_weights_expert(953, e, N, K) for e in range(E)}
    offs = np.array([0, 2, 2, 5])          # rows 0-1 expert 0, 2-4 expert 2, row 5 in no range
    y, _, valid = oracle.ref_grouped_gemm(x, offs, lambda e: ws[e], N, E, 128)
    assert valid.tolist() == [True] * 5 + [False]
    xv = oracle.decode_bf16(x)
    for r, e in [(0, 0), (1, 0), (2, 2), (3, 2), (4, 2)]:
        codes = oracle.decode_int4_sym(oracle.unpack_nibbles(ws[e]["wq"]))
        s = oracle.decode_bf16(ws[e]["scales"])
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(xv[r, k]) * float(codes[n, k]) * float(s[n, k // 128])
            assert abs(y[r, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    yd, _ = oracle.ref_wna16(x, ws[0]["wq"], ws[0]["scales"], None, 128)
    y1, _, _ = oracle.ref_grouped_gemm(x, np.array([0, R]), lambda e: ws[0], N, 1, 128)
    assert np.array_equal(y1, yd)


def test_quantized_moe_gemm_equals_per_token_dense():
    """8-bit activations: W4A8 (MXFP4 experts, e4m3 tokens) and W8A8 (INT8 experts, int8 tokens)
    grouped GEMMs equal the per-token dense oracles, times the router weight."""
    T, topk, E, N, K = 4, 2, 3, 16, 256
    ids = np.array([[0, 2], [1, 0], [2, 2], [1, -1]], np.int32)
    tw = np.random.default_rng(5).random((T, topk)).astype(np.float32)
    a8 = synth.make_w4a8_activations(961, T, K)
    ws = {e: synth.make_moe_weights_expert_mx(961, e, N, K) for e in range(E)}
    y, _, valid = oracle.ref_moe_gemm_q(a8["xq"], a8["s_tok"], ids, lambda e: ws[e], N, E, "e4m3", topk_weights=tw)
    assert valid.tolist() == [True] * 7 + [False]
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            if e < 0:
                continue
            yd, _ = oracle.ref_w4a8(a8["xq"][t:t + 1], a8["s_tok"][t:t + 1], ws[e]["wq"], ws[e]["scales"])
            assert np.array_equal(y[t * topk + j], yd[0] * float(tw[t, j]))
    a1 = synth.make_w8a8_activations(962, T, K)
    wi = {e: synth.make_moe_weights_expert_w8a8(962, e, N, K) for e in range(E)}
    y, _, _ = oracle.ref_moe_gemm_q(a1["xq"], a1["s_tok"], ids, lambda e: wi[e], N, E, "int8")
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            if e < 0:
                continue
            _, yd, _ = oracle.ref_w8a8(a1["xq"][t:t + 1], a1["s_tok"][t:t + 1], wi[e]["wq"], wi[e]["s_ch"])
            assert np.array_equal(y[t * topk + j], yd[0])
