"""Pins for the oracle's dense GEMMs: hand cases (tests/golden), a brute-force triple loop,
special cases that reduce to a plain library matmul, and non-square shapes that catch a
transposed operand."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _bf16(vals):
    return synth.bf16_bits(np.asarray(vals, dtype=np.float32))


def test_h1_int4_sym():
    c = GOLD["H1_int4_sym"]
    y, bits = oracle.ref_wna16(_bf16([c["x"]]), np.array([c["wq_bytes"]], np.uint8),
                               np.array([c["scales_bf16"]], np.uint16), None, c["g"])
    assert y[0, 0] == c["y"] and bits[0, 0] == c["y_bf16"]


def test_h2_uint4_asym():
    c = GOLD["H2_uint4_asym"]
    y, bits = oracle.ref_wna16(_bf16([c["x"]]), np.array([c["wq_bytes"]], np.uint8),
                               np.array([c["scales_bf16"]], np.uint16),
                               np.array([c["zeros"]], np.uint8), c["g"])
    assert y[0, 0] == c["y"] and bits[0, 0] == c["y_bf16"]


def test_h3_w8a8():
    c = GOLD["H3_w8a8"]
    acc, y, bits = oracle.ref_w8a8(np.array([c["xq"]], np.int8),
                                   np.array([c["s_tok_f32"]], np.float32),
                                   np.array([c["wq"]], np.int8),
                                   np.array([c["s_ch_f32"]], np.float32))
    assert acc[0, 0] == c["acc"] and bits[0, 0] == c["y_bf16"]


def test_h4_w4a8():
    c = GOLD["H4_w4a8_mxfp4"]
    K = c["K"]
    codes = np.zeros(K, np.uint8)
    codes[:4] = c["w_codes"]
    wq = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None]
    xq = np.zeros(K, np.uint8)
    xq[:4] = c["x_codes"]
    y, bits = oracle.ref_w4a8(xq[None], np.array([c["s_tok_f32"]], np.float32), wq,
                              np.array([[c["e8m0"]]], np.uint8))
    assert y[0, 0] == c["y"] and bits[0, 0] == c["y_bf16"]


# ---- brute force: scalar loops written from the definitions, tiny shapes -------------------
def _brute_wna16(xb, wq, s, z, g):
    M, K = xb.shape
    N = wq.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(wq[n, k // 2])
                code = (byte >> 4) if (k % 2) else (byte & 0xF)
                if z is None:
                    q = code - 16 if code >= 8 else code
                else:
                    q = code - int(z[n, k // g])
                sv = float(np.array([int(s[n, k // g]) << 16], np.uint32).view(np.float32)[0])
                xv = float(np.array([int(xb[m, k]) << 16], np.uint32).view(np.float32)[0])
                acc += xv * q * sv
            out[m, n] = acc
    return out


@pytest.mark.parametrize("asym", [False, True])
def test_wna16_brute_force(asym):
    g = 4
    M, N, K = 3, 5, 8          # non-square: a transposed operand cannot pass
    d = synth.make_wna16(900 + asym, M, N, K, asym=asym, g=g)
    y, _ = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d.get("zeros"), g)
    ref = _brute_wna16(d["x"], d["wq"], d["scales"], d.get("zeros"), g)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-15)
    assert y.shape == (M, N)


def test_w8a8_brute_force():
    M, N, K = 3, 4, 7
    g = np.random.default_rng(5)
    xq = g.integers(-127, 128, (M, K)).astype(np.int8)
    wq = g.integers(-127, 128, (N, K)).astype(np.int8)
    st = g.random(M).astype(np.float32)
    sc = g.random(N).astype(np.float32)
    acc, y, _ = oracle.ref_w8a8(xq, st, wq, sc)
    for m in range(M):
        for n in range(N):
            a = sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))
            assert acc[m, n] == a
            assert y[m, n] == a * float(st[m]) * float(sc[n])


def test_w4a8_brute_force():
    M, N, K = 2, 3, 64
    g = np.random.default_rng(6)
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    e = g.integers(120, 134, (N, K // 32)).astype(np.uint8)
    xq = g.integers(0, 256, (M, K)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x38           # no NaN codes
    st = g.random(M).astype(np.float32)
    y, _ = oracle.ref_w4a8(xq, st, wq, e)
    e2m1 = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                c = int(codes[n, k])
                wv = (-1 if c & 8 else 1) * e2m1[c & 7] * 2.0 ** (int(e[n, k // 32]) - 127)
                b = int(xq[m, k])
                ex, mn = (b >> 3) & 0xF, b & 7
                xv = (mn / 8 * 2.0 ** -6) if ex == 0 else (1 + mn / 8) * 2.0 ** (ex - 7)
                acc += (-xv if b & 0x80 else xv) * wv
            assert np.isclose(y[m, n], acc * float(st[m]), rtol=1e-13, atol=0)


# ---- special cases that reduce to a library matmul ----------------------------------------
def test_wna16_unit_scales_is_integer_matmul():
    g = np.random.default_rng(7)
    M, N, K, gs = 4, 6, 256, 128
    q = g.integers(0, 16, (N, K)).astype(np.uint8)
    wq = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    ones = np.full((N, K // gs), 0x3F80, np.uint16)
    zeros = np.zeros((N, K // gs), np.uint8)
    x = g.integers(-4, 5, (M, K)).astype(np.float32)
    y, _ = oracle.ref_wna16(synth.bf16_bits(x), wq, ones, zeros, gs)
    assert np.array_equal(y, x.astype(np.int64) @ q.astype(np.int64).T)
    # symmetric decode of the same codes: two's complement
    qs = np.where(q >= 8, q.astype(np.int64) - 16, q)
    y2, _ = oracle.ref_wna16(synth.bf16_bits(x), wq, ones, None, gs)
    assert np.array_equal(y2, x.astype(np.int64) @ qs.T)


def test_w4a8_unit_scales_is_matmul_of_decoded():
    g = np.random.default_rng(8)
    M, N, K = 3, 5, 96
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    e = np.full((N, K // 32), 127, np.uint8)
    x = g.standard_normal((M, K)).astype(np.float32)
    import torch
    xq = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    xv = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    wv = oracle.decode_e2m1(codes)
    y, _ = oracle.ref_w4a8(xq, np.ones(M, np.float32), wq, e)
    assert np.allclose(y, xv @ wv.T, rtol=1e-14, atol=0)


def test_mx_block_scale_applies_per_32():
    # scaling one block's exponent by +1 doubles exactly that block's contribution
    N, K = 1, 64
    codes = np.full((N, K), 0x2, np.uint8)      # all 1.0
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    xq = np.full((1, K), 0x38, np.uint8)        # all 1.0
    y0, _ = oracle.ref_w4a8(xq, np.ones(1, np.float32), wq, np.array([[127, 127]], np.uint8))
    y1, _ = oracle.ref_w4a8(xq, np.ones(1, np.float32), wq, np.array([[128, 127]], np.uint8))
    assert y0[0, 0] == 64.0 and y1[0, 0] == 96.0


def test_group_scale_indexing():
    # group g covers k in [g*gs, (g+1)*gs): only that group's scale may affect its columns
    N, K, gs = 1, 256, 128
    q = np.full((N, K), 1, np.uint8)
    wq = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    s = np.array([[0x3F80, 0x4000]], np.uint16)             # 1.0, 2.0
    x = np.zeros((1, K), np.float32)
    x[0, 127] = 1.0
    x[0, 128] = 10.0
    y, _ = oracle.ref_wna16(synth.bf16_bits(x), wq, s, None, gs)
    assert y[0, 0] == 1.0 * 1 * 1.0 + 10.0 * 1 * 2.0


def test_sampled_rows_cols_match_full():
    d = synth.make_wna16(901, 8, 32, 256, asym=True)
    y, b = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d["zeros"], 128)
    rows, cols = [1, 5, 7], [0, 3, 31]
    ys, bs = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d["zeros"], 128, rows=rows, cols=cols)
    assert np.array_equal(ys, y[np.ix_(rows, cols)]) and np.array_equal(bs, b[np.ix_(rows, cols)])
