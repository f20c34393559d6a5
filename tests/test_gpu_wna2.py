"""GPU parity of 2-bit WnA16 (UINT2 codes with a uint2 zero-point and a bf16 scale per channel and
group of 128, bf16 activations; codes turned into the offset-128 bf16 operand by bit-selects,
bf16 MFMA, group scale on the fp32 partial) against the CPU oracle, through the C ABI: dense,
MoE and grouped calls."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, every_configuration, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

D = hq.DESC_W2A16_ASYM


def _run(d, M, N, K):
    w = prepack(D, 1, N, K, d["wq"], d["scales"], d["zeros"])
    return gemm(D, M, N, K, to_dev(d["x"]), None, w)


@pytest.mark.parametrize("M,N,K", [
    (1, 512, 4096), (3, 272, 384), (16, 64, 128), (32, 256, 1024), (64, 512, 512),
    (1, 64, 8192),      # 4 workgroups: K split across workgroups, then the reduction launch
    (200, 256, 640),    # ping-pong 64 x 256 (half-unit weight copies), ragged M
    (300, 512, 1024),   # ping-pong 128 x 256
    (1000, 400, 512),   # no 256-wide tile divides N: skinny
])
def test_wna2_small(M, N, K):
    say(f"[wna2] M={M} N={N} K={K}")
    d = synth.make_wna2(1600, M, N, K)
    y = _run(d, M, N, K)
    ref, _ = oracle.ref_wna2(d["x"], d["wq"], d["scales"], d["zeros"], 128)
    check_float(y, ref, "wna2")


@pytest.mark.parametrize("M", [1, 16, 128, 8192])
def test_wna2_full_size_sampled(M):
    N, K = 14336, 4096
    say(f"[wna2 full] M={M}")
    d = synth.make_wna2(2, M, N, K)
    y = _run(d, M, N, K)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 96)]))
    ref, _ = oracle.ref_wna2(d["x"], d["wq"], d["scales"], d["zeros"], 128, rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"wna2 M={M}")


def test_wna2_every_kernel_configuration(monkeypatch):
    """Every skinny and ping-pong configuration that fits, at a ragged M over 256 rows
    (the ping-pong kernel's 128-wide tiles do not: their half-unit copies do not split over eight
    waves)."""
    M, N, K = 600, 512, 768
    d = synth.make_wna2(1601, M, N, K)
    w = prepack(D, 1, N, K, d["wq"], d["scales"], d["zeros"])
    x = to_dev(d["x"])
    ref, _ = oracle.ref_wna2(d["x"], d["wq"], d["scales"], d["zeros"], 128)
    ran = every_configuration(D, M, N, K, lambda: gemm(D, M, N, K, x, None, w),
                              lambda y, what: check_float(y, ref, f"wna2 {what}"), monkeypatch)
    assert ran.get(0, 0) >= 20 and ran.get(3, 0) >= 4
    monkeypatch.setenv("HQ_TUNE", "kind=3,cfg=2,split=1")     # 128 x 128: refused
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(D, M, N, K)


def test_wna2_extreme_codes_and_zeros():
    """Every code 0 or 3 against zero-points 0 and 3 (the largest |q - z|), scales over 2^-20 .. 2^20."""
    M, N, K = 24, 128, 512
    g = np.random.default_rng(5)
    x = synth.normal_bf16(g, (M, K))
    wq = np.where(g.random((N, K // 4)) < 0.5, 0x00, 0xFF).astype(np.uint8)
    zeros = np.where(g.random((N, K // 128)) < 0.5, 0, 3).astype(np.uint8)
    scales = synth.bf16_bits((2.0 ** g.integers(-20, 21, (N, K // 128))).astype(np.float32))
    y = _run({"x": x, "wq": wq, "scales": scales, "zeros": zeros}, M, N, K)
    ref, _ = oracle.ref_wna2(x, wq, scales, zeros, 128)
    check_float(y, ref, "wna2 extremes", rounding_floor=True)


def _experts(seed, active, N, K):
    return {int(e): dict(synth.make_wna2(seed * 1000 + int(e), 1, N, K), bits=2) for e in active}


def _stack(E, N, K, experts):
    stride = hq.hq_prepacked_bytes(D, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(D, 1, N, K, wd["wq"], wd["scales"], wd["zeros"])
    return w


@pytest.mark.parametrize("T,topk,E,N,K,bm", [
    (5, 2, 4, 64, 256, 16), (64, 8, 16, 512, 1024, 16), (150, 8, 8, 512, 384, 32),
    (400, 8, 16, 256, 768, 64),
])
def test_wna2_moe(T, topk, E, N, K, bm):
    inp = synth.make_moe_inputs(1700 + T, T, K, E, topk)
    ids = inp["topk_ids"]
    experts = _experts(17, np.unique(ids), N, K)
    w = _stack(E, N, K, experts)
    cap = hq.hq_moe_align_capacity(T, topk, E, bm)
    so = torch.empty(cap, dtype=torch.int32, device=DEV)
    be = torch.empty(max(cap // bm, 1), dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    npad = torch.empty(1, dtype=torch.int32, device=DEV)
    hq.hq_moe_align(to_dev(ids.astype(np.int32)), T, topk, E, bm, so, be, offs, npad)
    y = torch.full((T * topk, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wsb = hq.hq_moe_gemm_workspace_bytes(D, T, topk, E, N, K, bm)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    say(f"[wna2 moe] T={T} topk={topk} E={E} N={N} K={K} bm={bm}")
    hq.hq_moe_grouped_gemm(D, T, topk, E, N, K, to_dev(inp["x"]), None, w, so, be, npad, bm,
                           to_dev(inp["topk_weights"].reshape(-1)), y, ws, wsb)
    torch.cuda.synchronize()
    ref, _, valid = oracle.ref_moe_gemm(inp["x"], ids, lambda e: experts[e], N, E, 128,
                                        topk_weights=inp["topk_weights"])
    assert valid.all()
    check_float(y.cpu().numpy(), ref, f"wna2 moe T={T} bm={bm}")


def test_wna2_grouped():
    R, E, N, K = 300, 6, 512, 512
    counts = [80, 0, 120, 40, 59, 1]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.normal_bf16(synth.rng(1800, R), (R, K))
    experts = _experts(18, [e for e in range(E) if counts[e]], N, K)
    w = _stack(E, N, K, experts)
    wsb = hq.hq_grouped_gemm_workspace_bytes(D, R, E, N, K)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    y = torch.empty((R, N), dtype=torch.int16, device=DEV)
    say("[wna2 grouped]")
    hq.hq_grouped_gemm(D, R, E, N, K, to_dev(x), None, w, to_dev(offs), y, ws, wsb)
    torch.cuda.synchronize()
    ref, _, valid = oracle.ref_grouped_gemm(x, offs, lambda e: experts[e], N, E, 128)
    assert valid.all()
    check_float(y.cpu().numpy(), ref, "wna2 grouped")
