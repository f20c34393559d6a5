"""GPU parity of MXFP4 weights with bf16 activations ("W4A16-MXFP4": each weight converted to bf16
with its block scale by the scaled fp4 conversion, bf16 MFMA) for dense, MoE and grouped calls."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, every_configuration, gemm, moe_random_shapes, prepack, say, to_dev

pytestmark = pytest.mark.gpu

D = hq.DESC_W4A16_MXFP4


@pytest.mark.parametrize("M,N,K", [
    (1, 512, 7168), (3, 272, 384), (16, 64, 128), (32, 256, 1024), (64, 512, 512),
    (200, 256, 640),    # ping-pong 128 x 128, 5 K steps
    (300, 512, 1024),   # ping-pong 128 x 256, ragged M
    (1000, 384, 512),   # N not a multiple of 256
])
def test_w4a16mx_small(M, N, K):
    say(f"[w4a16mx] M={M} N={N} K={K}")
    d = synth.make_w4a16mx(1000, M, N, K)
    w = prepack(D, 1, N, K, d["wq"], d["scales"])
    y = gemm(D, M, N, K, to_dev(d["x"]), None, w)
    ref, _ = oracle.ref_w4a16_mx(d["x"], d["wq"], d["scales"])
    check_float(y, ref, "w4a16mx")


def test_w4a16mx_every_kernel_configuration(monkeypatch):
    """Ragged M over 256 rows, N = 512, six K steps, in every configuration that fits."""
    M, N, K = 600, 512, 768
    d = synth.make_w4a16mx(1309, M, N, K)
    w = prepack(D, 1, N, K, d["wq"], d["scales"])
    x = to_dev(d["x"])
    ref, _ = oracle.ref_w4a16_mx(d["x"], d["wq"], d["scales"])
    ran = every_configuration(D, M, N, K, lambda: gemm(D, M, N, K, x, None, w),
                              lambda y, what: check_float(y, ref, f"w4a16mx {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 2, 3))


@pytest.mark.parametrize("M", [1, 128, 8192])
def test_w4a16mx_full_size_sampled(M):
    N, K = 14336, 4096
    say(f"[w4a16mx full] M={M}")
    d = synth.make_w4a16mx(2, M, N, K)
    w = prepack(D, 1, N, K, d["wq"], d["scales"])
    y = gemm(D, M, N, K, to_dev(d["x"]), None, w)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 96)]))
    ref, _ = oracle.ref_w4a16_mx(d["x"], d["wq"], d["scales"], rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"w4a16mx M={M}")


def test_w4a16mx_block_scale_extremes():
    """Weight block scales over 2^-40 .. 2^40 (the converted bf16 weights stay in range)."""
    M, N, K = 64, 256, 1024
    d = synth.make_w4a16mx(1001, M, N, K)
    d["scales"] = np.random.default_rng(7).integers(87, 168, d["scales"].shape).astype(np.uint8)
    w = prepack(D, 1, N, K, d["wq"], d["scales"])
    y = gemm(D, M, N, K, to_dev(d["x"]), None, w)
    ref, _ = oracle.ref_w4a16_mx(d["x"], d["wq"], d["scales"])
    check_float(y, ref, "w4a16mx scale extremes", rounding_floor=True)


def _moe(T, topk, E, N, K, bm, seed, tw=True):
    inp = synth.make_moe_inputs(seed, T, K, E, topk)
    ids = inp["topk_ids"]
    experts = {int(e): synth.make_moe_weights_expert_mx(seed, int(e), N, K) for e in np.unique(ids)}
    stride = hq.hq_prepacked_bytes(D, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(D, 1, N, K, wd["wq"], wd["scales"])
    cap = hq.hq_moe_align_capacity(T, topk, E, bm)
    so = torch.empty(cap, dtype=torch.int32, device=DEV)
    be = torch.empty(max(cap // bm, 1), dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    npad = torch.empty(1, dtype=torch.int32, device=DEV)
    hq.hq_moe_align(to_dev(ids.astype(np.int32)), T, topk, E, bm, so, be, offs, npad)
    y = torch.full((T * topk, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wsb = hq.hq_moe_gemm_workspace_bytes(D, T, topk, E, N, K, bm)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    twd = to_dev(inp["topk_weights"].reshape(-1)) if tw else None
    say(f"[w4a16mx moe] T={T} topk={topk} E={E} N={N} K={K} bm={bm}")
    hq.hq_moe_grouped_gemm(D, T, topk, E, N, K, to_dev(inp["x"]), None, w, so, be, npad, bm, twd, y, ws, wsb)
    torch.cuda.synchronize()
    return inp, experts, y.cpu().numpy()


@pytest.mark.parametrize("T,topk,E,N,K,bm", [
    (5, 2, 4, 64, 256, 16), (64, 8, 16, 512, 1024, 16), (150, 8, 8, 512, 384, 32),
    (400, 8, 16, 1024, 768, 64), (200, 8, 32, 272, 384, 64), (600, 8, 16, 512, 512, 128),
    (300, 8, 64, 384, 640, 128),   # 128-row blocks on 128 x 128 tiles
])
def test_w4a16mx_moe(T, topk, E, N, K, bm):
    inp, experts, y = _moe(T, topk, E, N, K, bm, 1100 + T)
    ref, _, valid = oracle.ref_moe_gemm(inp["x"], inp["topk_ids"], lambda e: experts[e], N, E, 128,
                                        topk_weights=inp["topk_weights"])
    assert valid.all()
    check_float(y, ref, "w4a16mx moe")


def test_w4a16mx_moe_random_shapes():
    """MXFP4 experts with bf16 activations on six seeded random MoE problems."""
    for i, (T, topk, E, N, K, bm, tw) in enumerate(moe_random_shapes(32, 6)):
        inp, experts, y = _moe(T, topk, E, N, K, bm, 1600 + i, tw=tw)
        ref, _, valid = oracle.ref_moe_gemm(inp["x"], inp["topk_ids"], lambda e: experts[e], N, E, 128,
                                            topk_weights=inp["topk_weights"] if tw else None)
        assert valid.all()
        check_float(y, ref, f"w4a16mx moe random {i}")


@pytest.mark.parametrize("T", [8, 512])
def test_w4a16mx_moe_full_size_sampled(T):
    E, topk, N, K = 256, 8, 4096, 7168
    bm = hq.hq_moe_block_m(D, T, topk, E, N, K)
    inp, experts, y = _moe(T, topk, E, N, K, bm, 6, tw=False)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(T).integers(0, N, 96)]))
    ref, _, _ = oracle.ref_moe_gemm(inp["x"], inp["topk_ids"], lambda e: experts[e], N, E, 128, cols=cols)
    check_float(y[:, cols], ref, f"w4a16mx moe full T={T}")


def test_w4a16mx_grouped():
    R, E, N, K = 300, 6, 512, 512
    counts = [80, 0, 120, 40, 59, 1]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.normal_bf16(synth.rng(1200, R), (R, K))
    experts = {e: synth.make_moe_weights_expert_mx(1200, e, N, K) for e in range(E) if counts[e]}
    stride = hq.hq_prepacked_bytes(D, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(D, 1, N, K, wd["wq"], wd["scales"])
    wsb = hq.hq_grouped_gemm_workspace_bytes(D, R, E, N, K)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    y = torch.empty((R, N), dtype=torch.int16, device=DEV)
    say("[w4a16mx grouped]")
    hq.hq_grouped_gemm(D, R, E, N, K, to_dev(x), None, w, to_dev(offs), y, ws, wsb)
    torch.cuda.synchronize()
    ref, _, valid = oracle.ref_grouped_gemm(x, offs, lambda e: experts[e], N, E, 128)
    assert valid.all()
    check_float(y.cpu().numpy(), ref, "w4a16mx grouped")
