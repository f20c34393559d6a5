"""GPU parity of 8-bit weights with bf16 activations ("W8A16": INT8 or FP8 e4m3 codes with a
per-channel fp32 scale, each code converted exactly to bf16 in registers, bf16 MFMA, scale in the
epilogue) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, every_configuration, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

FMTS = [False, True]   # fp8


def _desc(fp8):
    return hq.DESC_W8A16_FP8 if fp8 else hq.DESC_W8A16_INT8


def _run(d, M, N, K, fp8):
    w = prepack(_desc(fp8), 1, N, K, d["wq"], d["s_ch"])
    return gemm(_desc(fp8), M, N, K, to_dev(d["x"]), None, w)


@pytest.mark.parametrize("fp8", FMTS)
@pytest.mark.parametrize("M,N,K", [
    (1, 512, 4096), (3, 272, 384), (16, 64, 128), (32, 256, 1024), (64, 512, 512),
    (1, 64, 8192),      # 4 workgroups: K split across workgroups, then the reduction launch
    (200, 256, 640),    # ping-pong 128 x 128, 5 K steps
    (300, 512, 1024),   # pipelined 128 x 256 (eight waves of 64 x 64), ragged M
    (700, 256, 640),    # ping-pong 128 x 128 around M = 768, 5 K steps
    (1100, 256, 128),   # pipelined 128 x 256, one K step
    (1000, 400, 512),   # N not a multiple of the 128-wide tile: skinny fallback
    (1000, 384, 512),   # N % 256 != 0: ping-pong 128 x 128 fallback
])
def test_w8a16_small(M, N, K, fp8):
    say(f"[w8a16 fp8={fp8}] M={M} N={N} K={K}")
    d = synth.make_w8a16(1300, M, N, K, fp8=fp8)
    y = _run(d, M, N, K, fp8)
    ref, _ = oracle.ref_w8a16(d["x"], d["wq"], d["s_ch"], fp8=fp8)
    check_float(y, ref, f"w8a16 fp8={fp8}")


@pytest.mark.parametrize("fp8", FMTS)
@pytest.mark.parametrize("M", [1, 16, 128, 8192])
def test_w8a16_full_size_sampled(M, fp8):
    N, K = 14336, 4096
    say(f"[w8a16 full fp8={fp8}] M={M}")
    d = synth.make_w8a16(2, M, N, K, fp8=fp8)
    y = _run(d, M, N, K, fp8)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 96)]))
    ref, _ = oracle.ref_w8a16(d["x"], d["wq"], d["s_ch"], fp8=fp8, rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"w8a16 fp8={fp8} M={M}")


@pytest.mark.parametrize("fp8", FMTS)
def test_w8a16_every_kernel_configuration(fp8, monkeypatch):
    """Every skinny, pipelined and ping-pong configuration that fits the shape (the tuner may pick
    any), at a ragged M over 256 rows."""
    M, N, K = 600, 512, 768
    d = synth.make_w8a16(1301, M, N, K, fp8=fp8)
    desc = _desc(fp8)
    w = prepack(desc, 1, N, K, d["wq"], d["s_ch"])
    x = to_dev(d["x"])
    ref, _ = oracle.ref_w8a16(d["x"], d["wq"], d["s_ch"], fp8=fp8)
    ran = every_configuration(desc, M, N, K, lambda: gemm(desc, M, N, K, x, None, w),
                              lambda y, what: check_float(y, ref, f"w8a16 fp8={fp8} {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 2, 3))


def test_w8a16_code_and_scale_extremes():
    """INT8 codes -128 .. 127 (-128 accepted as is), FP8 codes up to +-448 incl. subnormals, and
    per-channel scales over 2^-30 .. 2^30."""
    M, N, K = 48, 256, 512
    g = np.random.default_rng(9)
    x = synth.normal_bf16(g, (M, K))
    s = (2.0 ** g.integers(-30, 31, N)).astype(np.float32)
    q8 = g.integers(-128, 128, (N, K)).astype(np.int8)
    y = _run({"x": x, "wq": q8, "s_ch": s}, M, N, K, False)
    ref, _ = oracle.ref_w8a16(x, q8, s)
    check_float(y, ref, "w8a16 int8 extremes", rounding_floor=True)
    f8 = g.integers(0, 0x7F, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)).astype(np.uint8) << 7)
    y = _run({"x": x, "wq": f8, "s_ch": s}, M, N, K, True)
    ref, _ = oracle.ref_w8a16(x, f8, s, fp8=True)
    check_float(y, ref, "w8a16 fp8 extremes", rounding_floor=True)


def test_w8a16_int8_integer_activations_are_exact():
    """Integer activations and weights with a power-of-two scale: every product and partial sum is
    an integer below 2^24, so fp32 accumulation is exact and the output is the oracle rounded once."""
    M, N, K = 20, 128, 1024
    g = np.random.default_rng(11)
    xi = g.integers(-8, 9, (M, K)).astype(np.float32)
    x = synth.bf16_bits(xi)
    q = g.integers(-127, 128, (N, K)).astype(np.int8)
    s = np.full(N, 0.5, np.float32)
    y = _run({"x": x, "wq": q, "s_ch": s}, M, N, K, False)
    _, ref_bits = oracle.ref_w8a16(x, q, s)
    assert np.array_equal(y.view(np.uint16), ref_bits)


def _experts(seed, active, N, K, fp8, random_codes=False):
    out = {}
    for e in active:
        if random_codes:       # many experts: random codes, scales near absmax/127 or /448
            g = synth.rng(seed, 9, int(e))
            if fp8:
                q = g.integers(0, 0x7F, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)).astype(np.uint8) << 7)
            else:
                q = g.integers(-127, 128, (N, K)).astype(np.int8)
            s = (0.0002 * (1 + g.random(N))).astype(np.float32)
        else:
            d = synth.make_w8a16(seed * 1000 + int(e), 1, N, K, fp8=fp8)
            q, s = d["wq"], d["s_ch"]
        out[int(e)] = {"wq": q, "s_ch": s, "fp8": fp8}
    return out


def _stack(desc, E, N, K, experts):
    stride = hq.hq_prepacked_bytes(desc, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(desc, 1, N, K, wd["wq"], wd["s_ch"])
    return w


def _moe(fp8, T, topk, E, N, K, bm, seed, tw=True, random_codes=False, cols=None):
    desc = _desc(fp8)
    inp = synth.make_moe_inputs(seed, T, K, E, topk)
    ids = inp["topk_ids"]
    experts = _experts(seed, np.unique(ids), N, K, fp8, random_codes)
    w = _stack(desc, E, N, K, experts)
    cap = hq.hq_moe_align_capacity(T, topk, E, bm)
    so = torch.empty(cap, dtype=torch.int32, device=DEV)
    be = torch.empty(max(cap // bm, 1), dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    npad = torch.empty(1, dtype=torch.int32, device=DEV)
    hq.hq_moe_align(to_dev(ids.astype(np.int32)), T, topk, E, bm, so, be, offs, npad)
    y = torch.full((T * topk, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wsb = hq.hq_moe_gemm_workspace_bytes(desc, T, topk, E, N, K, bm)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    twd = to_dev(inp["topk_weights"].reshape(-1)) if tw else None
    say(f"[w8a16 moe fp8={fp8}] T={T} topk={topk} E={E} N={N} K={K} bm={bm}")
    hq.hq_moe_grouped_gemm(desc, T, topk, E, N, K, to_dev(inp["x"]), None, w, so, be, npad, bm, twd, y, ws, wsb)
    torch.cuda.synchronize()
    ref, _, valid = oracle.ref_moe_gemm(inp["x"], ids, lambda e: experts[e], N, E, 128,
                                        topk_weights=inp["topk_weights"] if tw else None, cols=cols)
    assert valid.all()
    got = y.cpu().numpy()
    check_float(got if cols is None else got[:, cols], ref, f"w8a16 moe fp8={fp8} T={T} bm={bm}")


@pytest.mark.parametrize("fp8", FMTS)
@pytest.mark.parametrize("T,topk,E,N,K,bm", [
    (5, 2, 4, 64, 256, 16), (64, 8, 16, 512, 1024, 16), (150, 8, 8, 512, 384, 32),
    (400, 8, 16, 1024, 768, 64), (200, 8, 32, 272, 384, 64), (600, 8, 16, 512, 512, 128),
    (300, 8, 64, 384, 640, 128),   # 128-row blocks on 128 x 128 tiles
])
def test_w8a16_moe(fp8, T, topk, E, N, K, bm):
    _moe(fp8, T, topk, E, N, K, bm, 1400 + T)


@pytest.mark.parametrize("fp8", FMTS)
@pytest.mark.parametrize("T", [8, 512])
def test_w8a16_moe_full_size_sampled(fp8, T):
    E, topk, N, K = 256, 8, 4096, 7168
    bm = hq.hq_moe_block_m(_desc(fp8), T, topk, E, N, K)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(T).integers(0, N, 96)]))
    _moe(fp8, T, topk, E, N, K, bm, 14, tw=False, random_codes=True, cols=cols)


@pytest.mark.parametrize("fp8", FMTS)
def test_w8a16_grouped(fp8):
    R, E, N, K = 300, 6, 512, 512
    counts = [80, 0, 120, 40, 59, 1]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.normal_bf16(synth.rng(1500, R), (R, K))
    experts = _experts(15, [e for e in range(E) if counts[e]], N, K, fp8)
    desc = _desc(fp8)
    w = _stack(desc, E, N, K, experts)
    wsb = hq.hq_grouped_gemm_workspace_bytes(desc, R, E, N, K)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    y = torch.empty((R, N), dtype=torch.int16, device=DEV)
    say(f"[w8a16 grouped fp8={fp8}]")
    hq.hq_grouped_gemm(desc, R, E, N, K, to_dev(x), None, w, to_dev(offs), y, ws, wsb)
    torch.cuda.synchronize()
    ref, _, valid = oracle.ref_grouped_gemm(x, offs, lambda e: experts[e], N, E, 128)
    assert valid.all()
    check_float(y.cpu().numpy(), ref, f"w8a16 grouped fp8={fp8}")
