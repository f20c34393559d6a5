"""GPU parity of the MoE grouped GEMM and the grouped GEMM with quantized activations: W4A8 (MXFP4
experts, FP8 e4m3 tokens; oracle float bar), W8A8 (INT8 experts, INT8 tokens; within 1 bf16 ulp
of the exactly rounded result), block-scaled FP8 (e4m3 experts with 128 x 128 block scales,
e4m3 tokens with a scale per 128 k), W4A4 and W4A8-MXFP8 (MXFP4 experts, MXFP4 / MXFP8 tokens
with e8m0 scales per 32 k); float formats at the oracle float bar."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, check_ulp, moe_random_shapes, prepack, say, to_dev

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0
FORMATS = {
    # name: (descriptor, oracle activation kind, per-token quantizer, expert generator, random expert)
    "w4a8": (hq.DESC_W4A8_MXFP4, "e4m3", synth.quantize_fp8_rows,
             lambda seed, e, N, K: synth.make_moe_weights_expert_mx(seed, e, N, K), synth.random_mxfp4_expert),
    "w8a8": (hq.DESC_W8A8, "int8", synth.quantize_int8_rows,
             lambda seed, e, N, K: synth.make_moe_weights_expert_w8a8(seed, e, N, K), synth.random_int8_expert),
    "fp8b": (hq.DESC_W8A8_FP8_BLOCK, "fp8b", lambda x: synth.quantize_fp8_blocks(x, 1, 128),
             lambda seed, e, N, K: synth.make_moe_weights_expert_fp8b(seed, e, N, K), synth.random_fp8b_expert),
    "w4a4": (hq.DESC_W4A4_MXFP4, "mxfp4", lambda x: tuple(synth.quantize_mxfp4(x).values()),
             lambda seed, e, N, K: synth.make_moe_weights_expert_mx(seed, e, N, K), synth.random_mxfp4_expert),
    "w4a8mx": (hq.DESC_W4A8_MXFP8, "mxfp8", synth.quantize_mxfp8_rows,
               lambda seed, e, N, K: synth.make_moe_weights_expert_mx(seed, e, N, K), synth.random_mxfp4_expert),
}
ALL = ["w4a8", "w8a8", "fp8b", "w4a4", "w4a8mx"]


def _ref(act, xq, s, ids, experts, N, E, topk_weights=None, cols=None):
    if act in ("mxfp4", "mxfp8"):
        return oracle.ref_moe_gemm_mx(xq, s, ids, lambda e: experts[e], N, E, act,
                                      topk_weights=topk_weights, cols=cols)
    if act == "fp8b":
        return oracle.ref_moe_gemm_fp8_block(xq, s, ids, lambda e: experts[e], N, E,
                                             topk_weights=topk_weights, cols=cols)
    return oracle.ref_moe_gemm_q(xq, s, ids, lambda e: experts[e], N, E, act, topk_weights=topk_weights,
                                 cols=cols)


def _stack(desc, E, N, K, experts):
    stride = hq.hq_prepacked_bytes(desc, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        sc = wd["scales"] if "scales" in wd else wd["ws"] if "ws" in wd else wd["s_ch"]
        w[e * stride:(e + 1) * stride] = prepack(desc, 1, N, K, wd["wq"], sc)
    return w


def _experts(fmt, seed, active, N, K, random_codes):
    _, _, _, make, rand = FORMATS[fmt]
    if random_codes:
        return {int(e): rand(synth.rng(seed, 8, int(e)), N, K) for e in active}
    return {int(e): make(seed, int(e), N, K) for e in active}


def _check(fmt, y, ref, bits, what):
    if fmt == "w8a8":
        check_ulp(y, bits, what)
    else:
        check_float(y, ref, what)


def _moe(fmt, T, topk, E, N, K, bm, with_weights, seed, random_codes=False, cols=None):
    desc, act, quant, _, _ = FORMATS[fmt]
    inp = synth.make_moe_inputs(seed, T, K, E, topk)
    xq, s_tok = quant(synth.bf16_bits_to_f32(inp["x"]))
    ids = inp["topk_ids"]
    experts = _experts(fmt, seed, np.unique(ids), N, K, random_codes)
    w = _stack(desc, E, N, K, experts)
    cap = hq.hq_moe_align_capacity(T, topk, E, bm)
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=DEV)
    block_expert = torch.empty(cap // bm, dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    npad = torch.empty(1, dtype=torch.int32, device=DEV)
    hq.hq_moe_align(to_dev(ids.astype(np.int32)), T, topk, E, bm, sorted_ids, block_expert, offs, npad)
    y = torch.full((T * topk, N), NAN_BF16, dtype=torch.int16, device=DEV)
    tw = inp["topk_weights"] if with_weights else None
    say(f"[moe {fmt}] T={T} topk={topk} E={E} N={N} K={K} bm={bm} weights={with_weights}")
    wsb = hq.hq_moe_gemm_workspace_bytes(desc, T, topk, E, N, K, bm)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    hq.hq_moe_grouped_gemm(desc, T, topk, E, N, K, to_dev(xq), to_dev(s_tok), w, sorted_ids, block_expert,
                           npad, bm, None if tw is None else to_dev(tw.reshape(-1)), y, ws, wsb)
    torch.cuda.synchronize()
    y = y.cpu().numpy().view(np.uint16)
    ref, bits, valid = _ref(act, xq, s_tok, ids, experts, N, E, topk_weights=tw, cols=cols)
    assert valid.all()
    got = y if cols is None else y[:, cols]
    _check(fmt, got, ref, bits, f"moe {fmt} T={T} bm={bm}")


MOE_CASES = [
    (5, 2, 4, 64, 256, 16, False),        # 16-row blocks, skinny kernel
    (64, 8, 16, 512, 1024, 16, True),
    (300, 4, 8, 256, 512, 32, False),     # 32-row blocks: skinny kernel
    (200, 8, 32, 272, 384, 64, True),     # N = 17 channel tiles: skinny kernel, 64-row blocks
    (300, 8, 16, 256, 640, 64, True),     # ping-pong 64 x 256, K/128 = 5
    (400, 8, 16, 1024, 768, 64, True),    # ping-pong 64 x 512 (W4A8) / 64 x 256 (W8A8)
    (600, 8, 16, 512, 512, 128, True),    # 128-row blocks: ping-pong 128 x 256
    (300, 8, 64, 256, 640, 128, False),   # 128-row blocks, mostly padding, K/128 = 5
    (300, 8, 64, 384, 640, 128, False),   # 128-row blocks on 128 x 128 tiles (N % 256 != 0)
]


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("T,topk,E,N,K,bm,tw", MOE_CASES)
def test_moe_q_small(fmt, T, topk, E, N, K, bm, tw):
    if fmt == "fp8b" and N % 128:
        pytest.skip("block-scaled FP8 weights need N % 128 == 0 (128 x 128 scale blocks)")
    _moe(fmt, T, topk, E, N, K, bm, tw, 600 + T)


@pytest.mark.parametrize("fmt", ALL)
def test_moe_q_random_shapes(fmt):
    """Six seeded random MoE problems per format (`moe_random_shapes`; block-scaled FP8 with N a
    multiple of 128)."""
    for i, case in enumerate(moe_random_shapes(33 + ALL.index(fmt), 6, 128 if fmt == "fp8b" else 16)):
        _moe(fmt, *case, 1700 + i)


@pytest.mark.parametrize("T,topk,E,N,K,bm,tw", [
    (600, 8, 16, 512, 512, 128, True),     # 128-row blocks: 128 x 256 / 128 x 128 tiles
    (300, 8, 64, 256, 640, 128, False),    # 128-row blocks, mostly padding, K/128 = 5
    (400, 8, 16, 512, 768, 64, True),      # 64-row blocks: 64 x 128 / 64 x 64 tiles
])
def test_moe_fp8b_pipelined_configurations(T, topk, E, N, K, bm, tw, monkeypatch):
    """Block-scaled FP8 experts on every pipelined configuration whose tile rows equal the block
    size (the tuning override may name any of them); the others are refused before any launch."""
    ran = 0
    for cfg in range(hq.hq_kernel_config_count(2)):
        monkeypatch.setenv("HQ_TUNE", f"kind=2,cfg={cfg},split=1")
        try:
            _moe("fp8b", T, topk, E, N, K, bm, tw, 900 + T)
        except hq.HQError as e:
            assert e.status == hq.HQ_ERR_UNSUPPORTED, str(e)
            continue
        ran += 1
    monkeypatch.delenv("HQ_TUNE")
    assert ran >= 2


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("T", [8, 128, 1024])
def test_moe_q_full_size_sampled(fmt, T):
    """DeepSeek-V3 gate_up shape (256 experts, top-8, K = 7168, N = 4096) at the block size the
    library recommends (16, 32, 64 rows for T = 8, 128, 1024; 128 rows at T = 1024 for block-scaled
    FP8), sampled output columns."""
    E, topk, N, K = 256, 8, 4096, 7168
    desc = FORMATS[fmt][0]
    bm = hq.hq_moe_block_m(desc, T, topk, E, N, K)
    cols = np.unique(np.concatenate([[0, N - 1], synth.rng(T, 3).integers(0, N, 96)]))
    _moe(fmt, T, topk, E, N, K, bm, True, 7, random_codes=True, cols=cols)


def _grouped(fmt, R, E, N, K, counts, seed, lead=0):
    desc, act, quant, _, _ = FORMATS[fmt]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64) + lead
    x = synth.bf16_bits_to_f32(synth.normal_bf16(synth.rng(seed, R), (R, K)))
    xq, s_row = quant(x)
    experts = _experts(fmt, seed, [e for e in range(E) if counts[e] > 0], N, K, False)
    w = _stack(desc, E, N, K, experts)
    wsb = hq.hq_grouped_gemm_workspace_bytes(desc, R, E, N, K)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    y = torch.full((R, N), NAN_BF16, dtype=torch.int16, device=DEV)
    say(f"[grouped {fmt}] R={R} E={E} N={N} K={K} offsets[:8]={offs[:8].tolist()}")
    hq.hq_grouped_gemm(desc, R, E, N, K, to_dev(xq), to_dev(s_row), w, to_dev(offs.astype(np.int32)),
                       y, ws, wsb)
    torch.cuda.synchronize()
    y = y.cpu().numpy().view(np.uint16)
    # the grouped GEMM is the MoE GEMM with top-1 routing: row r goes to the expert whose range
    # holds it, rows in no range to none
    ids = np.full((R, 1), -1, np.int64)
    for e in range(E):
        ids[max(offs[e], 0):min(offs[e + 1], R), 0] = e
    ref, bits, valid = _ref(act, xq, s_row, ids, experts, N, E)
    _check(fmt, y[valid], ref[valid], bits[valid], f"grouped {fmt} R={R}")
    assert (y[~valid] == NAN_BF16).all(), "rows outside every range must not be written"


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("R,E,N,K,counts,lead", [
    (100, 4, 256, 512, [30, 0, 50, 20], 0),
    (1000, 8, 512, 1024, [400, 10, 0, 250, 1, 200, 39, 100], 0),
    (7, 16, 128, 256, [0, 2, 0, 0, 1, 0, 0, 0, 3, 0, 0, 0, 0, 0, 1, 0], 0),
    (120, 6, 256, 384, [10, 30, 0, 25, 40, 5], 4),        # rows 0-3 and 114-119 in no range
])
def test_grouped_q(fmt, R, E, N, K, counts, lead):
    _grouped(fmt, R, E, N, K, counts, 80 + R, lead)
