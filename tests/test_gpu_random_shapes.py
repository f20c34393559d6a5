"""GPU parity on seeded random shapes: for every dense format, twelve (M, N, K) drawn over the
small-M, mid-M and large-M ranges (M up to 3300, N a multiple of the format's channel granule up to
1024, K a multiple of 128 up to 2048), so that the dispatch tables' choices between the small-M,
pipelined, ping-pong and LDS-tiled kernels are all exercised on ragged shapes the fixed cases do
not name. Each output is compared with the oracle element by element (W8A8: int32 accumulator
bit-exact, bf16 within 1 ulp; float paths: relative L2 <= 2e-3, max-abs <= 2e-2 * max|ref|)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import check_float, check_ulp, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

DESCS = {"w4a16a": hq.DESC_W4A16_ASYM, "w4a16s": hq.DESC_W4A16_SYM, "w2a16": hq.DESC_W2A16_ASYM,
         "w3a16": hq.DESC_W3A16_ASYM, "w8a8": hq.DESC_W8A8, "w4a8": hq.DESC_W4A8_MXFP4,
         "w4a4": hq.DESC_W4A4_MXFP4, "w4a8mx": hq.DESC_W4A8_MXFP8, "w4a16mx": hq.DESC_W4A16_MXFP4,
         "fp8block": hq.DESC_W8A8_FP8_BLOCK, "w8a16": hq.DESC_W8A16_INT8, "f8a16": hq.DESC_W8A16_FP8}


def _shapes(fmt, n, seed):
    g = np.random.default_rng(seed)
    nmul = 128 if fmt == "fp8block" else 16     # 128 x 128 weight scale blocks
    out = []
    while len(out) < n:
        M = int(g.choice([g.integers(1, 65), g.integers(65, 700), g.integers(700, 3300)]))
        N = int(nmul * g.integers(1, 1024 // nmul + 1))
        K = int(128 * g.integers(1, 17))
        if M * N * K <= 6e8:                    # the fp64 oracle stays within a second
            out.append((M, N, K))
    return out


def _run_case(fmt, M, N, K, seed):
    if fmt in ("w4a16a", "w4a16s"):
        asym = fmt == "w4a16a"
        d = synth.make_wna16(seed, M, N, K, asym=asym)
        desc = hq.DESC_W4A16_ASYM if asym else hq.DESC_W4A16_SYM
        w = prepack(desc, 1, N, K, d["wq"], d["scales"], d.get("zeros"))
        y = gemm(desc, M, N, K, to_dev(d["x"]), None, w)
        ref, _ = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d.get("zeros"), 128)
        check_float(y, ref, fmt)
    elif fmt in ("w2a16", "w3a16"):
        mk, rf, desc = ((synth.make_wna2, oracle.ref_wna2, hq.DESC_W2A16_ASYM) if fmt == "w2a16"
                         else (synth.make_wna3, oracle.ref_wna3, hq.DESC_W3A16_ASYM))
        d = mk(seed, M, N, K)
        w = prepack(desc, 1, N, K, d["wq"], d["scales"], d["zeros"])
        y = gemm(desc, M, N, K, to_dev(d["x"]), None, w)
        ref, _ = rf(d["x"], d["wq"], d["scales"], d["zeros"], 128)
        check_float(y, ref, fmt)
    elif fmt == "w8a8":
        d = synth.make_w8a8(seed, M, N, K)
        w = prepack(hq.DESC_W8A8, 1, N, K, d["wq"], d["s_ch"])
        xq, st = to_dev(d["xq"]), to_dev(d["s_tok"])
        acc = gemm(hq.DESC_W8A8_I32, M, N, K, xq, st, w, out_dtype=torch.int32)
        y = gemm(hq.DESC_W8A8, M, N, K, xq, st, w)
        ra, _, rb = oracle.ref_w8a8(d["xq"], d["s_tok"], d["wq"], d["s_ch"])
        assert np.array_equal(acc.astype(np.int64), ra), "w8a8 acc"
        check_ulp(y, rb, fmt)
    elif fmt == "w4a8":
        d = synth.make_w4a8(seed, M, N, K)
        w = prepack(hq.DESC_W4A8_MXFP4, 1, N, K, d["wq"], d["scales"])
        y = gemm(hq.DESC_W4A8_MXFP4, M, N, K, to_dev(d["xq"]), to_dev(d["s_tok"]), w)
        ref, _ = oracle.ref_w4a8(d["xq"], d["s_tok"], d["wq"], d["scales"])
        check_float(y, ref, fmt)
    elif fmt in ("w4a4", "w4a8mx"):
        mk, rf, desc = ((synth.make_w4a4, oracle.ref_w4a4, hq.DESC_W4A4_MXFP4) if fmt == "w4a4"
                         else (synth.make_w4a8mx, oracle.ref_w4a8_mx, hq.DESC_W4A8_MXFP8))
        d = mk(seed, M, N, K)
        w = prepack(desc, 1, N, K, d["wq"], d["scales"])
        y = gemm(desc, M, N, K, to_dev(d["xq"]), to_dev(np.ascontiguousarray(d["xs"]).reshape(-1)), w)
        ref, _ = rf(d["xq"], d["xs"], d["wq"], d["scales"])
        check_float(y, ref, fmt)
    elif fmt == "w4a16mx":
        d = synth.make_w4a16mx(seed, M, N, K)
        w = prepack(hq.DESC_W4A16_MXFP4, 1, N, K, d["wq"], d["scales"])
        y = gemm(hq.DESC_W4A16_MXFP4, M, N, K, to_dev(d["x"]), None, w)
        ref, _ = oracle.ref_w4a16_mx(d["x"], d["wq"], d["scales"])
        check_float(y, ref, fmt)
    elif fmt == "fp8block":
        d = synth.make_w8a8_fp8_block(seed, M, N, K)
        w = prepack(hq.DESC_W8A8_FP8_BLOCK, 1, N, K, d["wq"], d["ws"])
        y = gemm(hq.DESC_W8A8_FP8_BLOCK, M, N, K, to_dev(d["xq"]), to_dev(np.ascontiguousarray(d["xs"], np.float32)), w)
        ref, _ = oracle.ref_w8a8_fp8_block(d["xq"], d["xs"], d["wq"], d["ws"])
        check_float(y, ref, fmt)
    elif fmt in ("w8a16", "f8a16"):
        fp8 = fmt == "f8a16"
        d = synth.make_w8a16(seed, M, N, K, fp8=fp8)
        desc = hq.DESC_W8A16_FP8 if fp8 else hq.DESC_W8A16_INT8
        w = prepack(desc, 1, N, K, d["wq"], d["s_ch"])
        y = gemm(desc, M, N, K, to_dev(d["x"]), None, w)
        ref, _ = oracle.ref_w8a16(d["x"], d["wq"], d["s_ch"], fp8=fp8)
        check_float(y, ref, fmt)


@pytest.mark.parametrize("fmt", sorted(DESCS))
def test_random_shapes(fmt):
    for i, (M, N, K) in enumerate(_shapes(fmt, 12, 7000 + sorted(DESCS).index(fmt))):
        say(f"[random {fmt}] M={M} N={N} K={K} plan={hq.hq_gemm_plan(DESCS[fmt], M, N, K)}")
        _run_case(fmt, M, N, K, 5000 + 37 * i + M)
