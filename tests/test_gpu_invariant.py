"""Batch invariance (HQ_COMPUTE_BATCH_INVARIANT): an output row is bit-identical whatever M is and
whatever the other rows are, for every format; MoE rows likewise whatever T is. The invariant
results also meet the oracle bar."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, check_ulp, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

INV = hq.HQ_COMPUTE_BATCH_INVARIANT
SUBSETS = [slice(0, 1), slice(5, 21), slice(37, 165), slice(299, 300), slice(0, 300)]


def _inputs(fmt, M, N, K):
    if fmt in ("w4a16", "w4a16a"):
        d = synth.make_wna16(900, M, N, K, asym=fmt == "w4a16a")
        desc = hq.DESC_W4A16_ASYM if fmt == "w4a16a" else hq.DESC_W4A16_SYM
        return desc, (d["wq"], d["scales"], d.get("zeros")), d["x"], None
    if fmt == "w8a8":
        d = synth.make_w8a8(900, M, N, K)
        return hq.DESC_W8A8, (d["wq"], d["s_ch"], None), d["xq"], d["s_tok"]
    if fmt == "w4a8":
        d = synth.make_w4a8(900, M, N, K)
        return hq.DESC_W4A8_MXFP4, (d["wq"], d["scales"], None), d["xq"], d["s_tok"]
    if fmt == "w4a4":
        d = synth.make_w4a4(900, M, N, K)
        return hq.DESC_W4A4_MXFP4, (d["wq"], d["scales"], None), d["xq"], d["xs"]
    if fmt == "fp8block":
        d = synth.make_w8a8_fp8_block(900, M, N, K)
        return hq.DESC_W8A8_FP8_BLOCK, (d["wq"], d["ws"], None), d["xq"], d["xs"]
    if fmt == "w4a16mx":
        d = synth.make_w4a16mx(900, M, N, K)
        return hq.DESC_W4A16_MXFP4, (d["wq"], d["scales"], None), d["x"], None
    if fmt == "w3a16":
        d = synth.make_wna3(900, M, N, K)
        return hq.DESC_W3A16_ASYM, (d["wq"], d["scales"], d["zeros"]), d["x"], None
    if fmt == "w2a16":
        d = synth.make_wna2(900, M, N, K)
        return hq.DESC_W2A16_ASYM, (d["wq"], d["scales"], d["zeros"]), d["x"], None
    if fmt in ("w8a16", "f8a16"):
        d = synth.make_w8a16(900, M, N, K, fp8=fmt == "f8a16")
        desc = hq.DESC_W8A16_FP8 if fmt == "f8a16" else hq.DESC_W8A16_INT8
        return desc, (d["wq"], d["s_ch"], None), d["x"], None
    d = synth.make_w4a8mx(900, M, N, K)
    return hq.DESC_W4A8_MXFP8, (d["wq"], d["scales"], None), d["xq"], d["xs"]


@pytest.mark.parametrize("fmt", ["w4a16", "w4a16a", "w8a8", "w4a8", "w4a4", "w4a8mx", "w4a16mx", "fp8block",
                                 "w8a16", "f8a16", "w2a16", "w3a16"])
def test_rows_do_not_depend_on_the_batch(fmt):
    M, N, K = 300, 512, 1024
    desc, std, x, s = _inputs(fmt, M, N, K)
    inv = hq.with_flags(desc, INV)
    w = prepack(inv, 1, N, K, *std)
    full = None
    say(f"[invariant] {fmt}")
    plans = {hq.hq_gemm_plan(inv, m, N, K) for m in (1, 16, 300, 4096)}
    assert len(plans) == 1, plans
    for sub in SUBSETS:
        xs = x[sub]
        ss = None if s is None else np.ascontiguousarray(s[sub])
        m = xs.shape[0]
        y = gemm(inv, m, N, K, to_dev(np.ascontiguousarray(xs)), None if ss is None else to_dev(ss), w)
        if full is None:
            full = {}
        full[(sub.start, sub.stop)] = y
    ref_rows = full[(0, 300)]
    for (a, b), y in full.items():
        assert np.array_equal(y, ref_rows[a:b]), (fmt, a, b)
    # and the invariant results still meet the oracle bar
    if fmt in ("w4a16", "w4a16a"):
        ref, _ = oracle.ref_wna16(x, std[0], std[1], std[2], 128)
    elif fmt == "w8a8":
        _, _, ref_bits = oracle.ref_w8a8(x, s, std[0], std[1])
        check_ulp(ref_rows, ref_bits, "invariant w8a8")      # the W8A8 bar: within 1 bf16 ulp
        return
    elif fmt == "w4a8":
        ref, _ = oracle.ref_w4a8(x, s, std[0], std[1])
    elif fmt == "w4a4":
        ref, _ = oracle.ref_w4a4(x, s, std[0], std[1])
    elif fmt == "w4a16mx":
        ref, _ = oracle.ref_w4a16_mx(x, std[0], std[1])
    elif fmt == "fp8block":
        ref, _ = oracle.ref_w8a8_fp8_block(x, s, std[0], std[1])
    elif fmt == "w3a16":
        ref, _ = oracle.ref_wna3(x, std[0], std[1], std[2], 128)
    elif fmt == "w2a16":
        ref, _ = oracle.ref_wna2(x, std[0], std[1], std[2], 128)
    elif fmt in ("w8a16", "f8a16"):
        ref, _ = oracle.ref_w8a16(x, std[0], std[1], fp8=fmt == "f8a16")
    else:
        ref, _ = oracle.ref_w4a8_mx(x, s, std[0], std[1])
    check_float(ref_rows, ref, f"invariant {fmt}")


def test_moe_rows_do_not_depend_on_the_batch():
    """A token's routed rows are identical when it is alone (T = 1) and inside T = 200."""
    E, topk, N, K = 16, 4, 256, 512
    desc = hq.with_flags(hq.DESC_W4A16_SYM, INV)
    assert hq.hq_moe_block_m(desc, 200, topk, E, N, K) == 32
    inp = synth.make_moe_inputs(950, 200, K, E, topk)
    ids = inp["topk_ids"]
    experts = {e: synth.make_moe_weights_expert(950, e, N, K) for e in range(E)}
    stride = hq.hq_prepacked_bytes(desc, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(desc, 1, N, K, wd["wq"], wd["scales"])

    def run(x, tids):
        T = x.shape[0]
        cap = hq.hq_moe_align_capacity(T, topk, E, 32)
        so = torch.empty(cap, dtype=torch.int32, device=DEV)
        be = torch.empty(max(cap // 32, 1), dtype=torch.int32, device=DEV)
        offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        npad = torch.empty(1, dtype=torch.int32, device=DEV)
        idd = to_dev(np.ascontiguousarray(tids).astype(np.int32))
        hq.hq_moe_align(idd, T, topk, E, 32, so, be, offs, npad)
        wsb = hq.hq_moe_gemm_workspace_bytes(desc, T, topk, E, N, K, 32)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
        y = torch.empty((T * topk, N), dtype=torch.int16, device=DEV)
        hq.hq_moe_grouped_gemm(desc, T, topk, E, N, K, to_dev(np.ascontiguousarray(x)), None, w, so, be, npad,
                               32, None, y, ws, wsb)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    say("[invariant moe]")
    y_all = run(inp["x"], ids)
    for t in (0, 57, 199):
        y_one = run(inp["x"][t:t + 1], ids[t:t + 1])
        assert np.array_equal(y_one, y_all[t * topk:(t + 1) * topk]), t
    with pytest.raises(hq.HQError):
        hq.hq_moe_grouped_gemm(desc, 1, topk, E, N, K, to_dev(inp["x"][:1]), None, w, torch.zeros(64, dtype=torch.int32, device=DEV),
                               torch.zeros(4, dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV),
                               16, None, torch.empty((topk, N), dtype=torch.int16, device=DEV))
