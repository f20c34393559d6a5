"""Stream-K (HQ_COMPUTE_STREAM_K): small-M dense calls cut into equal (tile group, K unit) ranges,
one per workgroup, split tile groups summed by the last contributor. Every format against the
oracle at its bar (W8A8: int32 accumulator bit-exact), the full-size decode shapes, repeated calls
(the arrival counters must come back to zero), calls on two streams, and HIP graph replays."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, I32_SENTINEL, check_float, check_ulp, gemm, prepack, say, to_dev
from test_gpu_invariant import _inputs

pytestmark = pytest.mark.gpu

SK = hq.HQ_COMPUTE_STREAM_K
FORMATS = ["w4a16", "w4a16a", "w8a8", "w4a8", "w4a4", "w4a8mx", "w4a16mx", "fp8block", "w8a16", "f8a16",
           "w2a16", "w3a16"]


def _ref(fmt, x, s, std):
    if fmt in ("w4a16", "w4a16a"):
        return oracle.ref_wna16(x, std[0], std[1], std[2], 128)[0]
    if fmt == "w4a8":
        return oracle.ref_w4a8(x, s, std[0], std[1])[0]
    if fmt == "w4a4":
        return oracle.ref_w4a4(x, s, std[0], std[1])[0]
    if fmt == "w4a16mx":
        return oracle.ref_w4a16_mx(x, std[0], std[1])[0]
    if fmt == "fp8block":
        return oracle.ref_w8a8_fp8_block(x, s, std[0], std[1])[0]
    if fmt == "w3a16":
        return oracle.ref_wna3(x, std[0], std[1], std[2], 128)[0]
    if fmt == "w2a16":
        return oracle.ref_wna2(x, std[0], std[1], std[2], 128)[0]
    if fmt in ("w8a16", "f8a16"):
        return oracle.ref_w8a16(x, std[0], std[1], fp8=fmt == "f8a16")[0]
    return oracle.ref_w4a8_mx(x, s, std[0], std[1])[0]


def _dev(x, s):
    return to_dev(np.ascontiguousarray(x)), None if s is None else to_dev(np.ascontiguousarray(s).reshape(-1))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", [(1, 1664, 2560), (3, 2048, 3072), (16, 1408, 3584)])
def test_stream_k_matches_the_oracle(fmt, M, N, K):
    desc, std, x, s = _inputs(fmt, M, N, K)
    skd = hq.with_flags(desc, SK)
    kind, cfg, wgs = hq.hq_gemm_plan(skd, M, N, K)
    say(f"[stream-k] {fmt} M={M} N={N} K={K}: plan {(kind, cfg, wgs)}")
    assert kind == 4, "the shape must run the Stream-K form"
    w = prepack(skd, 1, N, K, *std)
    a, sc = _dev(x, s)
    if fmt == "w8a8":
        acc = gemm(hq.with_flags(hq.DESC_W8A8_I32, SK), M, N, K, a, sc, w, out_dtype=torch.int32)
        ref_acc, _, ref_bits = oracle.ref_w8a8(x, s, std[0], std[1])
        assert np.array_equal(acc.astype(np.int64), ref_acc), "int32 accumulator not bit-exact"
        check_ulp(gemm(skd, M, N, K, a, sc, w), ref_bits, "stream-k w8a8")
        return
    check_float(gemm(skd, M, N, K, a, sc, w), _ref(fmt, x, s, std), f"stream-k {fmt}")


@pytest.fixture(scope="module")
def decode_weights():
    N, K = 14336, 4096
    d = synth.make_wna16(2, 1, N, K, asym=True)
    return d, prepack(hq.DESC_W4A16_ASYM, 1, N, K, d["wq"], d["scales"], d["zeros"])


@pytest.mark.parametrize("M", [1, 16])
def test_stream_k_decode_shape_sampled(decode_weights, M):
    """The dense W4A16 decode shape (N=14336, K=4096): 224 tile groups of the plain launch cut
    over 256 workgroups; three calls in a row give the same bits (counters reset, fixed order)."""
    N, K = 14336, 4096
    d, w = decode_weights
    skd = hq.with_flags(hq.DESC_W4A16_ASYM, SK)
    assert hq.hq_gemm_plan(skd, M, N, K)[0] == 4
    x = synth.normal_bf16(synth.rng(2, M), (M, K))
    xd = to_dev(x)
    ys = [gemm(skd, M, N, K, xd, None, w) for _ in range(3)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(M).integers(0, N, 256)]))
    ref, _ = oracle.ref_wna16(x, d["wq"], d["scales"], d["zeros"], 128, cols=cols)
    check_float(ys[0][:, cols], ref, f"stream-k decode M={M}")


def test_stream_k_on_two_streams_and_in_a_graph(decode_weights):
    """Calls on two streams (each stream its own counters) and replays of a captured graph agree
    bit for bit with an eager call on the default stream."""
    N, K, M = 14336, 4096, 1
    _, w = decode_weights
    skd = hq.with_flags(hq.DESC_W4A16_ASYM, SK)
    x = to_dev(synth.normal_bf16(synth.rng(77, 1), (M, K)))
    wsb = hq.hq_gemm_workspace_bytes(skd, M, N, K)
    ref = gemm(skd, M, N, K, x, None, w)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, wss = [], []
    for i, st in enumerate(streams):
        y = torch.full((M, N), 0x7FC0, dtype=torch.int16, device=DEV)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        with torch.cuda.stream(st):
            for _ in range(4):
                hq.hq_gemm(skd, M, N, K, x, None, w, y, ws, wsb, st)
        outs.append(y)
        wss.append(ws)
    torch.cuda.synchronize()
    for y in outs:
        assert np.array_equal(y.cpu().numpy(), ref)
    g = torch.cuda.CUDAGraph()
    yg = torch.full((M, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wsg = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    with torch.cuda.graph(g):
        hq.hq_gemm(skd, M, N, K, x, None, w, yg, wsg, wsb)
    for r in range(3):
        yg.fill_(0x7FC0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(yg.cpu().numpy(), ref), f"graph replay {r}"
        assert np.array_equal(gemm(skd, M, N, K, x, None, w), ref)   # eager work between replays


def test_stream_k_flag_ignored_where_it_does_not_apply():
    d = hq.with_flags(hq.DESC_W4A16_ASYM, SK)
    assert hq.hq_gemm_plan(d, 17, 14336, 4096)[0] != 4          # more than one row block
    assert hq.hq_gemm_plan(d, 1, 14336 * 2, 4096)[0] != 4       # 448 tile groups fill the chip
    inv = hq.with_flags(hq.DESC_W4A16_ASYM, SK | hq.HQ_COMPUTE_BATCH_INVARIANT)
    assert hq.hq_gemm_plan(inv, 1, 14336, 4096)[0] == 0
