"""GPU parity of the dense fused-dequantization GEMM against the CPU oracle, through the C ABI.

Small and ragged shapes compare every output; the full benchmark shapes compare a sampled set of
rows and columns (the oracle computes just those) in the launch configuration the benchmark
uses. Tolerances: float paths relative L2 <= 2e-3 and max-abs <= 2e-2 * max|ref| against the
unrounded fp64 oracle; W8A8 int32 accumulator bit-exact and bf16 output within 1 ulp."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import check_float, check_ulp, every_configuration, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu


def _sample(M, N, rng, nr=48, nc=96):
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, nr)])) if M > nr else np.arange(M)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, nc)]))
    return rows, cols


# ---- WNA16 -------------------------------------------------------------------------------------
WNA16_SMALL = [
    # (M, N, K, asym)
    (16, 256, 512, False),    # the tiny dense W4A16 workload
    (1, 256, 512, False),
    (37, 272, 384, False),    # ragged M, odd number of channel tiles
    (5, 48, 128, False),      # a single K unit
    (64, 512, 1024, False),
    (100, 1024, 2048, False),
    (1, 2048, 1024, True),
    (16, 1024, 4096, True),
    (33, 304, 512, True),
    (128, 512, 512, True),
    (300, 256, 1024, True),
    (600, 512, 640, True),    # 128 x 256 ping-pong tiles, ragged M
    (600, 480, 512, False),   # no pipelined tile divides N: LDS-tiled fallback
    (600, 480, 384, True),    # LDS-tiled fallback with K/128 = 3 groups
    (150, 256, 896, True),    # 128 x 128 ping-pong tiles, K/128 = 7 groups
    (24, 512, 1024, True),    # two 16-row blocks per skinny workgroup
    (300, 512, 4224, True),   # 128 x 256 ping-pong tiles, K/128 = 33 groups (two 32-group blocks)
]


@pytest.mark.parametrize("M,N,K,asym", WNA16_SMALL)
def test_wna16_small(M, N, K, asym):
    say(f"[wna16] M={M} N={N} K={K} asym={asym}")
    d = synth.make_wna16(100 + asym, M, N, K, asym=asym)
    desc = hq.DESC_W4A16_ASYM if asym else hq.DESC_W4A16_SYM
    w = prepack(desc, 1, N, K, d["wq"], d["scales"], d.get("zeros"))
    y = gemm(desc, M, N, K, to_dev(d["x"]), None, w)
    ref, _ = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d.get("zeros"), 128)
    check_float(y, ref, "wna16")


@pytest.mark.parametrize("asym", [True, False])
def test_wna16_every_kernel_configuration(asym, monkeypatch):
    """INT4 W4A16 at a ragged M over 256 rows, N = 512, six groups, in every configuration."""
    M, N, K = 600, 512, 768
    d = synth.make_wna16(1304 + asym, M, N, K, asym=asym)
    desc = hq.DESC_W4A16_ASYM if asym else hq.DESC_W4A16_SYM
    w = prepack(desc, 1, N, K, d["wq"], d["scales"], d.get("zeros"))
    x = to_dev(d["x"])
    ref, _ = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d.get("zeros"), 128)
    ran = every_configuration(desc, M, N, K, lambda: gemm(desc, M, N, K, x, None, w),
                              lambda y, what: check_float(y, ref, f"wna16 asym={asym} {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 1, 2, 3))


def test_wna16_deterministic():
    M, N, K = 3, 512, 4096
    d = synth.make_wna16(7, M, N, K, asym=True)
    w = prepack(hq.DESC_W4A16_ASYM, 1, N, K, d["wq"], d["scales"], d["zeros"])
    x = to_dev(d["x"])
    y1 = gemm(hq.DESC_W4A16_ASYM, M, N, K, x, None, w)
    y2 = gemm(hq.DESC_W4A16_ASYM, M, N, K, x, None, w)
    assert np.array_equal(y1, y2)


@pytest.fixture(scope="module")
def cfg2_weights():
    N, K = 14336, 4096
    d = synth.make_wna16(2, 1, N, K, asym=True)
    w = prepack(hq.DESC_W4A16_ASYM, 1, N, K, d["wq"], d["scales"], d["zeros"])
    return d, w


@pytest.mark.parametrize("M", [1, 16, 128, 1024, 8192])
def test_wna16_full_size_sampled(cfg2_weights, M):
    N, K = 14336, 4096
    d, w = cfg2_weights
    say(f"[wna16 full] M={M} N={N} K={K}")
    x = synth.normal_bf16(synth.rng(2, M), (M, K))
    y = gemm(hq.DESC_W4A16_ASYM, M, N, K, to_dev(x), None, w)
    rows, cols = _sample(M, N, np.random.default_rng(M))
    ref, _ = oracle.ref_wna16(x, d["wq"], d["scales"], d["zeros"], 128, rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"wna16 M={M}")

def test_wna16_past_32bit_activation_offsets():
    """M x K bf16 activations past 4 GiB: the direct-to-LDS kernels address activation rows with
    32-bit offsets, so the dispatcher moves such a call to the LDS-tiled kernel (64-bit row
    addresses). Rows repeat with a prime period, so a row read at a wrapped offset would hold other
    values; sampled rows on both sides of the 4 GiB mark against the oracle."""
    M, N, K = 262144 + 300, 256, 8192
    desc = hq.DESC_W4A16_ASYM
    assert hq.hq_gemm_plan(desc, M, N, K)[0] == 1
    d = synth.make_wna16(1700, 997, N, K, asym=True)
    x = synth.periodic_rows(d["x"], M)
    say(f"[wna16 past 4 GiB] M={M} N={N} K={K}: {x.nbytes / 2**30:.2f} GiB of activations")
    w = prepack(desc, 1, N, K, d["wq"], d["scales"], d["zeros"])
    y = gemm(desc, M, N, K, to_dev(x), None, w)
    rows = np.unique(np.concatenate([[0, 262143, 262144, 262145, M - 1],
                                     np.random.default_rng(3).integers(0, M, 40)]))
    ref, _ = oracle.ref_wna16(x, d["wq"], d["scales"], d["zeros"], 128, rows=rows)
    del x
    check_float(y[rows], ref, "wna16 past 4 GiB")


# ---- W8A8 -------------------------------------------------------------------------------------
W8A8_SMALL = [(1, 256, 8192), (64, 512, 1024), (7, 272, 320), (16, 256, 64),
              (200, 512, 2048),    # 64 x 128 pipelined tiles, four waves of 64 x 32
              (100, 512, 1024),    # 64 x 64 pipelined tiles, ragged M
              (20, 512, 1024),     # two 16-row blocks per skinny workgroup
              (700, 384, 1024),    # 256 x 128 ping-pong tiles
              (400, 256, 640),     # 128 x 128 ping-pong tiles, four LDS slots
              (300, 256, 128),     # four slots, one K step
              (480, 384, 256),     # four slots, two K steps
              (1100, 512, 1024),   # 256 x 256 pipelined tiles, ragged M
              (2100, 640, 512),    # 256 x 256 tiles do not divide N: LDS-tiled fallback
              (2050, 512, 640)]    # 256 x 256 pipelined tiles, ragged M


@pytest.mark.parametrize("M,N,K", W8A8_SMALL)
def test_w8a8_small(M, N, K):
    say(f"[w8a8] M={M} N={N} K={K}")
    d = synth.make_w8a8(300, M, N, K)
    w = prepack(hq.DESC_W8A8, 1, N, K, d["wq"], d["s_ch"])
    xq, st = to_dev(d["xq"]), to_dev(d["s_tok"])
    acc = gemm(hq.DESC_W8A8_I32, M, N, K, xq, st, w, out_dtype=torch.int32)
    y = gemm(hq.DESC_W8A8, M, N, K, xq, st, w)
    ref_acc, _, ref_bits = oracle.ref_w8a8(d["xq"], d["s_tok"], d["wq"], d["s_ch"])
    assert np.array_equal(acc.astype(np.int64), ref_acc), "int32 accumulator not bit-exact"
    check_ulp(y, ref_bits, "w8a8 bf16")


@pytest.mark.parametrize("M", [1, 64, 512, 4096])
def test_w8a8_full_size_sampled(M):
    N = K = 8192
    say(f"[w8a8 full] M={M}")
    d = synth.make_w8a8(3, M, N, K)
    w = prepack(hq.DESC_W8A8, 1, N, K, d["wq"], d["s_ch"])
    xq, st = to_dev(d["xq"]), to_dev(d["s_tok"])
    acc = gemm(hq.DESC_W8A8_I32, M, N, K, xq, st, w, out_dtype=torch.int32)
    y = gemm(hq.DESC_W8A8, M, N, K, xq, st, w)
    rows, cols = _sample(M, N, np.random.default_rng(M))
    ref_acc, _, ref_bits = oracle.ref_w8a8(d["xq"], d["s_tok"], d["wq"], d["s_ch"], rows=rows, cols=cols)
    assert np.array_equal(acc[np.ix_(rows, cols)].astype(np.int64), ref_acc)
    check_ulp(y[np.ix_(rows, cols)], ref_bits, f"w8a8 M={M}")


def test_w8a8_every_kernel_configuration(monkeypatch):
    """W8A8 at a ragged M over 256 rows, N = 512, six K steps: int32 accumulator bit-exact in
    every configuration."""
    M, N, K = 600, 512, 768
    d = synth.make_w8a8(1302, M, N, K)
    w = prepack(hq.DESC_W8A8, 1, N, K, d["wq"], d["s_ch"])
    xq, st = to_dev(d["xq"]), to_dev(d["s_tok"])
    ref_acc, _, _ = oracle.ref_w8a8(d["xq"], d["s_tok"], d["wq"], d["s_ch"])

    def check(acc, what):
        assert np.array_equal(acc.astype(np.int64), ref_acc), f"w8a8 {what}: accumulator not bit-exact"

    ran = every_configuration(hq.DESC_W8A8_I32, M, N, K,
                               lambda: gemm(hq.DESC_W8A8_I32, M, N, K, xq, st, w, out_dtype=torch.int32),
                               check, monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 1, 2, 3))


# ---- W4A8-MXFP4 -------------------------------------------------------------------------------
W4A8_SMALL = [(1, 512, 7168), (32, 256, 1024), (3, 272, 384), (16, 64, 128), (130, 512, 1024),
              (500, 256, 1024),    # 64 x 64 pipelined tiles, ragged M
              (700, 256, 1024),    # 64 x 128 pipelined tiles
              (1200, 512, 768),    # 128 x 128 pipelined tiles
              (1600, 512, 384),    # 128 x 128 pipelined tiles, ragged M, 3 K steps
              (2500, 512, 640),    # 128 x 256 pipelined tiles (eight waves), ragged M
              (1600, 320, 640),    # N % 128 != 0: the LDS-tiled kernel
              (3200, 256, 384),    # 256 x 256 pipelined tiles, ragged M
              (48, 256, 1024),     # 33..64 rows: two 32-row skinny blocks of 32 channels
              (64, 512, 2048),
              (100, 512, 1024),    # 65..128 rows: four 32-row blocks of 64 channels, ragged M
              (128, 256, 1536)]


@pytest.mark.parametrize("M,N,K", W4A8_SMALL)
def test_w4a8_small(M, N, K):
    say(f"[w4a8] M={M} N={N} K={K}")
    d = synth.make_w4a8(400, M, N, K)
    w = prepack(hq.DESC_W4A8_MXFP4, 1, N, K, d["wq"], d["scales"])
    y = gemm(hq.DESC_W4A8_MXFP4, M, N, K, to_dev(d["xq"]), to_dev(d["s_tok"]), w)
    ref, _ = oracle.ref_w4a8(d["xq"], d["s_tok"], d["wq"], d["scales"])
    check_float(y, ref, "w4a8")


def test_w4a8_every_kernel_configuration(monkeypatch):
    """W4A8-MXFP4 at a ragged M over 256 rows, N = 512, six K steps, in every configuration."""
    M, N, K = 600, 512, 768
    d = synth.make_w4a8(1303, M, N, K)
    w = prepack(hq.DESC_W4A8_MXFP4, 1, N, K, d["wq"], d["scales"])
    xq, st = to_dev(d["xq"]), to_dev(d["s_tok"])
    ref, _ = oracle.ref_w4a8(d["xq"], d["s_tok"], d["wq"], d["scales"])
    ran = every_configuration(hq.DESC_W4A8_MXFP4, M, N, K,
                               lambda: gemm(hq.DESC_W4A8_MXFP4, M, N, K, xq, st, w),
                               lambda y, what: check_float(y, ref, f"w4a8 {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 1, 2, 3))


@pytest.mark.parametrize("M", [1, 32, 64, 128, 256, 2048, 8192])
def test_w4a8_full_size_sampled(M):
    N, K = 4096, 7168
    say(f"[w4a8 full] M={M}")
    d = synth.make_w4a8(4, M, N, K)
    w = prepack(hq.DESC_W4A8_MXFP4, 1, N, K, d["wq"], d["scales"])
    y = gemm(hq.DESC_W4A8_MXFP4, M, N, K, to_dev(d["xq"]), to_dev(d["s_tok"]), w)
    rows, cols = _sample(M, N, np.random.default_rng(M))
    ref, _ = oracle.ref_w4a8(d["xq"], d["s_tok"], d["wq"], d["scales"], rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"w4a8 M={M}")


def test_w4a8_block_scale_extremes():
    """Block exponents far from 127 (the e8m0 operand path) and a zero block."""
    M, N, K = 4, 32, 256
    d = synth.make_w4a8(401, M, N, K)
    g = np.random.default_rng(0)
    d["scales"] = g.integers(100, 150, d["scales"].shape).astype(np.uint8)
    d["scales"][0, 0] = 0
    w = prepack(hq.DESC_W4A8_MXFP4, 1, N, K, d["wq"], d["scales"])
    y = gemm(hq.DESC_W4A8_MXFP4, M, N, K, to_dev(d["xq"]), to_dev(d["s_tok"]), w)
    ref, _ = oracle.ref_w4a8(d["xq"], d["s_tok"], d["wq"], d["scales"])
    check_float(y, ref, "w4a8 scale extremes")
