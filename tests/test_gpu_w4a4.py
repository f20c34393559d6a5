"""GPU parity of the W4A4-MXFP4 path (MXFP4 activations x MXFP4 weights on the fp4 scaled MFMA)
and of the MXFP4 activation quantizer, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, every_configuration, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

D = hq.DESC_W4A4_MXFP4


def _gemm(d, M, N, K):
    w = prepack(D, 1, N, K, d["wq"], d["scales"])
    # the activations' e8m0 block scales travel through the a_scale pointer
    xs = to_dev(np.ascontiguousarray(d["xs"]).reshape(-1))
    return gemm(D, M, N, K, to_dev(d["xq"]), xs, w)


@pytest.mark.parametrize("M,N,K", [
    (1, 512, 7168), (32, 256, 1024), (3, 272, 384), (16, 64, 128), (130, 512, 1024),
    (100, 512, 1024),    # 65..128 rows: four 32-row skinny blocks of 64 channels, ragged M
    (128, 256, 1536),
    (64, 256, 1024),     # 33..64 rows: two 32-row blocks
    (300, 256, 512),     # pipelined 64 x 64 (four stages), ragged M
    (150, 256, 512),     # skinny, 64-row blocks, ragged M
    (700, 384, 640),     # pipelined 64 x 128 (four stages), 5 K steps
    (1000, 256, 128),    # pipelined 64 x 128, one K step
    (900, 128, 256),     # pipelined 64 x 128, two K steps
    (1500, 256, 640),    # pipelined 128 x 256, eight waves of 64 x 64, ragged M, 5 K steps
    (1200, 384, 512),    # N % 256 != 0 above 1024 rows: ping-pong 128 x 128 fallback
    (4200, 256, 512),    # pipelined 128 x 256 (four waves of 64 x 128, three stages), ragged M
    (2300, 512, 384),    # pipelined 128 x 256, three K steps
    (257, 128, 256),
])
def test_w4a4_small(M, N, K):
    say(f"[w4a4] M={M} N={N} K={K}")
    d = synth.make_w4a4(600, M, N, K)
    y = _gemm(d, M, N, K)
    ref, _ = oracle.ref_w4a4(d["xq"], d["xs"], d["wq"], d["scales"])
    check_float(y, ref, "w4a4")


def test_w4a4_every_kernel_configuration(monkeypatch):
    """Ragged M over 256 rows, N = 512, six K steps, in every configuration that fits."""
    M, N, K = 600, 512, 768
    d = synth.make_w4a4(1306, M, N, K)
    ref, _ = oracle.ref_w4a4(d["xq"], d["xs"], d["wq"], d["scales"])
    ran = every_configuration(D, M, N, K, lambda: _gemm(d, M, N, K),
                              lambda y, what: check_float(y, ref, f"w4a4 {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 2, 3))


@pytest.mark.parametrize("M", [1, 32, 256, 2048, 8192])
def test_w4a4_full_size_sampled(M):
    N, K = 4096, 7168
    say(f"[w4a4 full] M={M}")
    d = synth.make_w4a4(4, M, N, K)
    y = _gemm(d, M, N, K)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 96)]))
    ref, _ = oracle.ref_w4a4(d["xq"], d["xs"], d["wq"], d["scales"], rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"w4a4 M={M}")


def test_w4a4_past_32bit_activation_offsets():
    """MXFP4 activation codes past 4 GiB: the call leaves the direct-to-LDS kernels (32-bit row
    offsets) for the small-M kernel (64-bit row addresses); rows repeat with a prime period, so a
    wrapped row would hold other values; sampled rows around the 4 GiB mark against the oracle."""
    M, N, K = 2 ** 20 + 100, 128, 8192
    assert hq.hq_gemm_plan(D, M, N, K)[0] == 0
    d = synth.make_w4a4(1701, 997, N, K)
    d = dict(d, xq=synth.periodic_rows(d["xq"], M), xs=synth.periodic_rows(d["xs"], M))
    say(f"[w4a4 past 4 GiB] M={M} N={N} K={K}: {d['xq'].nbytes / 2**30:.2f} GiB of codes")
    y = _gemm(d, M, N, K)
    rows = np.unique(np.concatenate([[0, 2 ** 20 - 1, 2 ** 20, M - 1], np.random.default_rng(4).integers(0, M, 40)]))
    ref, _ = oracle.ref_w4a4(d["xq"], d["xs"], d["wq"], d["scales"], rows=rows)
    check_float(y[rows], ref, "w4a4 past 4 GiB")


def test_w4a4_block_scale_extremes():
    """Activation and weight block scales spread over 2^-40 .. 2^40 per block (products stay in
    fp32 range): every block scale must reach its own 32 k."""
    M, N, K = 64, 256, 1024
    d = synth.make_w4a4(601, M, N, K)
    g = np.random.default_rng(5)
    d["xs"] = g.integers(87, 168, d["xs"].shape).astype(np.uint8)
    d["scales"] = g.integers(87, 168, d["scales"].shape).astype(np.uint8)
    y = _gemm(d, M, N, K)
    ref, _ = oracle.ref_w4a4(d["xq"], d["xs"], d["wq"], d["scales"])
    check_float(y, ref, "w4a4 scale extremes", rounding_floor=True)


def _quantize_gpu(x_bits):
    M, K = x_bits.shape
    xq = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    xs = torch.full((M, K // 32), 0x5A, dtype=torch.uint8, device=DEV)
    hq.hq_quantize_activations(hq.HQ_ACT_MXFP4, M, K, to_dev(x_bits.view(np.int16)), xq, xs)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy()


def test_mxfp4_activation_quantizer_bit_exact():
    """Random N(0,1) and wide-range rows, random finite bf16 bit patterns (subnormals
    included), all-zero and all-subnormal blocks, ties: codes and scales bit-exact."""
    g = np.random.default_rng(21)
    rows = [synth.normal_bf16(g, (40, 512), std=s) for s in (1.0, 1e-3, 1e4)]
    rb = g.integers(0, 0x10000, (64, 512), dtype=np.uint32).astype(np.uint16)
    rows.append(np.where((rb & 0x7F80) == 0x7F80, rb & 0x807F, rb).astype(np.uint16))
    sub = (g.integers(0, 0x80, (16, 512)) | (g.integers(0, 2, (16, 512)) << 15)).astype(np.uint16)
    sub[:8, ::32] = np.arange(1, 9)[:, None] << 7       # block maxima 2^-126 .. 2^-119: e <= -121
    rows.append(sub)
    ties = synth.bf16_bits(np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32), (2, 16)))
    ties[1] = synth.bf16_bits(np.zeros(512, np.float32))
    rows.append(ties)
    x = np.concatenate(rows)
    say(f"[mxfp4 quant] rows={x.shape[0]} K=512")
    q, s = _quantize_gpu(x)
    rq, rs = oracle.quantize_mxfp4_act(x)
    assert np.array_equal(s, rs), np.argwhere(s != rs)[:5]
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:5]


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (333, 7168)])
def test_mxfp4_activation_quantizer_shapes(M, K):
    x = synth.normal_bf16(np.random.default_rng(M), (M, K), std=2.0)
    say(f"[mxfp4 quant] M={M} K={K}")
    q, s = _quantize_gpu(x)
    rq, rs = oracle.quantize_mxfp4_act(x)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)


def test_quantize_then_w4a4_gemm_chain():
    """bf16 activations -> GPU MXFP4 quantizer -> GPU W4A4 GEMM, against the oracle's quantizer
    and GEMM on the same bf16 input."""
    M, N, K = 48, 512, 2048
    x = synth.normal_bf16(np.random.default_rng(7), (M, K))
    w = synth.quantize_mxfp4(np.random.default_rng(8).standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    say("[w4a4 chain]")
    q, s = _quantize_gpu(x)
    y = _gemm({"xq": q, "xs": s, "wq": w["wq"], "scales": w["scales"]}, M, N, K)
    rq, rs = oracle.quantize_mxfp4_act(x)
    ref, _ = oracle.ref_w4a4(rq, rs, w["wq"], w["scales"])
    check_float(y, ref, "w4a4 chain")


def test_w4a4_argument_errors():
    with pytest.raises(hq.HQError):     # the activations' block scales are required
        gemm(D, 4, 256, 512, torch.zeros(4 * 256, dtype=torch.uint8, device=DEV), None,
             torch.zeros(hq.hq_prepacked_bytes(D, 1, 256, 512), dtype=torch.uint8, device=DEV))
    with pytest.raises(hq.HQError):     # K % 32
        hq.hq_quantize_activations(hq.HQ_ACT_MXFP4, 2, 48, torch.zeros(96, dtype=torch.int16, device=DEV),
                                   torch.zeros(48, dtype=torch.uint8, device=DEV),
                                   torch.zeros(4, dtype=torch.uint8, device=DEV))
