"""GPU parity of block-scaled FP8 W8A8 (e4m3 x e4m3 on the scaled MFMA, one 128-k step per
128 x 128 weight block, scales applied per step) and of its 128-k block activation quantizer."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, every_configuration, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

D = hq.DESC_W8A8_FP8_BLOCK


def _gemm(d, M, N, K):
    w = prepack(D, 1, N, K, d["wq"], d["ws"])
    return gemm(D, M, N, K, to_dev(d["xq"]), to_dev(np.ascontiguousarray(d["xs"], np.float32)), w)


@pytest.mark.parametrize("M,N,K", [
    (1, 512, 7168), (3, 384, 384), (16, 128, 128), (32, 256, 1024), (64, 512, 512),
    (300, 256, 640),     # ping-pong, ragged M, 5 K steps
    (1000, 384, 512),    # N not a multiple of 256
    (700, 512, 1024),    # ping-pong 128 x 128, four LDS slots
    (1100, 512, 640),    # pipelined 128 x 256 (waves of 32 x 128), ragged M, 5 K steps
    (1000, 256, 128),    # pipelined 128 x 256, one K step (fewer than the three stages)
    (2600, 256, 256),    # pipelined 128 x 256 between 2048 and 3072 rows, ragged M
    (300, 256, 128),     # ping-pong 128 x 128 with four LDS slots, one K step
    (480, 128, 256),     # ping-pong, four slots, two K steps
    (200, 256, 128),     # pipelined 64 x 128 (129..256 rows), one K step
    (100, 256, 128),     # small-M kernel (M <= 128), one K step
    (150, 128, 256),     # pipelined 64 x 128, two K steps
    (90, 128, 256),      # small-M kernel, two K steps
    (2100, 256, 256),    # pipelined 256 x 256 (two stages), two K steps, ragged last tile
    (3000, 512, 384),    # pipelined 256 x 256, three K steps
])
def test_fp8block_small(M, N, K):
    say(f"[fp8block] M={M} N={N} K={K}")
    d = synth.make_w8a8_fp8_block(1300, M, N, K)
    y = _gemm(d, M, N, K)
    ref, _ = oracle.ref_w8a8_fp8_block(d["xq"], d["xs"], d["wq"], d["ws"])
    check_float(y, ref, "fp8block")


def test_fp8block_every_kernel_configuration(monkeypatch):
    """Ragged M over 256 rows, N = 512, six K steps, in every configuration that fits."""
    M, N, K = 600, 512, 768
    d = synth.make_w8a8_fp8_block(1308, M, N, K)
    ref, _ = oracle.ref_w8a8_fp8_block(d["xq"], d["xs"], d["wq"], d["ws"])
    ran = every_configuration(D, M, N, K, lambda: _gemm(d, M, N, K),
                              lambda y, what: check_float(y, ref, f"fp8block {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 2, 3))


@pytest.mark.parametrize("M", [1, 512, 1024, 4096])
def test_fp8block_full_size_sampled(M):
    N = K = 8192
    say(f"[fp8block full] M={M}")
    d = synth.make_w8a8_fp8_block(3, M, N, K)
    y = _gemm(d, M, N, K)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 96)]))
    ref, _ = oracle.ref_w8a8_fp8_block(d["xq"], d["xs"], d["wq"], d["ws"], rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"fp8block M={M}")


def test_fp8block_scale_extremes():
    """Activation and weight block scales spread over 2^-30 .. 2^30: every step must use its own
    row scale and its own block scale."""
    M, N, K = 64, 256, 1024
    d = synth.make_w8a8_fp8_block(1301, M, N, K)
    g = np.random.default_rng(8)
    d["xs"] = (np.exp2(g.integers(-30, 31, d["xs"].shape)) * (1 + g.random(d["xs"].shape))).astype(np.float32)
    d["ws"] = (np.exp2(g.integers(-30, 31, d["ws"].shape)) * (1 + g.random(d["ws"].shape))).astype(np.float32)
    y = _gemm(d, M, N, K)
    ref, _ = oracle.ref_w8a8_fp8_block(d["xq"], d["xs"], d["wq"], d["ws"])
    check_float(y, ref, "fp8block scale extremes", rounding_floor=True)


def _quantize_gpu(x_bits):
    M, K = x_bits.shape
    xq = torch.full((M, K), 0x5A, dtype=torch.uint8, device=DEV)
    xs = torch.full((M, K // 128), -1.0, dtype=torch.float32, device=DEV)
    hq.hq_quantize_activations(hq.HQ_ACT_FP8E4M3_BLOCK128, M, K, to_dev(x_bits.view(np.int16)), xq, xs)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy()


def test_fp8block_activation_quantizer_bit_exact():
    g = np.random.default_rng(23)
    x = np.concatenate([synth.normal_bf16(g, (40, 512), std=s) for s in (1.0, 1e-3, 300.0)])
    x[5, 128:256] = 0                                   # an all-zero block: scale 1, codes 0
    say(f"[fp8block quant] rows={x.shape[0]}")
    q, s = _quantize_gpu(x)
    rq, rs = oracle.quantize_fp8_block_act(x)
    assert np.array_equal(s, rs), np.argwhere(s != rs)[:5]
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:5]


def test_quantize_then_fp8block_gemm_chain():
    M, N, K = 48, 512, 2048
    x = synth.normal_bf16(np.random.default_rng(11), (M, K))
    w = synth.make_w8a8_fp8_block(1302, 1, N, K)
    say("[fp8block chain]")
    q, s = _quantize_gpu(x)
    y = _gemm({"xq": q, "xs": s, "wq": w["wq"], "ws": w["ws"]}, M, N, K)
    rq, rs = oracle.quantize_fp8_block_act(x)
    ref, _ = oracle.ref_w8a8_fp8_block(rq, rs, w["wq"], w["ws"])
    check_float(y, ref, "fp8block chain")


def test_fp8block_argument_errors():
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(hq.HQError):    # N % 128
        hq.hq_gemm(D, 4, 272, 256, buf, buf, buf, buf, buf, 1 << 16)
    with pytest.raises(hq.HQError):    # the activation block scales are required
        hq.hq_gemm(D, 4, 256, 256, buf, None, buf, buf, buf, 1 << 16)
