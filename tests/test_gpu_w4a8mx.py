"""GPU parity of W4A8 with MXFP8 activations (e4m3 x e2m1 on the scaled MFMA, an e8m0 scale per
32-k block on both operands) and of the MXFP8 activation quantizer, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, every_configuration, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu

D = hq.DESC_W4A8_MXFP8


def _gemm(d, M, N, K):
    w = prepack(D, 1, N, K, d["wq"], d["scales"])
    return gemm(D, M, N, K, to_dev(d["xq"]), to_dev(np.ascontiguousarray(d["xs"]).reshape(-1)), w)


@pytest.mark.parametrize("M,N,K", [
    (1, 512, 7168), (32, 256, 1024), (3, 272, 384), (64, 256, 512),
    (300, 256, 512),     # pipelined 64 x 64, ragged M
    (200, 256, 1024),    # skinny, 64-row blocks
    (100, 512, 1024),    # 65..128 rows: four 32-row skinny blocks of 64 channels, ragged M
    (128, 256, 1536),
    (48, 256, 1024),     # 33..64 rows
    (1100, 384, 640),    # ping-pong 128 x 128 fallback (four LDS slots), 5 K steps
    (700, 512, 640),     # pipelined 64 x 128 (four stages)
    (1600, 256, 1024),   # ping-pong 128 x 256, four slots, ragged M
    (800, 256, 128),     # pipelined 64 x 128, one K step
    (2000, 256, 256),    # ping-pong 128 x 256, four slots, two K steps
    (2500, 256, 384),    # pipelined 256 x 256 (two stages), ragged M, three K steps
])
def test_w4a8mx_small(M, N, K):
    say(f"[w4a8mx] M={M} N={N} K={K}")
    d = synth.make_w4a8mx(700, M, N, K)
    y = _gemm(d, M, N, K)
    ref, _ = oracle.ref_w4a8_mx(d["xq"], d["xs"], d["wq"], d["scales"])
    check_float(y, ref, "w4a8mx")


def test_w4a8mx_every_kernel_configuration(monkeypatch):
    """Ragged M over 256 rows, N = 512, six K steps, in every configuration that fits."""
    M, N, K = 600, 512, 768
    d = synth.make_w4a8mx(1307, M, N, K)
    ref, _ = oracle.ref_w4a8_mx(d["xq"], d["xs"], d["wq"], d["scales"])
    ran = every_configuration(D, M, N, K, lambda: _gemm(d, M, N, K),
                              lambda y, what: check_float(y, ref, f"w4a8mx {what}"), monkeypatch)
    assert sum(ran.values()) >= 20 and all(ran.get(k, 0) > 0 for k in (0, 2, 3))


@pytest.mark.parametrize("M", [1, 256, 8192])
def test_w4a8mx_full_size_sampled(M):
    N, K = 4096, 7168
    say(f"[w4a8mx full] M={M}")
    d = synth.make_w4a8mx(4, M, N, K)
    y = _gemm(d, M, N, K)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, 96)]))
    ref, _ = oracle.ref_w4a8_mx(d["xq"], d["xs"], d["wq"], d["scales"], rows=rows, cols=cols)
    check_float(y[np.ix_(rows, cols)], ref, f"w4a8mx M={M}")


def test_w4a8mx_block_scale_extremes():
    M, N, K = 64, 256, 1024
    d = synth.make_w4a8mx(701, M, N, K)
    g = np.random.default_rng(6)
    d["xs"] = g.integers(87, 168, d["xs"].shape).astype(np.uint8)
    d["scales"] = g.integers(87, 168, d["scales"].shape).astype(np.uint8)
    y = _gemm(d, M, N, K)
    ref, _ = oracle.ref_w4a8_mx(d["xq"], d["xs"], d["wq"], d["scales"])
    check_float(y, ref, "w4a8mx scale extremes", rounding_floor=True)


def _quantize_gpu(x_bits):
    M, K = x_bits.shape
    xq = torch.full((M, K), 0x5A, dtype=torch.uint8, device=DEV)
    xs = torch.full((M, K // 32), 0x5A, dtype=torch.uint8, device=DEV)
    hq.hq_quantize_activations(hq.HQ_ACT_MXFP8, M, K, to_dev(x_bits.view(np.int16)), xq, xs)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy()


def test_mxfp8_activation_quantizer_bit_exact():
    g = np.random.default_rng(22)
    rows = [synth.normal_bf16(g, (40, 512), std=s) for s in (1.0, 1e-3, 300.0)]
    rb = g.integers(0, 0x10000, (64, 512), dtype=np.uint32).astype(np.uint16)
    rows.append(np.where((rb & 0x7F80) == 0x7F80, rb & 0x807F, rb).astype(np.uint16))
    sub = (g.integers(0, 0x80, (16, 512)) | (g.integers(0, 2, (16, 512)) << 15)).astype(np.uint16)
    sub[:8, ::32] = np.arange(1, 9)[:, None] << 7
    rows.append(sub)
    x = np.concatenate(rows)
    say(f"[mxfp8 quant] rows={x.shape[0]} K=512")
    q, s = _quantize_gpu(x)
    rq, rs = oracle.quantize_mxfp8_act(x)
    assert np.array_equal(s, rs), np.argwhere(s != rs)[:5]
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:5]


def test_quantize_then_w4a8mx_gemm_chain():
    M, N, K = 48, 512, 2048
    x = synth.normal_bf16(np.random.default_rng(9), (M, K))
    w = synth.quantize_mxfp4(np.random.default_rng(10).standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    say("[w4a8mx chain]")
    q, s = _quantize_gpu(x)
    y = _gemm({"xq": q, "xs": s, "wq": w["wq"], "scales": w["scales"]}, M, N, K)
    rq, rs = oracle.quantize_mxfp8_act(x)
    ref, _ = oracle.ref_w4a8_mx(rq, rs, w["wq"], w["scales"])
    check_float(y, ref, "w4a8mx chain")
