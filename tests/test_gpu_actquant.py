"""GPU parity of the per-token activation quantization (hq_quantize_activations) against the
oracle: codes and scales bit-exact (integer decisions taken in binary32 on both sides)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, say, to_dev

pytestmark = pytest.mark.gpu

ACTS = {"int8": hq.HQ_ACT_INT8_PER_TOKEN, "e4m3": hq.HQ_ACT_FP8E4M3_PER_TOKEN}


def _run(act, x_bits):
    M, K = x_bits.shape
    xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    hq.hq_quantize_activations(ACTS[act], M, K, to_dev(x_bits), xq, s)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), s.cpu().numpy()


def _check(act, x_bits):
    q, s = _run(act, x_bits)
    rq, rs = oracle.quantize_per_token(x_bits, act)
    assert np.array_equal(s, rs), "scales differ"
    bad = np.flatnonzero(q.view(np.uint8).ravel() != rq.view(np.uint8).ravel())
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}"


@pytest.mark.parametrize("act", ["int8", "e4m3"])
@pytest.mark.parametrize("M,K,scale", [(1, 8, 1.0), (5, 7168, 1.0), (64, 8192, 1.0), (33, 2056, 1e-3),
                                       (300, 4096, 50.0), (8, 65536, 1.0)])
def test_actquant_matches_oracle(act, M, K, scale):
    say(f"[actquant {act}] M={M} K={K} scale={scale}")
    x = synth.normal_bf16(synth.rng(9, M, K), (M, K), std=scale)
    _check(act, x)


@pytest.mark.parametrize("act", ["int8", "e4m3"])
def test_actquant_edge_rows(act):
    """All-zero rows, a row of one repeated value, tiny values near the e4m3 subnormal range,
    ties of the quotient (power-of-two scales), signed zeros."""
    K = 64
    rows = [np.zeros(K, np.float32), np.full(K, -3.0, np.float32),
            np.linspace(-2.0 ** -8, 2.0 ** -8, K).astype(np.float32),
            np.array([15.875, -15.875, 0.0625, 0.1875, -0.3125, 1.0, -0.0, 0.0] * 8, np.float32),
            np.array([112.0, 0.25, 0.28125, 0.265625, 0.296875, -2.0 ** -11, 3 * 2.0 ** -12, -2.0 ** -16] * 8, np.float32)]
    _check(act, synth.bf16_bits(np.stack(rows)))


def test_actquant_feeds_the_gemm():
    """bf16 activations -> hq_quantize_activations -> hq_gemm (W8A8) equals the oracle GEMM on the
    oracle's own quantization of the same activations."""
    M, N, K = 40, 256, 1024
    d = synth.make_w8a8(310, 1, N, K)
    x = synth.normal_bf16(synth.rng(310, M), (M, K))
    q, s = _run("int8", x)
    packed = np.zeros(hq.hq_prepacked_bytes(hq.DESC_W8A8_I32, 1, N, K), np.uint8)
    hq.hq_prepack_weights(hq.DESC_W8A8_I32, 1, N, K, d["wq"], d["s_ch"], None, packed)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    hq.hq_gemm(hq.DESC_W8A8_I32, M, N, K, to_dev(q), to_dev(s), to_dev(packed), acc)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_per_token(x, "int8")
    ref_acc, _, _ = oracle.ref_w8a8(rq, rs, d["wq"], d["s_ch"])
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref_acc)
