"""CPU-only checks of the C ABI: the library loads, exports every entry point declared in
include/hq.h, and rejects invalid arguments on the host before any HIP call (these calls never
reach a launch, so they run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_gemm_prepacked_amd as hq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "hq.h")).read()
    return sorted(set(re.findall(r"\b(hq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "hq_gemm" in names and "hq_moe_grouped_gemm" in names
    lib = ctypes.CDLL(hq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(hq.EXPORTED)


def test_version():
    assert hq.hq_version() >= 100


def test_desc_rejections():
    bad = hq.make_desc(hq.HQ_W_INT4_SYM, 64, hq.HQ_SCALE_BF16, 0, hq.HQ_ACT_BF16)
    assert hq.hq_prepacked_bytes(bad, 1, 256, 512) == 0
    with pytest.raises(hq.HQError) as ei:
        hq.hq_gemm(bad, 4, 256, 512, 16, None, 16, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_UNSUPPORTED and "group_size" in str(ei.value)
    wrong_size = hq.make_desc(hq.HQ_W_INT4_SYM, 128, hq.HQ_SCALE_BF16, 0, hq.HQ_ACT_BF16)
    wrong_size.struct_size = 8
    with pytest.raises(hq.HQError) as ei:
        hq.hq_gemm(wrong_size, 4, 256, 512, 16, None, 16, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_INVALID_ARGUMENT
    unknown = hq.make_desc(9, 128, hq.HQ_SCALE_BF16, 0, hq.HQ_ACT_BF16)
    with pytest.raises(hq.HQError):
        hq.hq_gemm(unknown, 4, 256, 512, 16, None, 16, 16, stream=0)
    # an INT32 accumulator output exists only for W8A8
    i32_on_int4 = hq.make_desc(hq.HQ_W_INT4_SYM, 128, hq.HQ_SCALE_BF16, 0, hq.HQ_ACT_BF16, hq.HQ_OUT_INT32_ACC)
    with pytest.raises(hq.HQError):
        hq.hq_gemm(i32_on_int4, 4, 256, 512, 16, None, 16, 16, stream=0)


@pytest.mark.parametrize("M,N,K,a,w,y,scale,code", [
    (4, 250, 512, 16, 16, 16, None, hq.HQ_ERR_UNSUPPORTED),      # N % 16
    (4, 256, 500, 16, 16, 16, None, hq.HQ_ERR_UNSUPPORTED),      # K % 128
    (4, 256, 512, 0, 16, 16, None, hq.HQ_ERR_INVALID_ARGUMENT),  # null a
    (4, 256, 512, 8, 16, 16, None, hq.HQ_ERR_INVALID_ARGUMENT),  # misaligned a
    (4, 256, 512, 16, 16, 16, 64, hq.HQ_ERR_INVALID_ARGUMENT),   # a_scale with bf16 activations
    (-1, 256, 512, 16, 16, 16, None, hq.HQ_ERR_INVALID_ARGUMENT),
    (4, 0, 512, 16, 16, 16, None, hq.HQ_ERR_INVALID_ARGUMENT),
])
def test_gemm_argument_rejections(M, N, K, a, w, y, scale, code):
    with pytest.raises(hq.HQError) as ei:
        hq.hq_gemm(hq.DESC_W4A16_SYM, M, N, K, a or None, scale, w, y, stream=0)
    assert ei.value.status == code


def test_gemm_m0_is_noop():
    hq.hq_gemm(hq.DESC_W4A16_SYM, 0, 256, 512, 16, None, 16, 16, stream=0)


def test_w8a8_needs_scale_and_workspace_checked():
    with pytest.raises(hq.HQError) as ei:
        hq.hq_gemm(hq.DESC_W8A8, 4, 256, 512, 16, None, 16, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_INVALID_ARGUMENT
    need = hq.hq_gemm_workspace_bytes(hq.DESC_W8A8, 1, 256, 8192)
    assert need > 0  # one row over a deep K asks for a K split
    with pytest.raises(hq.HQError) as ei:
        hq.hq_gemm(hq.DESC_W8A8, 1, 256, 8192, 16, 64, 16, 16, ws=16, ws_bytes=need - 1, stream=0)
    assert ei.value.status == hq.HQ_ERR_WORKSPACE


def test_moe_rejections():
    d = hq.DESC_W4A16_SYM
    with pytest.raises(hq.HQError):
        hq.hq_moe_align(16, 4, 8, 256, 24, 16, 16, 16, 16, stream=0)        # block_m % 16
    with pytest.raises(hq.HQError):
        hq.hq_moe_align(16, 4, 8, 1000, 16, 16, 16, 16, 16, stream=0)       # E > 512
    with pytest.raises(hq.HQError):
        hq.hq_moe_align(16, 4, 8, 256, 16, 0, 16, 16, 16, stream=0)         # null output
    with pytest.raises(hq.HQError) as ei:      # MX activations need their e8m0 scale rows
        hq.hq_moe_grouped_gemm(hq.DESC_W4A4_MXFP4, 4, 8, 256, 256, 512, 16, None, 16, 16, 16, 16, 16,
                               None, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_INVALID_ARGUMENT
    with pytest.raises(hq.HQError) as ei:      # int32 accumulators are a dense-only output
        hq.hq_moe_grouped_gemm(hq.DESC_W8A8_I32, 4, 8, 256, 256, 512, 16, 64, 16, 16, 16, 16, 16,
                               None, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_UNSUPPORTED
    for dq in (hq.DESC_W8A8, hq.DESC_W4A8_MXFP4):   # per-token activations need their scales
        with pytest.raises(hq.HQError) as ei:
            hq.hq_moe_grouped_gemm(dq, 4, 8, 256, 256, 512, 16, None, 16, 16, 16, 16, 16, None, 16, stream=0)
        assert ei.value.status == hq.HQ_ERR_INVALID_ARGUMENT
    with pytest.raises(hq.HQError) as ei:
        hq.hq_moe_grouped_gemm(d, 4, 8, 256, 256, 512, 16, None, 16, 16, 16, 16, 48, None, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_UNSUPPORTED
    with pytest.raises(hq.HQError) as ei:      # 128-row blocks need N % 128 == 0
        hq.hq_moe_grouped_gemm(d, 4, 8, 256, 272, 512, 16, None, 16, 16, 16, 16, 128, None, 16, stream=0)
    assert ei.value.status == hq.HQ_ERR_UNSUPPORTED


def test_moe_capacity_bounds_padding():
    for T, topk, E, bm in [(1, 8, 256, 16), (4096, 8, 256, 64), (3, 2, 4, 16)]:
        cap = hq.hq_moe_align_capacity(T, topk, E, bm)
        assert cap % bm == 0 and cap >= T * topk
        assert cap >= T * topk + min(E, T * topk) * (bm - 1)
    assert hq.hq_moe_block_m(hq.DESC_W4A16_SYM, 1, 8, 256, 4096, 7168) in (16, 32, 64)


def test_prepack_rejections():
    d = hq.DESC_W4A16_ASYM
    n, k = 32, 256
    wq = np.zeros((n, k // 2), np.uint8)
    s = np.zeros((n, k // 128), np.uint16)
    out = np.zeros(hq.hq_prepacked_bytes(d, 1, n, k), np.uint8)
    with pytest.raises(hq.HQError):
        hq.hq_prepack_weights(d, 1, n, k, wq, s, None, out)            # zeros missing
    with pytest.raises(hq.HQError) as ei:
        hq.hq_prepack_weights(d, 1, n, k, wq, s, np.zeros_like(s, np.uint8), out[:-1])
    assert ei.value.status == hq.HQ_ERR_WORKSPACE


def test_grouped_gemm_host_validation():
    """Refused on the host before any launch: block-scaled activations, E out of range, a_scale
    given for bf16 activations or missing for per-token ones."""
    d = hq.DESC_W4A16_SYM
    assert hq.hq_grouped_gemm_workspace_bytes(d, 4096, 256, 4096, 7168) > 4096 * 4
    assert hq.hq_grouped_gemm_workspace_bytes(d, 16, 0, 256, 256) == 0
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(hq.DESC_W4A4_MXFP4, 4, 2, 256, 512, 16, 16, 16, 16, 16, 16, 1 << 20, stream=0)
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(hq.DESC_W8A8, 4, 2, 256, 512, 16, None, 16, 16, 16, 16, 1 << 20, stream=0)
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(d, 4, 600, 256, 512, 16, None, 16, 16, 16, 16, 1 << 20, stream=0)
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(d, 4, 2, 256, 512, 16, 16, 16, 16, 16, 16, 1 << 20, stream=0)


def test_w8a16_descriptors():
    """INT8 and FP8 weights with bf16 activations: per-channel fp32 scales only, K % 128, bf16
    output, no activation scale."""
    for desc in (hq.DESC_W8A16_INT8, hq.DESC_W8A16_FP8):
        assert hq.hq_prepacked_bytes(desc, 1, 256, 512) > 0
        assert hq.hq_prepacked_bytes(desc, 1, 256, 448) == 0          # K % 128
        with pytest.raises(hq.HQError) as ei:
            hq.hq_gemm(desc, 4, 256, 512, 16, 64, 16, 16, stream=0)   # a_scale with bf16 activations
        assert ei.value.status == hq.HQ_ERR_INVALID_ARGUMENT
    for wf in (hq.HQ_W_INT8_SYM, hq.HQ_W_FP8_E4M3):
        for bad in (hq.make_desc(wf, 128, hq.HQ_SCALE_FP32, 0, hq.HQ_ACT_BF16),
                    hq.make_desc(wf, 0, hq.HQ_SCALE_BF16, 0, hq.HQ_ACT_BF16),
                    hq.make_desc(wf, 0, hq.HQ_SCALE_FP32, 0, hq.HQ_ACT_BF16, hq.HQ_OUT_INT32_ACC)):
            assert hq.hq_prepacked_bytes(bad, 1, 256, 512) == 0
            with pytest.raises(hq.HQError) as ei:
                hq.hq_gemm(bad, 4, 256, 512, 16, None, 16, 16, stream=0)
            assert ei.value.status == hq.HQ_ERR_UNSUPPORTED


def test_w2a16_descriptor():
    d = hq.DESC_W2A16_ASYM
    assert hq.hq_prepacked_bytes(d, 1, 256, 512) > 0
    assert hq.hq_gemm_plan(d, 8, 256, 512)[0] == 0               # small M: the skinny kernel
    assert hq.hq_gemm_plan(d, 8192, 256, 512)[0:2] == (3, 0)     # large M: ping-pong 128 x 256
    assert hq.hq_gemm_plan(d, 8192, 384, 512)[0] == 0            # no 256-wide tile divides N
    for bad in (hq.make_desc(hq.HQ_W_UINT2_ASYM, 64, hq.HQ_SCALE_BF16, 1, hq.HQ_ACT_BF16),
                hq.make_desc(hq.HQ_W_UINT2_ASYM, 128, hq.HQ_SCALE_BF16, 0, hq.HQ_ACT_BF16),
                hq.make_desc(hq.HQ_W_UINT2_ASYM, 128, hq.HQ_SCALE_BF16, 1, hq.HQ_ACT_INT8_PER_TOKEN)):
        assert hq.hq_prepacked_bytes(bad, 1, 256, 512) == 0
    with pytest.raises(hq.HQError):
        hq.hq_prepack_weights(d, 1, 256, 512, np.zeros((256, 128), np.uint8), np.zeros((256, 4), np.uint16),
                              None, np.zeros(hq.hq_prepacked_bytes(d, 1, 256, 512), np.uint8))   # zeros missing


def test_w3a16_descriptor():
    d = hq.DESC_W3A16_ASYM
    assert hq.hq_prepacked_bytes(d, 1, 256, 512) > 0
    assert hq.hq_gemm_plan(d, 128, 256, 512)[0] == 0             # the small-M kernel to M = 128
    assert hq.hq_gemm_plan(d, 8192, 256, 512)[:2] == (3, 0)      # ping-pong 128 x 256 beyond
    assert hq.hq_gemm_plan(d, 8192, 400, 512)[0] == 0            # no ping-pong tile divides N
    with pytest.raises(hq.HQError):                               # zeros missing
        hq.hq_prepack_weights(d, 1, 256, 512, np.zeros((256, 192), np.uint8), np.zeros((256, 4), np.uint16),
                              None, np.zeros(hq.hq_prepacked_bytes(d, 1, 256, 512), np.uint8))
    bad = hq.make_desc(hq.HQ_W_UINT3_ASYM, 32, hq.HQ_SCALE_BF16, 1, hq.HQ_ACT_BF16)
    assert hq.hq_prepacked_bytes(bad, 1, 256, 512) == 0
