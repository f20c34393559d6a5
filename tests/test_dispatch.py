"""The built-in per-M dispatch (host logic, no GPU): the kernel kind and configuration a dense call
runs at the crossovers measured on MI355X and documented beside the tables in
quantized_gemm_prepacked_amd/csrc/gemm_dispatch.hip. Kinds: 0 small-M (skinny), 2 async-pipelined,
3 ping-pong."""
import pytest

import quantized_gemm_prepacked_amd as hq

# format: (descriptor, N, K, [(M, (kind, cfg))])
TABLE = {
    "w4a16": (hq.DESC_W4A16_ASYM, 14336, 4096,
              [(1, (0, 30)), (4, (0, 30)), (5, (0, 28)), (16, (0, 28)), (33, (0, 22)), (64, (0, 22)), (65, (2, 15)), (128, (2, 15)), (129, (3, 3)),
               (256, (3, 3)), (257, (3, 0)), (8192, (3, 0))]),
    "w4a16mx": (hq.DESC_W4A16_MXFP4, 14336, 4096,
                [(1, (0, 32)), (4, (0, 32)), (5, (0, 28)), (64, (0, 3)), (65, (0, 4)), (128, (0, 4)), (129, (3, 3)), (256, (3, 3)), (257, (3, 0)), (8192, (3, 0))]),
    "w2a16": (hq.DESC_W2A16_ASYM, 14336, 4096,
              [(1, (0, 31)), (4, (0, 31)), (5, (0, 28)), (128, (0, 22)), (129, (3, 13)), (256, (3, 13)), (257, (3, 0)), (512, (3, 0)), (8192, (3, 0))]),
    "w3a16": (hq.DESC_W3A16_ASYM, 14336, 4096,
              [(1, (0, 31)), (5, (0, 28)), (32, (0, 29)), (128, (0, 22)), (129, (3, 3)), (256, (3, 3)), (257, (3, 0)), (8192, (3, 0))]),
    "w8a16": (hq.DESC_W8A16_INT8, 14336, 4096,
              [(1, (0, 33)), (4, (0, 33)), (5, (0, 27)), (32, (0, 29)), (128, (0, 4)), (129, (3, 3)), (256, (3, 3)),
               (257, (2, 12)), (640, (2, 12)), (641, (3, 3)), (896, (3, 3)), (897, (2, 12)), (8192, (2, 12))]),
    "f8a16": (hq.DESC_W8A16_FP8, 14336, 4096,
              [(1, (0, 30)), (5, (0, 27)), (32, (0, 22)), (128, (0, 4)), (129, (3, 3)), (256, (3, 3)),
               (257, (2, 12)), (768, (3, 3)), (1024, (2, 12)), (8192, (2, 12))]),
    "w8a8": (hq.DESC_W8A8, 8192, 8192,
             [(1, (0, 2)), (8, (0, 2)), (9, (0, 1)), (16, (0, 1)), (32, (0, 23)), (33, (0, 29)),
              (64, (0, 29)), (65, (2, 3)), (128, (2, 3)), (129, (2, 15)), (256, (2, 15)), (257, (3, 11)), (512, (3, 11)),
              (513, (3, 1)), (1024, (3, 1)), (1025, (2, 8))]),
    "fp8block": (hq.DESC_W8A8_FP8_BLOCK, 8192, 8192,
                 [(1, (0, 21)), (4, (0, 21)), (5, (0, 20)), (16, (0, 20)), (32, (0, 23)), (64, (0, 29)),
                  (65, (0, 4)), (128, (0, 4)), (129, (2, 2)), (256, (2, 2)), (257, (3, 10)), (640, (3, 10)), (641, (2, 14)),
                  (1280, (2, 14)), (1281, (2, 11)), (2048, (2, 11)), (2049, (2, 14)), (3072, (2, 14)),
                  (3073, (2, 11)), (8192, (2, 11))]),
    "w4a8": (hq.DESC_W4A8_MXFP4, 4096, 7168,
             [(1, (0, 21)), (32, (0, 18)), (64, (0, 23)), (65, (0, 29)), (128, (0, 29)), (129, (0, 22)),
              (256, (0, 22)), (257, (2, 3)), (512, (2, 3)), (513, (2, 2)), (1024, (2, 2)), (1025, (2, 0)),
              (2048, (2, 0)), (2049, (2, 12)), (3072, (2, 12)), (3073, (2, 11))]),
    "w4a4": (hq.DESC_W4A4_MXFP4, 4096, 7168, [(1, (0, 21)), (32, (0, 18)), (64, (0, 23)), (128, (0, 29)), (129, (0, 4)), (160, (0, 4)), (161, (2, 3)), (640, (2, 3)), (641, (2, 2)), (1024, (2, 2)), (1025, (2, 13)), (2048, (2, 13)), (2049, (2, 6)), (8192, (2, 6))]),
    "w4a8mx": (hq.DESC_W4A8_MXFP8, 4096, 7168, [(1, (0, 21)), (32, (0, 18)), (64, (0, 28)), (128, (0, 29)), (129, (0, 4)), (256, (0, 4)), (257, (2, 3)), (512, (2, 3)), (513, (2, 2)), (1024, (2, 2)), (1025, (3, 8)), (2048, (3, 8)), (2049, (2, 11)), (8192, (2, 11))]),
}


@pytest.fixture(autouse=True)
def _built_in_table(monkeypatch):
    monkeypatch.delenv("HQ_TUNE", raising=False)
    monkeypatch.delenv("HQ_TUNING_FILE", raising=False)
    hq.hq_load_tuning_table(None)
    yield
    hq.hq_load_tuning_table(None)


@pytest.mark.parametrize("fmt", sorted(TABLE))
def test_built_in_dispatch(fmt):
    desc, N, K, points = TABLE[fmt]
    for M, (kind, cfg) in points:
        k, c, split = hq.hq_gemm_plan(desc, M, N, K)
        assert (k, c) == (kind, cfg), (fmt, M, (k, c))
        assert split == 1


def test_fallbacks_when_no_tile_divides_n():
    # 2-bit weights on the ping-pong kernel need 256-wide tiles; 8-bit bf16-activation formats
    # take 128 x 128; with N = 400 neither divides and the skinny kernel runs
    for desc in (hq.DESC_W2A16_ASYM, hq.DESC_W8A16_INT8, hq.DESC_W4A16_MXFP4):
        assert hq.hq_gemm_plan(desc, 4096, 400, 4096)[0] == 0
    assert hq.hq_gemm_plan(hq.DESC_W2A16_ASYM, 4096, 384, 4096)[0] == 0
    assert hq.hq_gemm_plan(hq.DESC_W8A16_INT8, 4096, 384, 4096)[0] == 3


def test_activation_offsets_past_32_bits_leave_the_lds_kernels():
    """The direct-to-LDS kernels address activation rows with 32-bit offsets: a call whose
    activations reach 4 GiB runs on the LDS-tiled kernel (WNA16) or the small-M kernel (formats
    without a tiled form), both of which address rows with 64 bits."""
    K = 8192
    assert hq.hq_gemm_plan(hq.DESC_W4A16_ASYM, 262143, 256, K)[0] == 3      # 4 GiB - 16 KiB of bf16
    assert hq.hq_gemm_plan(hq.DESC_W4A16_ASYM, 262144, 256, K)[0] == 1
    assert hq.hq_gemm_plan(hq.DESC_W4A4_MXFP4, 2 ** 20 - 1, 256, K)[0] in (2, 3)  # 4-bit codes
    assert hq.hq_gemm_plan(hq.DESC_W4A4_MXFP4, 2 ** 20, 256, K)[0] == 0


def test_moe_block_sizes_follow_the_measured_crossovers():
    """hq_moe_block_m at the DeepSeek-V3 gate_up shape (top-8 of 256 experts): 16-row blocks below
    2 routed rows per expert, 32 from 2, 64 from 8, 128 for INT4 / MXFP4 experts with bf16
    activations from 24 (block-scaled FP8 from 8); 8-bit per-token activations stay at 64."""
    N, K, E, topk = 4096, 7168, 256, 8
    want = [(hq.DESC_W4A16_SYM, {32: 16, 64: 32, 256: 64, 512: 64, 767: 64, 768: 128, 4096: 128}),
            (hq.DESC_W4A16_MXFP4, {512: 64, 768: 128}),
            (hq.DESC_W8A8_FP8_BLOCK, {64: 32, 256: 128, 4096: 128}),
            (hq.DESC_W4A8_MXFP4, {256: 64, 4096: 64})]
    for desc, pts in want:
        for T, bm in pts.items():
            assert hq.hq_moe_block_m(desc, T, topk, E, N, K) == bm, (T, bm)
