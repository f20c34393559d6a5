"""CPU oracle for the fused-dequantization quantized GEMM -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct reference for what the HIP library computes:

    Y = X . dequant(Wq, scales, zero-points)^T        (dense)
    Y[t*topk + j] = X[t] . dequant(W_{e(t,j)})^T      (MoE, e = routed expert)

It follows the Humming announcement (English page), which states that the unified quantization
representation "preserves each scheme's quantization semantics" (section "A unified
quantization representation"): the fused kernel must equal dequantize-then-multiply. So each
function here decodes the standard-format codes by their format definitions, dequantizes in
float64, multiplies in float64 (integer-exact for W8A8), applies the output scales and rounds
once to bf16 with round-to-nearest-even.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. It shares no code, table or helper with the HIP library and never imports
it; both consume the seeded inputs of ``synth``.

``actquant`` defines the per-token dynamic quantization of bf16 activations that precedes the
W8A8 and W4A8 GEMMs.

Pins (in ``tests/test_oracle_*.py``, CPU only): format decode tables against hand values and
torch's own dtype casts, the zero-exponent/symmetric-integer equivalence stated in the section
"Results: quantization support", hand-computed cases under ``tests/golden/``, a brute-force
triple loop, and special cases that reduce to a plain library matmul.
"""
from .codecs import (  # noqa: F401
    unpack_nibbles, unpack_crumbs, unpack_triplets, decode_int4_sym, decode_uint4, decode_int8, decode_e2m1, decode_e8m0,
    decode_e4m3, decode_bf16, round_to_bf16, decode_sign_magnitude,
)
from .gemm import (  # noqa: F401
    dequant_wna16, dequant_mxfp4, ref_wna16, ref_w8a8, ref_w4a8, ref_w4a4, ref_w4a8_mx, ref_w4a16_mx, ref_w8a8_fp8_block,
    ref_w8a16, dequant_wna2, ref_wna2, dequant_wna3, ref_wna3,
)
from .moe import (  # noqa: F401
    ref_moe_align, ref_moe_gemm, ref_moe_gemm_q, ref_moe_gemm_fp8_block, ref_moe_gemm_mx, ref_grouped_gemm, ref_silu_mul, ref_moe_combine, ref_moe_layer, ref_moe_layer_w4a8,
)
from .actquant import (  # noqa: F401
    encode_e4m3, quantize_per_token, encode_e2m1, quantize_mxfp4_act, quantize_mxfp8_act,
    quantize_fp8_block_act,
)
