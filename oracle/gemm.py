"""Dense quantized GEMM, written as its plain definition (test infrastructure).

Y = X . W^T with W = dequant(Wq, scales, zero-points): W is logically [N, K] (the usual linear
layer layout), X is [M, K], Y is [M, N]. The Humming announcement describes the computation in
its sections "A unified quantization representation" (weight format, scale granularity, scale
dtype and zero-points are separate parameters; activations have their own format) and "Shared
CUDA components across formats and architectures" (dequantization and scaling are part of the
GEMM; scaling can be fused into the output stage). The three weight/activation pairs covered
are those of section "Why quantized inference needs a general-purpose kernel library"
(WNA16, W8A8, W4A8) with MXFP4 weights as in section "W8A8 / W4A8 / W4A4".

``rows``/``cols`` restrict the result to a subset of outputs (for sampled checks at full size);
the arithmetic per output is unchanged.
"""
from __future__ import annotations

import numpy as np

from .codecs import (
    unpack_nibbles, unpack_crumbs, unpack_triplets, decode_int4_sym, decode_uint4, decode_e2m1, decode_e8m0, decode_e4m3,
    decode_bf16, round_to_bf16, decode_int8,
)


def _sel(a: np.ndarray, idx):
    return a if idx is None else a[np.asarray(idx)]


def dequant_wna16(wq: np.ndarray, scales_bf16: np.ndarray, zeros: np.ndarray | None, g: int,
                  cols=None) -> np.ndarray:
    """Group-wise INT4 weights -> float64 [N, K].

    symmetric:  w[n, k] = q[n, k] * s[n, k // g],           q in [-8, 7]
    asymmetric: w[n, k] = (q[n, k] - z[n, k // g]) * s[n, k // g],  q, z in [0, 15]
    """
    codes = unpack_nibbles(_sel(wq, cols))
    s = decode_bf16(_sel(scales_bf16, cols))
    N, K = codes.shape
    grp = np.arange(K) // g
    if zeros is None:
        q = decode_int4_sym(codes)
        return q.astype(np.float64) * s[:, grp]
    q = decode_uint4(codes)
    z = decode_uint4(_sel(zeros, cols))
    return (q - z[:, grp]).astype(np.float64) * s[:, grp]


def dequant_wna2(wq: np.ndarray, scales_bf16: np.ndarray, zeros: np.ndarray, g: int, cols=None) -> np.ndarray:
    """Group-wise asymmetric UINT2 weights -> float64 [N, K] (the page's WnA16 at a 2-bit weight
    width, section "Results: kernel microbenchmarks"):
        w[n, k] = (q[n, k] - z[n, k // g]) * s[n, k // g],    q, z in [0, 3]
    wq packs four codes per byte (lowest k in the lowest bits), scales are bf16 bits."""
    q = unpack_crumbs(_sel(wq, cols)).astype(np.int64)
    s = decode_bf16(_sel(scales_bf16, cols))
    z = np.asarray(_sel(zeros, cols)).astype(np.int64) & 0x3
    grp = np.arange(q.shape[1]) // g
    return (q - z[:, grp]).astype(np.float64) * s[:, grp]


def dequant_wna3(wq: np.ndarray, scales_bf16: np.ndarray, zeros: np.ndarray, g: int, cols=None) -> np.ndarray:
    """Group-wise asymmetric UINT3 weights -> float64 [N, K] (the page's WnA16 at a 3-bit width):
        w[n, k] = (q[n, k] - z[n, k // g]) * s[n, k // g],    q, z in [0, 7]
    wq packs each row as a little-endian bit string of 3-bit codes (3K/8 bytes)."""
    q = unpack_triplets(_sel(wq, cols)).astype(np.int64)
    s = decode_bf16(_sel(scales_bf16, cols))
    z = np.asarray(_sel(zeros, cols)).astype(np.int64) & 0x7
    grp = np.arange(q.shape[1]) // g
    return (q - z[:, grp]).astype(np.float64) * s[:, grp]


def dequant_mxfp4(wq: np.ndarray, scales_e8m0: np.ndarray, cols=None) -> np.ndarray:
    """MXFP4 weights -> float64 [N, K]:  w[n, k] = e2m1(c[n, k]) * 2^(e[n, k // 32] - 127)."""
    codes = unpack_nibbles(_sel(wq, cols))
    K = codes.shape[1]
    x = decode_e8m0(_sel(scales_e8m0, cols))
    return decode_e2m1(codes) * x[:, np.arange(K) // 32]


def ref_wna16(x_bf16: np.ndarray, wq: np.ndarray, scales_bf16: np.ndarray,
              zeros: np.ndarray | None, g: int, rows=None, cols=None):
    """WNA16: bf16 activations times group-INT4 weights. Returns (y float64, y bf16 bits)."""
    x = decode_bf16(_sel(x_bf16, rows))
    w = dequant_wna16(wq, scales_bf16, zeros, g, cols)
    y = x @ w.T
    return y, round_to_bf16(y)


def ref_w8a8(xq: np.ndarray, s_tok: np.ndarray, wq: np.ndarray, s_ch: np.ndarray,
             rows=None, cols=None):
    """W8A8 INT8: acc[m, n] = sum_k xq[m, k] * wq[n, k] (exact integer), then
    y = acc * s_tok[m] * s_ch[n] in float64, rounded once to bf16.
    Returns (acc int64, y float64, y bf16 bits).

    The integer sum is formed with a float64 matmul: every product is below 2^14 in magnitude
    and every partial sum below 2^27 for K <= 8192, so each is an integer that float64 holds
    exactly whatever the summation order; the result is then converted back to int64.
    """
    a = decode_int8(_sel(xq, rows))
    b = decode_int8(_sel(wq, cols))
    K = a.shape[1]
    assert K * 128 * 128 < 2 ** 53
    acc = (a.astype(np.float64) @ b.astype(np.float64).T).astype(np.int64)
    st = np.asarray(_sel(s_tok, rows), dtype=np.float32).astype(np.float64)
    sc = np.asarray(_sel(s_ch, cols), dtype=np.float32).astype(np.float64)
    y = acc.astype(np.float64) * st[:, None] * sc[None, :]
    return acc, y, round_to_bf16(y)


def ref_w4a8(xq: np.ndarray, s_tok: np.ndarray, wq: np.ndarray, scales_e8m0: np.ndarray,
             rows=None, cols=None):
    """W4A8-MXFP4: y[m, n] = s_tok[m] * sum_k e4m3(xq[m, k]) * w[n, k], w = dequant_mxfp4.
    Returns (y float64, y bf16 bits)."""
    x = decode_e4m3(_sel(xq, rows))
    w = dequant_mxfp4(wq, scales_e8m0, cols)
    st = np.asarray(_sel(s_tok, rows), dtype=np.float32).astype(np.float64)
    y = (x @ w.T) * st[:, None]
    return y, round_to_bf16(y)


def ref_w4a4(xq: np.ndarray, xs_e8m0: np.ndarray, wq: np.ndarray, scales_e8m0: np.ndarray,
             rows=None, cols=None):
    """W4A4-MXFP4: both operands MXFP4 (e2m1 codes with an e8m0 scale per 32-element block
    along K), y[m, n] = sum_k x[m, k] * w[n, k] with x and w each dequantized per the MX
    definition; the products and sums are exact in float64. Returns (y float64, y bf16 bits)."""
    x = dequant_mxfp4(xq, xs_e8m0, rows)
    w = dequant_mxfp4(wq, scales_e8m0, cols)
    y = x @ w.T
    return y, round_to_bf16(y)


def ref_w4a8_mx(xq: np.ndarray, xs_e8m0: np.ndarray, wq: np.ndarray, scales_e8m0: np.ndarray,
                rows=None, cols=None):
    """W4A8 with MXFP8 activations: x[m, k] = e4m3(xq[m, k]) * 2^(xs[m, k // 32] - 127) (an e8m0
    scale per 32-element block instead of a per-token fp32 scale), w = dequant_mxfp4; the sum is
    exact in float64. Returns (y float64, y bf16 bits)."""
    xc = decode_e4m3(_sel(xq, rows))
    K = xc.shape[1]
    x = xc * decode_e8m0(_sel(xs_e8m0, rows))[:, np.arange(K) // 32]
    w = dequant_mxfp4(wq, scales_e8m0, cols)
    y = x @ w.T
    return y, round_to_bf16(y)


def ref_w4a16_mx(x_bf16: np.ndarray, wq: np.ndarray, scales_e8m0: np.ndarray, rows=None, cols=None):
    """MXFP4 weights with bf16 activations ("W4A16-MXFP4"): y = x . dequant_mxfp4(w)^T, exact
    float64 products and sums, rounded once to bf16. Returns (y float64, y bf16 bits)."""
    x = decode_bf16(_sel(x_bf16, rows))
    w = dequant_mxfp4(wq, scales_e8m0, cols)
    y = x @ w.T
    return y, round_to_bf16(y)


def ref_w8a8_fp8_block(xq: np.ndarray, xs: np.ndarray, wq: np.ndarray, ws: np.ndarray, rows=None, cols=None):
    """FP8 W8A8 with block scales (the page's "FP8 W8A8 with blockwise scaling"): e4m3 activations
    with an fp32 scale per (token, 128-k block), e4m3 weights with an fp32 scale per (128-n block,
    128-k block):
        y[m, n] = sum_g xs[m, g] * ws[n // 128, g] * sum_{k in g} e4m3(xq[m, k]) * e4m3(wq[n, k])
    exact in float64, rounded once to bf16. Returns (y float64, y bf16 bits)."""
    x = decode_e4m3(_sel(xq, rows))
    w = decode_e4m3(_sel(wq, cols))
    sa = np.asarray(_sel(xs, rows), dtype=np.float32).astype(np.float64)
    n_idx = np.arange(wq.shape[0]) if cols is None else np.asarray(cols)
    sw = np.asarray(ws, dtype=np.float32).astype(np.float64)[n_idx // 128]      # [N', G]
    G = x.shape[1] // 128
    y = np.zeros((x.shape[0], w.shape[0]))
    for g in range(G):
        part = x[:, 128 * g:128 * (g + 1)] @ w[:, 128 * g:128 * (g + 1)].T
        y += part * sa[:, g:g + 1] * sw[None, :, g]
    return y, round_to_bf16(y)


def ref_w8a16(x_bf16: np.ndarray, wq: np.ndarray, s_ch: np.ndarray, fp8: bool = False,
              rows=None, cols=None):
    """8-bit weights with bf16 activations (the page's WnA16 at an 8-bit weight width, section
    "Results: kernel microbenchmarks", WnA16 paragraph on integer and floating-point weights up
    to FP8): symmetric INT8 codes (two's complement, [-127, 127]) or FP8 e4m3 codes, each with an
    fp32 scale per output channel (scale granularity "per channel", section "A unified
    quantization representation"):
        w[n, k] = decode(wq[n, k]) * s_ch[n],        y = x . w^T
    dequantized and multiplied in float64, rounded once to bf16. Returns (y float64, y bf16 bits)."""
    x = decode_bf16(_sel(x_bf16, rows))
    c = _sel(wq, cols)
    q = decode_e4m3(c) if fp8 else decode_int8(c).astype(np.float64)
    s = np.asarray(_sel(s_ch, cols), dtype=np.float32).astype(np.float64)
    w = q * s[:, None]
    y = x @ w.T
    return y, round_to_bf16(y)


def ref_wna2(x_bf16: np.ndarray, wq: np.ndarray, scales_bf16: np.ndarray, zeros: np.ndarray, g: int,
             rows=None, cols=None):
    """2-bit WnA16: bf16 activations times group-wise UINT2 weights with zero-points,
    y = x . dequant_wna2(w)^T in float64, rounded once to bf16. Returns (y float64, y bf16 bits)."""
    x = decode_bf16(_sel(x_bf16, rows))
    w = dequant_wna2(wq, scales_bf16, zeros, g, cols)
    y = x @ w.T
    return y, round_to_bf16(y)


def ref_wna3(x_bf16: np.ndarray, wq: np.ndarray, scales_bf16: np.ndarray, zeros: np.ndarray, g: int,
             rows=None, cols=None):
    """3-bit WnA16: bf16 activations times group-wise UINT3 weights with zero-points,
    y = x . dequant_wna3(w)^T in float64, rounded once to bf16. Returns (y float64, y bf16 bits)."""
    x = decode_bf16(_sel(x_bf16, rows))
    w = dequant_wna3(wq, scales_bf16, zeros, g, cols)
    y = x @ w.T
    return y, round_to_bf16(y)
