"""Seeded synthetic inputs for the quantized GEMM: random draws and standard-format quantizers.

This module is shared by the CPU oracle's tests, the GPU parity tests and the benchmark. It
produces the *inputs* of the fused-dequantization GEMM: bf16 activations, quantized activation
codes with their per-token scales, and weights in the standard quantization format (codes,
scales, zero-points kept as separate tensors, as the Humming announcement's section "A unified
quantization representation" describes). It holds none of the GEMM's own arithmetic: there is
no decoding of codes back to values, no dequantization, no contraction and no output epilogue
here. Those live, independently, in ``oracle/`` (CPU reference) and in the HIP library.

Value recipes (the pages give none; these follow the workload descriptions the benchmark uses):

* activations: fp32 draws from N(0, 1), rounded to bf16 (round-to-nearest-even);
* weights: fp32 draws from N(0, 0.02);
* symmetric INT4, group g along K:  s = bf16(absmax/7),  q = clamp(rne(w/s), -8, 7);
* asymmetric UINT4, group g:  s = bf16((max-min)/15),  z = clamp(rne(-min/s), 0, 15),
  q = clamp(rne(w/s) + z, 0, 15);
* INT8 per row (weights per output channel, activations per token):  s = fp32(absmax/127),
  q = clamp(rne(x/s), -127, 127);
* MXFP4 (OCP Microscaling v1.0 rule), blocks of 32 along K:  shared exponent
  e = floor(log2(amax)) - 2 (2 is e2m1's largest exponent), stored as e8m0 byte e + 127; elements
  are e2m1(w / 2^e), nearest with ties to the even code, saturating at +-6;
* FP8 e4m3 per token:  s = fp32(absmax/448),  codes = e4m3(clamp(x/s, +-448)), nearest-even.

Seeds: ``numpy.random.default_rng([config_id, 0])`` draws weights and
``default_rng([config_id, M])`` draws activations and routing, so every (config, M) point is
reproducible and the oracle and the GPU consume byte-identical tensors.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "rng", "bf16_bits", "bf16_bits_to_f32", "normal_bf16",
    "quantize_int4_sym", "quantize_uint4_asym", "quantize_int8_rows",
    "quantize_mxfp4", "quantize_fp8_rows", "moe_routing",
    "make_wna16", "make_w8a8", "make_w4a8", "make_w8a8_activations", "make_w4a8_activations",
    "make_moe_weights_expert", "make_moe_inputs", "random_int4_sym_expert",
    "E2M1_MAGNITUDES",
]


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


# --------------------------------------------------------------------------------------------
# bf16 helpers (bit-level; bf16 is the upper half of an IEEE binary32)
# --------------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def _rne(x: np.ndarray) -> np.ndarray:
    return np.rint(x)  # numpy rounds halves to even


# --------------------------------------------------------------------------------------------
# Weight quantizers -> standard format
# --------------------------------------------------------------------------------------------
def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[N, K] codes in 0..15 -> [N, K/2] bytes, low nibble holds the even k."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def quantize_int4_sym(w: np.ndarray, g: int):
    """Symmetric INT4, group g along K. Returns wq uint8 [N, K/2] (two's complement nibbles),
    scales bf16 bits uint16 [N, K/g]."""
    N, K = w.shape
    wg = w.reshape(N, K // g, g).astype(np.float32)
    amax = np.abs(wg).max(axis=2)
    s_bits = bf16_bits(amax / np.float32(7.0))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    safe = np.where(s == 0, 1.0, s)
    q = np.clip(_rne(wg / safe[:, :, None]), -8, 7)
    q = np.where(s[:, :, None] == 0, 0, q).astype(np.int8).reshape(N, K)
    return {"wq": _pack_nibbles(q.astype(np.uint8) & 0xF), "scales": s_bits}


def quantize_uint4_asym(w: np.ndarray, g: int):
    """Asymmetric UINT4 with a uint4 zero-point per (n, group). Returns wq uint8 [N, K/2],
    scales bf16 bits [N, K/g], zeros uint8 [N, K/g] (values 0..15)."""
    N, K = w.shape
    wg = w.reshape(N, K // g, g).astype(np.float32)
    lo = wg.min(axis=2)
    hi = wg.max(axis=2)
    s_bits = bf16_bits((hi - lo) / np.float32(15.0))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    degenerate = s == 0
    s_bits = np.where(degenerate, np.uint16(0x3F80), s_bits).astype(np.uint16)  # s = 1.0
    s = np.where(degenerate, 1.0, s)
    z = np.clip(_rne(-lo.astype(np.float64) / s), 0, 15)
    z = np.where(degenerate, 0, z)
    q = np.clip(_rne(wg / s[:, :, None]) + z[:, :, None], 0, 15).astype(np.uint8).reshape(N, K)
    return {"wq": _pack_nibbles(q), "scales": s_bits, "zeros": z.astype(np.uint8)}


def _pack_crumbs(codes: np.ndarray) -> np.ndarray:
    """[N, K] codes in 0..3 -> [N, K/4] bytes, code k in bits 2 (k % 4) .. 2 (k % 4) + 1."""
    c = codes.astype(np.uint8)
    return (c[:, 0::4] | (c[:, 1::4] << 2) | (c[:, 2::4] << 4) | (c[:, 3::4] << 6)).astype(np.uint8)


def quantize_uint2_asym(w: np.ndarray, g: int):
    """Asymmetric UINT2 with a uint2 zero-point per (n, group): s = bf16((max - min) / 3),
    z = clamp(rne(-min / s), 0, 3), q = clamp(rne(w / s) + z, 0, 3) (a constant group: s = 1,
    z = 0). Returns wq uint8 [N, K/4], scales bf16 bits [N, K/g], zeros uint8 [N, K/g]."""
    N, K = w.shape
    wg = w.reshape(N, K // g, g).astype(np.float32)
    lo = wg.min(axis=2)
    hi = wg.max(axis=2)
    s_bits = bf16_bits((hi - lo) / np.float32(3.0))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    degenerate = s == 0
    s_bits = np.where(degenerate, np.uint16(0x3F80), s_bits).astype(np.uint16)
    s = np.where(degenerate, 1.0, s)
    z = np.clip(_rne(-lo.astype(np.float64) / s), 0, 3)
    z = np.where(degenerate, 0, z)
    q = np.clip(_rne(wg / s[:, :, None]) + z[:, :, None], 0, 3).astype(np.uint8).reshape(N, K)
    return {"wq": _pack_crumbs(q), "scales": s_bits, "zeros": z.astype(np.uint8)}


def _pack_triplets(codes: np.ndarray) -> np.ndarray:
    """[N, K] codes in 0..7 -> [N, 3K/8] bytes: the row as a little-endian bit string, code k in
    bits 3k .. 3k + 2."""
    c = codes.astype(np.uint8)
    bits = np.stack([c & 1, (c >> 1) & 1, (c >> 2) & 1], axis=-1).reshape(c.shape[0], -1)
    return np.packbits(bits, axis=-1, bitorder="little")


def quantize_uint3_asym(w: np.ndarray, g: int):
    """Asymmetric UINT3 with a uint3 zero-point per (n, group): s = bf16((max - min) / 7),
    z = clamp(rne(-min / s), 0, 7), q = clamp(rne(w / s) + z, 0, 7) (a constant group: s = 1,
    z = 0). Returns wq uint8 [N, 3K/8], scales bf16 bits [N, K/g], zeros uint8 [N, K/g]."""
    N, K = w.shape
    wg = w.reshape(N, K // g, g).astype(np.float32)
    lo = wg.min(axis=2)
    hi = wg.max(axis=2)
    s_bits = bf16_bits((hi - lo) / np.float32(7.0))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    degenerate = s == 0
    s_bits = np.where(degenerate, np.uint16(0x3F80), s_bits).astype(np.uint16)
    s = np.where(degenerate, 1.0, s)
    z = np.clip(_rne(-lo.astype(np.float64) / s), 0, 7)
    z = np.where(degenerate, 0, z)
    q = np.clip(_rne(wg / s[:, :, None]) + z[:, :, None], 0, 7).astype(np.uint8).reshape(N, K)
    return {"wq": _pack_triplets(q), "scales": s_bits, "zeros": z.astype(np.uint8)}


def make_wna3(config_id: int, M: int, N: int, K: int, g: int = 128):
    """Dense 3-bit WnA16: bf16 N(0,1) activations, weights N(0, 0.02) quantized to UINT3 with a
    zero-point per (channel, group of g)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return {"x": normal_bf16(rng(config_id, M), (M, K)), **quantize_uint3_asym(w, g)}


def make_wna2(config_id: int, M: int, N: int, K: int, g: int = 128):
    """Dense 2-bit WnA16: bf16 N(0,1) activations, weights N(0, 0.02) quantized to UINT2 with a
    zero-point per (channel, group of g)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return {"x": normal_bf16(rng(config_id, M), (M, K)), **quantize_uint2_asym(w, g)}


def quantize_int8_rows(x: np.ndarray):
    """Per-row symmetric INT8 in [-127, 127] with fp32 scale absmax/127 (all-zero row: s = 1)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = np.clip(_rne(x.astype(np.float64) / s[:, None].astype(np.float64)), -127, 127)
    return q.astype(np.int8), s


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (4 bits, bit 3 = sign), ties to the even code, saturating at 6."""
    a = np.minimum(np.abs(v), 6.0)
    mids = (E2M1_MAGNITUDES[1:] + E2M1_MAGNITUDES[:-1]) / 2.0
    lo = np.searchsorted(mids, a, side="left")          # lower code when a sits on a midpoint
    on_mid = (lo < len(mids)) & (a == mids[np.minimum(lo, len(mids) - 1)])
    code = np.where(on_mid & (lo % 2 == 1), lo + 1, lo).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8)
    return code | (sign << 3)


def quantize_mxfp4(w: np.ndarray):
    """MXFP4: e2m1 elements in 32-element blocks along K with an e8m0 shared exponent.
    Returns wq uint8 [N, K/2] (low nibble = even k), scales uint8 [N, K/32] (e8m0 bytes)."""
    N, K = w.shape
    out_q = np.empty((N, K // 2), dtype=np.uint8)
    out_s = np.empty((N, K // 32), dtype=np.uint8)
    step = max(1, (1 << 22) // K)
    for r0 in range(0, N, step):
        wb = w[r0:r0 + step].astype(np.float64).reshape(-1, K // 32, 32)
        amax = np.abs(wb).max(axis=2)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0
        e = np.clip(e, -127, 127)
        e = np.where(amax > 0, e, -127)
        codes = _encode_e2m1(wb / np.exp2(e)[:, :, None]).reshape(wb.shape[0], K)
        out_q[r0:r0 + step] = _pack_nibbles(codes)
        out_s[r0:r0 + step] = (e + 127).astype(np.uint8)
    return {"wq": out_q, "scales": out_s}


def quantize_fp8_rows(x: np.ndarray):
    """Per-row FP8 e4m3 (OCP 'fn') codes with fp32 scale absmax/448 (all-zero row: s = 1)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    v = np.clip(x / s[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), s


# --------------------------------------------------------------------------------------------
# MoE routing
# --------------------------------------------------------------------------------------------
def moe_routing(g: np.random.Generator, T: int, E: int = 256, topk: int = 8,
                zipf_s: float = 1.1, bias_rng: np.random.Generator | None = None):
    """Router logits N(0,1) plus a per-expert Zipf(s) prior in logit space,
    bias[e] = -s * ln(rank[e]) with rank a seeded permutation of 1..E. Returns
    topk_ids int32 [T, topk] (largest logits, ties to the lower expert index) and
    topk_weights fp32 [T, topk] (softmax over all E logits, gathered and renormalised)."""
    bg = bias_rng if bias_rng is not None else g
    rank = bg.permutation(E) + 1
    bias = -zipf_s * np.log(rank.astype(np.float64))
    logits = g.standard_normal((T, E)) + bias[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, order, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


# --------------------------------------------------------------------------------------------
# Workload recipes (config id, then point)
# --------------------------------------------------------------------------------------------
def make_wna16(config_id: int, M: int, N: int, K: int, asym: bool, g: int = 128):
    """Dense WNA16: bf16 activations [M, K] and INT4 (sym) / UINT4 (asym) group-g weights."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    qw = quantize_uint4_asym(w, g) if asym else quantize_int4_sym(w, g)
    x = normal_bf16(rng(config_id, M), (M, K))
    return {"x": x, **qw}


def periodic_rows(block: np.ndarray, M: int) -> np.ndarray:
    """Rows 0..M-1 taken from `block` in turn (row r = block[r % len(block)]): a large activation
    matrix from a small random one. With a block length that divides no power of two (a prime),
    a row read at an offset wrapped by any power of two of bytes holds other values."""
    reps = -(-M // block.shape[0])
    return np.ascontiguousarray(np.tile(block, (reps,) + (1,) * (block.ndim - 1))[:M])


def make_w8a8_activations(config_id: int, M: int, K: int):
    """Per-token INT8 activations quantized from bf16 N(0,1)."""
    x = bf16_bits_to_f32(normal_bf16(rng(config_id, M), (M, K)))
    xq, s_tok = quantize_int8_rows(x)
    return {"xq": xq, "s_tok": s_tok}


def make_w8a8(config_id: int, M: int, N: int, K: int):
    """Dense W8A8: per-channel INT8 weights, per-token INT8 activations from bf16 N(0,1)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    wq, s_ch = quantize_int8_rows(w)
    return {**make_w8a8_activations(config_id, M, K), "wq": wq, "s_ch": s_ch}


def make_w4a8_activations(config_id: int, M: int, K: int):
    """Per-token FP8 e4m3 activations quantized from bf16 N(0,1)."""
    x = bf16_bits_to_f32(normal_bf16(rng(config_id, M), (M, K)))
    xq, s_tok = quantize_fp8_rows(x)
    return {"xq": xq, "s_tok": s_tok}


def make_w4a8(config_id: int, M: int, N: int, K: int):
    """Dense W4A8-MXFP4: MXFP4 weights, per-token FP8 e4m3 activations from bf16 N(0,1)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    qw = quantize_mxfp4(w)
    return {**make_w4a8_activations(config_id, M, K), **qw}


def quantize_mxfp8_rows(x: np.ndarray):
    """MXFP8 (OCP MX): e4m3 elements in 32-element blocks along K with an e8m0 shared exponent
    floor(log2 amax) - 8; elements by torch's e4m3 cast of the clamped scaled values.
    Returns codes uint8 [M, K], scales uint8 [M, K/32]."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    xb = x.reshape(M, K // 32, 32)
    amax = np.abs(xb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0
    e = np.where(amax > 0, np.clip(e, -127, 127), -127)
    v = np.clip(xb / np.exp2(e)[:, :, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v.reshape(M, K)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), (e + 127).astype(np.uint8)


def make_w4a8mx(config_id: int, M: int, N: int, K: int):
    """W4A8 with MXFP8 activations: MXFP4 weights (as W4A8), MXFP8 activations from bf16 N(0,1)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    x = bf16_bits_to_f32(normal_bf16(rng(config_id, M), (M, K)))
    xq, xs = quantize_mxfp8_rows(x)
    return {"xq": xq, "xs": xs, **quantize_mxfp4(w)}


def make_w4a16mx(config_id: int, M: int, N: int, K: int):
    """Dense W4A16-MXFP4: bf16 N(0,1) activations, MXFP4 weights from N(0, 0.02)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return {"x": normal_bf16(rng(config_id, M), (M, K)), **quantize_mxfp4(w)}


def make_w8a16(config_id: int, M: int, N: int, K: int, fp8: bool = False):
    """Dense 8-bit weights with bf16 activations: bf16 N(0,1) activations; weights N(0, 0.02)
    quantized per output channel to symmetric INT8 (s = absmax/127) or FP8 e4m3 (s = absmax/448)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    wq, s_ch = quantize_fp8_rows(w) if fp8 else quantize_int8_rows(w)
    return {"x": normal_bf16(rng(config_id, M), (M, K)), "wq": wq, "s_ch": s_ch}


def make_moe_weights_expert_mx(config_id: int, e: int, N: int, K: int):
    """One expert's MXFP4 weights, drawn from its own stream [config, 1, e]."""
    w = rng(config_id, 1, e).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return quantize_mxfp4(w)


def quantize_fp8_blocks(x: np.ndarray, bm: int, bk: int):
    """e4m3 codes with an fp32 scale per (bm x bk) block: s = amax / 448 (1 for a zero block),
    codes by torch's e4m3 cast of clamp(x / s). Returns codes uint8 [R, C], scales fp32 [R/bm, C/bk]."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    xb = x.reshape(R // bm, bm, C // bk, bk)
    amax = np.abs(xb).max(axis=(1, 3))
    s = (amax / np.float32(448.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    v = np.clip(xb / s[:, None, :, None], -448.0, 448.0).astype(np.float32).reshape(R, C)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), s


def make_w8a8_fp8_block(config_id: int, M: int, N: int, K: int):
    """Block-scaled FP8 W8A8: weights N(0, 0.02) with a scale per 128 x 128 block, activations
    bf16 N(0,1) with a scale per (token, 128 k)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    wq, ws = quantize_fp8_blocks(w, 128, 128)
    x = bf16_bits_to_f32(normal_bf16(rng(config_id, M), (M, K)))
    xq, xs = quantize_fp8_blocks(x, 1, 128)
    return {"xq": xq, "xs": xs, "wq": wq, "ws": ws}


def make_moe_weights_expert_w8a8(config_id: int, e: int, N: int, K: int):
    """One expert's INT8 weights with an fp32 scale per channel, from its own stream [config, 2, e]."""
    w = rng(config_id, 2, e).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    q, s = quantize_int8_rows(w)
    return {"wq": q, "s_ch": s}


def make_moe_weights_expert_fp8b(config_id: int, e: int, N: int, K: int):
    """One expert's FP8 e4m3 weights with an fp32 scale per 128 x 128 block, from its own stream
    [config, 3, e]."""
    w = rng(config_id, 3, e).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    q, s = quantize_fp8_blocks(w, 128, 128)
    return {"wq": q, "ws": s}


def random_fp8b_expert(g: np.random.Generator, N: int, K: int):
    """Random finite e4m3 codes with block scales near 1/448 (MoE benchmark and large parity tests:
    drawing and quantizing normals for many experts is slow, the kernel's work does not depend on
    the values)."""
    q = g.integers(0, 256, (N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] -= 1                       # the two NaN codes -> +-448
    s = (np.float32(1.0 / 448.0) * (1 + 0.25 * g.random((N // 128, K // 128)))).astype(np.float32)
    return {"wq": q, "ws": s}


def make_w4a4_activations(config_id: int, M: int, K: int):
    """MXFP4 activations (e2m1 codes + e8m0 per 32 k) quantized from bf16 N(0,1) by the OCP MX
    rule (the same quantizer as the weights')."""
    x = bf16_bits_to_f32(normal_bf16(rng(config_id, M), (M, K)))
    q = quantize_mxfp4(x)
    return {"xq": q["wq"], "xs": q["scales"]}


def make_w4a4(config_id: int, M: int, N: int, K: int):
    """Dense W4A4-MXFP4: MXFP4 weights (as W4A8) and MXFP4 activations from bf16 N(0,1)."""
    w = rng(config_id, 0).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return {**make_w4a4_activations(config_id, M, K), **quantize_mxfp4(w)}


def random_int4_sym_expert(g: np.random.Generator, N: int, K: int, gs: int = 128):
    """Standard-format symmetric INT4 weights with uniformly random codes and bf16 scales near
    absmax/7 of N(0, 0.02) groups. Used where only the data volume matters (throughput runs
    over hundreds of experts), since drawing and quantizing billions of normals is slow."""
    wq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = (0.0094 * (1.0 + 0.1 * g.standard_normal((N, K // gs)))).astype(np.float32)
    return {"wq": wq, "scales": bf16_bits(s)}


def random_int8_expert(g: np.random.Generator, N: int, K: int):
    """INT8 weights with uniformly random codes in [-127, 127] and fp32 channel scales near
    absmax/127 of N(0, 0.02) rows (for throughput runs over hundreds of experts)."""
    wq = g.integers(-127, 128, (N, K), dtype=np.int8)
    s = (7e-4 * (1.0 + 0.1 * g.standard_normal(N))).astype(np.float32)
    return {"wq": wq, "s_ch": s}


def random_mxfp4_expert(g: np.random.Generator, N: int, K: int):
    """MXFP4 weights with uniformly random e2m1 codes and e8m0 exponents 2^-9 .. 2^-6 (the range
    N(0, 0.02) blocks quantize to), for throughput runs over hundreds of experts."""
    wq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = g.integers(118, 122, (N, K // 32), dtype=np.uint8)
    return {"wq": wq, "scales": scales}


def make_moe_weights_expert(config_id: int, e: int, N: int, K: int, g: int = 128):
    """One expert's symmetric INT4 group-g weights, drawn from its own stream [config, 0, e]."""
    w = rng(config_id, 0, e).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return quantize_int4_sym(w, g)


def make_moe_inputs(config_id: int, T: int, K: int, E: int = 256, topk: int = 8):
    """MoE activations bf16 [T, K] and skewed routing (the expert prior is seeded per config,
    so every T shares one expert popularity order)."""
    g = rng(config_id, T)
    x = normal_bf16(g, (T, K))
    ids, w = moe_routing(g, T, E, topk, bias_rng=rng(config_id, 1 << 20))
    return {"x": x, "topk_ids": ids, "topk_weights": w}
