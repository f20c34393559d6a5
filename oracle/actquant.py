"""Per-token dynamic activation quantization for the oracle (test infrastructure).

The step just before the W8A8 and W4A8 GEMMs: bf16 activations become 8-bit codes plus one fp32
scale per row (token). The Humming announcement lists per-token activation scales among the
"input scale layout" compute options (section "Tuning and JIT compilation per workload") and
credits tokenwise FP8 activations for its end-to-end gain (section "End-to-end performance")
but fixes no rule; the plain reading used here is symmetric absmax scaling per row:

    amax   = max_k |x[m, k]|                         (exact: bf16 values)
    s[m]   = fp32(amax / Q), Q = 127 (INT8) or 448 (largest finite e4m3); s = 1 for an all-zero row
    v      = fp32(x[m, k] / s[m])                   (one IEEE binary32 division, round to nearest even)
    INT8   : q = clamp(round_half_even(v), -127, 127)
    e4m3   : q = nearest finite e4m3 ("fn") code to clamp(v, -448, 448), ties to the even code;
             a negative value that rounds to zero gives -0 (0x80)

MXFP4 activations (for W4A4) follow the OCP Microscaling (MX) v1.0 rule instead, per row and per
block of 32 consecutive k (the MXFP4 format the announcement's W4A4 path consumes, section
"Results: kernel microbenchmarks"):

    e      = floor(log2(max_k |x|)) - 2, clamped to [-127, 127]   (2 = largest e2m1 exponent)
    scale  = e8m0 byte e + 127; an all-zero block takes e = -127 (byte 0)
    v      = x * 2^-e                                   (exact: a power-of-two scaling)
    code   = nearest e2m1 value to v, ties to the even code, saturating at +-6; the sign bit is
             set only for a non-zero magnitude (a negative value that rounds to zero gives +0)

FP8 activations with block scales (for the block-scaled FP8 W8A8) apply the per-token e4m3 rule
above to every block of 128 consecutive k of a row instead of the whole row: s[m, g] =
fp32(max |x| over the block / 448) (1 for an all-zero block), codes = e4m3 of
clamp(fp32(x / s[m, g]), -448, 448).

MXFP8 activations (e4m3 elements, for W4A8 with MX activations) take the same rule with the
largest e4m3 exponent, 8: e = floor(log2(max |x|)) - 8 clamped to [-127, 127], v = x * 2^-e,
code = the e4m3 encoding above of clamp(v, -448, 448) (|v| < 512 always).

Both divisions are binary32 on purpose: the codes are integers decided by floating point, and
the kernel takes that decision in binary32, so the reference takes it in the same precision
(numpy float32 division is IEEE correctly rounded).
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_bf16, decode_e2m1, decode_e4m3

_E4M3_FINITE = np.array([c for c in range(0x80) if not (c & 0x7F) == 0x7F], dtype=np.int64)
_E4M3_VALUES = decode_e4m3(_E4M3_FINITE)          # non-negative finite magnitudes, ascending


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest finite OCP e4m3 code (uint8), ties to the even code, saturating at +-448.

    Brute force over the 127 non-negative finite magnitudes: the lowest code at minimum distance
    unless two codes tie, then the even one. The sign bit is copied from v (so -0.0 and negative
    values that round to zero give 0x80).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[..., None] - _E4M3_VALUES)                     # [..., 127]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    idx_lo = np.argmax(cand, axis=-1)                          # first (smaller) minimiser
    two = cand.sum(axis=-1) > 1                                # a tie: two neighbours
    lo_code = _E4M3_FINITE[idx_lo]
    code = np.where(two & (lo_code % 2 == 1), _E4M3_FINITE[np.minimum(idx_lo + 1, len(_E4M3_FINITE) - 1)], lo_code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _row_scale(x: np.ndarray, q: float) -> np.ndarray:
    amax = np.abs(x).max(axis=1).astype(np.float32)
    s = (amax / np.float32(q)).astype(np.float32)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def quantize_per_token(x_bf16: np.ndarray, act: str):
    """x_bf16: uint16 bf16 bits [M, K]; act: "int8" or "e4m3". Returns (codes uint8/int8 [M, K],
    scales float32 [M])."""
    x = decode_bf16(x_bf16).astype(np.float32)                 # exact
    if act == "int8":
        s = _row_scale(x, 127.0)
        v = (x / s[:, None]).astype(np.float32)                # binary32 division
        q = np.clip(np.rint(v), -127, 127).astype(np.int8)     # rint = half to even
        return q, s
    if act == "e4m3":
        s = _row_scale(x, 448.0)
        v = (x / s[:, None]).astype(np.float32)
        return encode_e4m3(np.clip(v, np.float32(-448.0), np.float32(448.0))), s
    raise ValueError(act)


_E2M1_POS = decode_e2m1(np.arange(8))                  # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (4 bits, bit 3 = sign) by brute force over the 8 magnitudes: the lowest
    code at minimum distance, or the even one of two tied neighbours; saturates at 6; the sign
    bit only for a non-zero magnitude."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - _E2M1_POS)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    lo = np.argmax(cand, axis=-1)
    two = cand.sum(axis=-1) > 1
    code = np.where(two & (lo % 2 == 1), lo + 1, lo)
    sign = (np.signbit(v) & (code != 0)).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def quantize_mxfp4_act(x_bf16: np.ndarray):
    """x_bf16: uint16 bf16 bits [M, K] (K % 32 == 0). Returns (packed e2m1 codes uint8 [M, K/2],
    low nibble = even k; e8m0 scale bytes uint8 [M, K/32])."""
    x = decode_bf16(x_bf16)                                     # exact, float64
    M, K = x.shape
    blocks = x.reshape(M, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.floor(np.log2(amax[nz])).astype(np.int64) - 2  # log2 of a bf16 value: exact floor
    e = np.clip(e, -127, 127)
    v = blocks * np.ldexp(1.0, -e)[:, :, None]
    codes = encode_e2m1(v).reshape(M, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def _mx_block_exponent(blocks: np.ndarray, emax: int) -> np.ndarray:
    amax = np.abs(blocks).max(axis=2)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.floor(np.log2(amax[nz])).astype(np.int64) - emax
    return np.clip(e, -127, 127)


def quantize_mxfp8_act(x_bf16: np.ndarray):
    """x_bf16: uint16 bf16 bits [M, K] (K % 32 == 0). Returns (e4m3 codes uint8 [M, K], e8m0
    scale bytes uint8 [M, K/32])."""
    x = decode_bf16(x_bf16)
    M, K = x.shape
    blocks = x.reshape(M, K // 32, 32)
    e = _mx_block_exponent(blocks, 8)
    v = blocks * np.ldexp(1.0, -e)[:, :, None]
    codes = encode_e4m3(np.clip(v, -448.0, 448.0)).reshape(M, K)
    return codes, (e + 127).astype(np.uint8)


def quantize_fp8_block_act(x_bf16: np.ndarray, block: int = 128):
    """x_bf16: uint16 bf16 bits [M, K] (K % block == 0). Returns (e4m3 codes uint8 [M, K], fp32
    scales [M, K/block]): the per-token e4m3 rule applied to each block of `block` k."""
    M, K = x_bf16.shape
    G = K // block
    xb = np.ascontiguousarray(np.asarray(x_bf16).reshape(M, G, block).transpose(1, 0, 2))  # [G, M, block]
    codes = np.empty((M, K), dtype=np.uint8)
    scales = np.empty((M, G), dtype=np.float32)
    for g in range(G):
        q, s = quantize_per_token(xb[g], "e4m3")
        codes[:, g * block:(g + 1) * block] = q
        scales[:, g] = s
    return codes, scales
