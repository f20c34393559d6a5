"""Format decoders for the oracle (test infrastructure).

The Humming announcement names the formats (INT4, INT8, FP4, FP8, MXFP4, BF16; groups,
zero-points; section "Why quantized inference needs a general-purpose kernel library") but
defines no bit layouts. The definitions used here are the public ones:

* INT4 symmetric: a nibble is a two's-complement integer in [-8, 7].
* UINT4: a nibble is an unsigned integer in [0, 15]; zero-points are uint4 as well.
* INT8: two's complement.
* e2m1 (FP4, OCP Microscaling v1.0): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0,
  no infinities or NaN; exponent field 0 is subnormal.
* e8m0 (OCP MX scale): value 2^(b - 127), 0xFF is NaN.
* e4m3 (OCP 8-bit FP, "fn"): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
  exponent field 0 is subnormal; S.1111.111 is NaN; no infinities.
* bf16: the upper 16 bits of an IEEE binary32.
* zero-exponent "float e0mN" formats (section "Results: quantization support"): sign bit plus
  an N-bit magnitude, value = +-magnitude.
* packing: two 4-bit codes per byte, the low nibble holds the even K index (the pages are
  silent; this is the usual convention for packed 4-bit tensors).
"""
from __future__ import annotations

import numpy as np


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] nibble codes (uint8), low nibble first."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def unpack_crumbs(packed: np.ndarray) -> np.ndarray:
    """[..., K/4] bytes -> [..., K] 2-bit codes (uint8): code k sits in bits 2 (k % 4) and
    2 (k % 4) + 1 of byte k // 4 (lowest k in the lowest bits)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 4,), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (p >> (2 * j)) & 0x3
    return out


def unpack_triplets(packed: np.ndarray) -> np.ndarray:
    """[..., 3K/8] bytes -> [..., K] 3-bit codes (uint8): the row is one little-endian bit string
    and code k occupies its bits 3k .. 3k + 2 (lowest bit first)."""
    p = np.asarray(packed, dtype=np.uint8)
    bits = np.unpackbits(p, axis=-1, bitorder="little")                  # [..., 3K]
    b = bits.reshape(p.shape[:-1] + (-1, 3)).astype(np.uint8)
    return b[..., 0] | (b[..., 1] << 1) | (b[..., 2] << 2)


def decode_int4_sym(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64) & 0xF
    return np.where(c >= 8, c - 16, c)


def decode_uint4(codes: np.ndarray) -> np.ndarray:
    return np.asarray(codes).astype(np.int64) & 0xF


def decode_int8(b: np.ndarray) -> np.ndarray:
    return np.asarray(b).astype(np.uint8).view(np.int8).astype(np.int64)


def _e2m1_value(code: int) -> float:
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = (man / 2.0) * 2.0 ** (1 - 1)          # subnormal: 0.m x 2^(1 - bias)
    else:
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)  # normal: 1.m x 2^(e - bias)
    return sign * mag


_E2M1 = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    return _E2M1[np.asarray(codes).astype(np.int64) & 0xF]


def decode_e8m0(b: np.ndarray) -> np.ndarray:
    bi = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, bi - 127)
    return np.where(bi == 255, np.nan, v)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** (1 - 7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


_E4M3 = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(b: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(b).astype(np.int64) & 0xFF]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns with ONE round-to-nearest-even step (no detour via fp32).

    bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at 2^-133 (subnormals).
    Results beyond the largest finite bf16 become +-inf, NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                             # xf = f * 2^e, 0.5 <= |f| < 1
    quantum_exp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(xf, -quantum_exp))         # exact scaling; rint = half to even
    r = np.ldexp(r, quantum_exp)
    max_bf16 = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), dtype=np.float32)[0])
    over = np.abs(r) > max_bf16
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)                  # exact: r is a bf16 value (or overflows)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(over, np.where(r > 0, 0x7F80, 0xFF80), bits)
    nan_bits = np.uint16(0x7FC0)
    inf_bits = np.where(x > 0, 0x7F80, 0xFF80)
    out[...] = np.where(finite, bits, np.where(np.isnan(x), nan_bits, inf_bits))
    return out


def decode_sign_magnitude(codes: np.ndarray, bits: int) -> np.ndarray:
    """Zero-exponent float (e0m{bits-1}): top bit is the sign, the rest is the magnitude."""
    c = np.asarray(codes).astype(np.int64) & ((1 << bits) - 1)
    mag = c & ((1 << (bits - 1)) - 1)
    return np.where(c >> (bits - 1), -mag, mag)
