// device_ops.h -- gfx950 device building blocks of the fused-dequantization GEMM: operand
// fragments, in-register dequantization, MFMA wrappers and the output epilogue.
//
// MFMA operand convention (16x16xK, wave64): for A (activations, 16 rows) lane l supplies row
// (l & 15); for B (weights, 16 output channels) lane l supplies channel (l & 15); the K slice a
// lane supplies is selected by (l >> 4) and is the SAME for A and B, which is all a contraction
// needs. The fp32/int32 result tile D[16x16] leaves row 4*(l>>4)+i, column (l & 15) in element
// i of lane l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace hq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Weights are read exactly once per workgroup: stream them past the caches.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 4 bytes (3-bit weights: a lane's high bits), streamed.
__device__ __forceinline__ uint32_t ldg4_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// 8 bytes (2-bit weights: a lane's half unit), streamed; returned in the low two dwords.
__device__ __forceinline__ u32x4 ldg8_stream(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return u32x4{v[0], v[1], 0u, 0u};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two fp32 -> two bf16 bit patterns (round to nearest even), low half from a: gfx950's paired
// conversion instruction, one VALU operation for both (finite values and infinities round exactly
// as f32_to_bf16_rne does; a NaN stays a NaN).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- WNA16 dequantization -------------------------------------------------------------------
// One dword holds 8 unsigned 4-bit codes u of consecutive k in the slot order k0 k2 k4 k6 k1 k3
// k5 k7 (layout.h). Returns the 8 values (u - z), exactly representable in bf16 since
// |u - z| <= 15, as the MFMA's 8-element bf16 operand in k order.
__device__ __forceinline__ bf16x8 dequant_int4x8(uint32_t v, float z) {
  const uint32_t lo = v & 0x0F0F0F0Fu;          // bytes: k0 k4 k1 k5
  const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;   // bytes: k2 k6 k3 k7
  f32x2 p0 = {float(lo & 0xFFu) - z, float((lo >> 16) & 0xFFu) - z};
  f32x2 p1 = {float(hi & 0xFFu) - z, float((hi >> 16) & 0xFFu) - z};
  f32x2 p2 = {float((lo >> 8) & 0xFFu) - z, float(lo >> 24) - z};
  f32x2 p3 = {float((hi >> 8) & 0xFFu) - z, float(hi >> 24) - z};
  bf16x2 b0 = __builtin_convertvector(p0, bf16x2);
  bf16x2 b1 = __builtin_convertvector(p1, bf16x2);
  bf16x2 b2 = __builtin_convertvector(p2, bf16x2);
  bf16x2 b3 = __builtin_convertvector(p3, bf16x2);
  bf16x8 r = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
  return r;
}

// Cheaper form for kernels that remove the offset separately: returns (128 + u) for the 8 codes,
// exact in bf16 (0x4300 is 128.0 and its last mantissa bit weighs 1, so OR-ing a 4-bit u into the
// low bits adds u). One bit-select per pair of weights.
// Each output dword is (v >> 4j) & 0x000F000F | 0x43004300. gfx9 VOP3 encodings take no literal
// operand, so with both constants as literals the compiler emits v_and + v_or; holding them in
// registers (empty asm statements make them opaque) lets it select one v_and_or_b32 per dword.
__device__ __forceinline__ bf16x8 dequant_int4x8_offset128(uint32_t v) {
  uint32_t m = 0x000F000Fu, c = 0x43004300u;
  asm("" : "+s"(m));
  asm("" : "+v"(c));
  const uint32_t p0 = (v & m) | c;
  const uint32_t p1 = ((v >> 4) & m) | c;
  const uint32_t p2 = ((v >> 8) & m) | c;
  const uint32_t p3 = ((v >> 12) & m) | c;
  const u32x4 r = {p0, p1, p2, p3};
  return __builtin_bit_cast(bf16x8, r);
}

// 2-bit form (WNA2): one dword holds 16 codes u in [0, 3] of consecutive k, code 2s + e in bits
// 16 e + 2 s (layout.h); returns (128 + u) for the 8 codes of k 8 h .. 8 h + 7 (h = 0, 1) as the
// MFMA operand in k order, one bit-select per pair of weights as for 4-bit codes.
__device__ __forceinline__ bf16x8 dequant_uint2x8_offset128(uint32_t v, int h) {
  uint32_t m = 0x00030003u, c = 0x43004300u;
  asm("" : "+s"(m));
  asm("" : "+v"(c));
  const uint32_t w = v >> (8 * h);
  const uint32_t p0 = (w & m) | c;
  const uint32_t p1 = ((w >> 2) & m) | c;
  const uint32_t p2 = ((w >> 4) & m) | c;
  const uint32_t p3 = ((w >> 6) & m) | c;
  const u32x4 r = {p0, p1, p2, p3};
  return __builtin_bit_cast(bf16x8, r);
}

// 3-bit form (WNA3): low two bits of the 16 codes of dword `lo` as for 2-bit codes, high bits in
// dword `hi` (code 2s + e of low dword h in bit 16 e + 8 h + s); returns (128 + u) for codes
// 8 half .. 8 half + 7 of low dword h.
__device__ __forceinline__ bf16x8 dequant_uint3x8_offset128(uint32_t lo, uint32_t hi, int h, int half) {
  const uint32_t w = lo >> (8 * half);
  const uint32_t v = hi >> (8 * h + 4 * half);
  uint32_t p[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    p[s] = ((w >> (2 * s)) & 0x00030003u) | (((v >> s) & 0x00010001u) << 2) | 0x43004300u;
  const u32x4 r = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// The offset-128 operand of MFMA d (0..3) of a 128-k group from a lane's packed codes: 4-bit
// codes hold it in dword d, 2-bit codes in half d & 1 of dword d >> 1, 3-bit codes as 2-bit ones
// plus their high bits in dword 2.
template <int FAM>
__device__ __forceinline__ bf16x8 dequant_offset128(const u32x4& q, int d) {
  if constexpr (FAM == FAM_WNA2) return dequant_uint2x8_offset128(q[d >> 1], d & 1);
  else if constexpr (FAM == FAM_WNA3) return dequant_uint3x8_offset128(q[d >> 1], q[2], d >> 1, d & 1);
  else return dequant_int4x8_offset128(q[d]);
}

// -(128 + z) in all 8 bf16 slots (z in [0, 15]): the constant operand that removes the offset of
// dequant_int4x8_offset128 inside an MFMA chain.
__device__ __forceinline__ bf16x8 neg_offset_bf16x8(uint32_t z) {
  const uint32_t h = 0xC300u | z;
  const uint32_t pr = h | (h << 16);
  const u32x4 r = {pr, pr, pr, pr};
  return __builtin_bit_cast(bf16x8, r);
}

// ---- MFMA wrappers ------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with A = fp8 e4m3 (format 0) and B = fp4 e2m1 (format 4).
// Operand K layouts (established with an on-device probe of single-element products):
//   A, 8-bit: lane group g = l>>4 holds k = 16g + j in byte j (j < 16) and k = 64 + 16g + (j-16)
//             in byte j (j >= 16), i.e. two 16-byte halves;
//   B, 4-bit: lane group g holds k = 32g + j in nibble j (low nibble first), one contiguous block.
// The e8m0 scale of K block b (k in [32b, 32b+32)) is taken from lane group b's scale register,
// for A and for B alike. A is passed unscaled (127 = 2^0); B's scale is the weight block's.
__device__ __forceinline__ f32x4 mfma_fp8_fp4(u32x4 a_lo, u32x4 a_hi, u32x4 b, int b_scale,
                                              f32x4 c, int a_scale = 127) {
  i32x8 av = {int(a_lo[0]), int(a_lo[1]), int(a_lo[2]), int(a_lo[3]),
              int(a_hi[0]), int(a_hi[1]), int(a_hi[2]), int(a_hi[3])};
  i32x8 bv = {int(b[0]), int(b[1]), int(b[2]), int(b[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 4, 0, a_scale, 0, b_scale);
}

// Both operands fp8 e4m3 (formats 0 and 0), unit block scales: one 128-k step of A and B in the
// 8-bit layout above (each as two 16-byte halves).
__device__ __forceinline__ f32x4 mfma_fp8_fp8(u32x4 a_lo, u32x4 a_hi, u32x4 b_lo, u32x4 b_hi, f32x4 c) {
  i32x8 av = {int(a_lo[0]), int(a_lo[1]), int(a_lo[2]), int(a_lo[3]),
              int(a_hi[0]), int(a_hi[1]), int(a_hi[2]), int(a_hi[3])};
  i32x8 bv = {int(b_lo[0]), int(b_lo[1]), int(b_lo[2]), int(b_lo[3]),
              int(b_hi[0]), int(b_hi[1]), int(b_hi[2]), int(b_hi[3])};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

// Both operands fp4 e2m1 (formats 4 and 4), each with its own e8m0 block scales: 4-bit A takes
// the same K layout as 4-bit B (lane group g holds k = 32g + j in nibble j).
__device__ __forceinline__ f32x4 mfma_fp4_fp4(u32x4 a, int a_scale, u32x4 b, int b_scale, f32x4 c) {
  i32x8 av = {int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
  i32x8 bv = {int(b[0]), int(b[1]), int(b[2]), int(b[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, a_scale, 0, b_scale);
}

// ---- MXFP4 weights for the bf16 MFMA -----------------------------------------------------------
// e8m0 byte -> its power of two as binary32 (0 -> 2^-127, a subnormal; 255 -> NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : e == 255 ? __uint_as_float(0x7FC00000u) : __uint_as_float(e << 23);
}

// One dword of 8 e2m1 codes (k in nibble order, low nibble first) -> the 8 values times the block
// scale s, as the bf16 MFMA operand in k order: gfx950's scaled fp4 -> bf16 conversion, two
// codes per instruction. e2m1 values times a power of two are exact in bf16 (two significant
// bits) wherever the power of two is in bf16's range.
__device__ __forceinline__ bf16x8 dequant_fp4x8_scaled(uint32_t v, float s) {
  const bf16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0);
  const bf16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1);
  const bf16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2);
  const bf16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3);
  return bf16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// ---- 8-bit weights for the bf16 MFMA -----------------------------------------------------------
// Two dwords of 8 consecutive-k weight codes (byte b = k b, two's-complement INT8 or OCP e4m3) ->
// the 8 values as the bf16 MFMA operand in k order. Both are exact: |q| <= 128 needs 8
// significant bits, and every finite e4m3 value (4 significant bits, exponents 2^-9 .. 2^8) is a
// bf16 value. INT8: one sign-extending byte -> fp32 conversion per code (an SDWA byte select)
// and one fp32 pair -> bf16 pair pack per two codes; FP8: gfx950's fp8 pair -> bf16 pair
// conversion at unit scale, one per two codes.
__device__ __forceinline__ bf16x2 int8_pair_to_bf16(uint32_t v, int shift) {
  const f32x2 p = {float(int8_t(v >> shift)), float(int8_t(v >> (shift + 8)))};
  return __builtin_convertvector(p, bf16x2);
}
__device__ __forceinline__ bf16x8 dequant_int8x8(uint32_t lo, uint32_t hi) {
  const bf16x2 r0 = int8_pair_to_bf16(lo, 0), r1 = int8_pair_to_bf16(lo, 16);
  const bf16x2 r2 = int8_pair_to_bf16(hi, 0), r3 = int8_pair_to_bf16(hi, 16);
  return bf16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}
__device__ __forceinline__ bf16x8 dequant_fp8x8(uint32_t lo, uint32_t hi) {
  const bf16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}
// MFMA d (0..3) of a 128-k step of W8A16 / F8A16 weights: unit d >> 1 of the step (q0 / q1),
// dwords 2 (d & 1) and 2 (d & 1) + 1 (layout.h).
template <bool FP8>
__device__ __forceinline__ bf16x8 dequant_w8_step(const u32x4& q0, const u32x4& q1, int d) {
  const u32x4& q = d < 2 ? q0 : q1;
  const int i = 2 * (d & 1);
  if constexpr (FP8) return dequant_fp8x8(q[i], q[i + 1]);
  else return dequant_int8x8(q[i], q[i + 1]);
}

// Position of 16-byte chunk `chunk` of activation row `row` in an LDS tile with `cpr` chunks per
// row (an XOR swizzle, so each row's chunks stay a permutation of its own slots). For 128-byte
// rows the key is the row's low three bits. For 256-byte rows the plain key (row & 15) leaves the
// chunks that one ds_read_b128 fetches for lane groups 0 and 1 (chunks d and 4 + d) in the same
// bank group, which measures as a two-way conflict on gfx950; rotating the four key bits left by
// one measures conflict-free.
__device__ __forceinline__ int lds_chunk_swizzle(int row, int chunk, int cpr) {
  const int key = cpr == 16 ? (((row & 7) << 1) | ((row >> 3) & 1)) : (row & (cpr - 1));
  return chunk ^ key;
}

// ---- direct-to-LDS copies and wait counters ---------------------------------------------------
// One global -> LDS copy per lane: lane i's `bytes` (4 or 16) land at lds + bytes * i, where lds
// must be wave-uniform. The copy counts in the wave's vmcnt like any vector load, once per
// instruction whatever the lane mask.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters unconstrained (gfx9 encoding; n < 64).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads (and scalar loads) have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace hq
