// layout.h -- the prepacked weight layout shared by the host prepack and the gfx950 kernels.
//
// The weights are split into "units": 16 output channels (one MFMA column tile) by one K unit.
// A unit's codes are exactly 1 KiB, laid out as the B operand of a wave-wide MFMA: 64 lanes x
// 16 bytes, so one coalesced 128-bit load per lane fetches the whole unit. Lane l owns output
// channel n = 16*nt + (l & 15) and a contiguous K slice selected by (l >> 4):
//
//   WNA16 (INT4, K unit 128 = one quantization group, v_mfma_f32_16x16x32_bf16 x 4):
//     lane l holds k = 128*kt + 32*(l>>4) + 8*d + j  in dword d (0..3), j = 0..7.
//     Inside a dword, nibble slot p (bits 4p..4p+3) holds j = 2*(p & 3) + (p >> 2), i.e. the
//     order k0 k2 k4 k6 k1 k3 k5 k7, so (dword >> 4i) & 0x000F000F yields the pair (k 2i, 2i+1)
//     as two 16-bit lanes. Codes are stored as unsigned u in [0, 15]: u = q (asymmetric) or
//     u = q + 8 (symmetric, i.e. the two's-complement nibble with bit 3 flipped); the kernel
//     always computes u - z with z = 8 for symmetric weights.
//   W8A8 (INT8, K unit 64, v_mfma_i32_16x16x64_i8):
//     lane l holds k = 64*kt + 16*(l>>4) + j in byte j (0..15).
//   W4A8 (FP4, K unit 128 = four MX blocks, v_mfma_scale_f32_16x16x128_f8f6f4):
//     lane l holds k = 128*kt + 32*(l>>4) + j in nibble j (0..31, low nibble first): exactly one
//     32-element MX block, so the lane's e8m0 byte is that block's scale (the MFMA takes block b's
//     scale from lane group b). The fp8 activations are fed in the instruction's own 8-bit A
//     layout (two 16-byte halves per lane, see device_ops.h).
//
//   W8A16 / F8A16 (8-bit INT8 or FP8 e4m3 weights with bf16 activations, K step 128 = two 64-k
//   units, v_mfma_f32_16x16x32_bf16 x 4 per step): in step kt, unit j (0, 1) lane l holds
//     k = 128*kt + 32*(l>>4) + 16*j + b in byte b (0..15),
//   so a lane's two units cover its lane group's 32 consecutive k of the step, the WNA16 K
//   order: MFMA d (0..3) of the step takes unit d>>1, bytes 8*(d&1) .. +7.
//   WNA2 (UINT2 with zero-points, group 128, bf16 activations; v_mfma_f32_16x16x32_bf16 x 4 per
//   group): a unit is 16 channels x 128 k in 512 bytes (half a 1 KiB unit); lane l holds 8 bytes,
//   k = 128*kt + 32*(l>>4) + 16*h + c in dword h (0, 1), code c = 2s + e (s = 0..7, e = 0, 1) in
//   bits 16*e + 2*s .. +1, so (dword >> 2s) & 0x00030003 yields the pair (k 2s, 2s+1) as two
//   16-bit lanes. Scales and zeros as WNA16's (zeros 0..3 in the 4-bit slots).
//   WNA3 (UINT3 with zero-points): a unit is 768 bytes, the low two bits of each code in WNA2's
//   512-byte layout, then 256 bytes of high bits: lane l's dword at 512 + 4*l holds the high bit
//   of code c = 2s + e of dword h in bit 16*e + 8*h + s.
//
// Regions per expert (each starts at a 256-byte aligned offset; experts are stacked with a
// 256-byte aligned stride):
//   codes : [N/16][K/KU] units of 1024 bytes (K units of one channel tile are contiguous)
//   WNA16 scales: [N/16][K/128][16] bf16;  zeros (asym): [N/16][K/128][8] bytes, byte i holds
//                 the zero of channel 2i (low nibble) and 2i+1 (high nibble)
//   W8A8, W8A16, F8A16 scales: [N] fp32 per channel
//   W4A8  scales: [N/16][K/128][64] e8m0 bytes, byte l = scale of lane l's block
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace hq {

// W4A4, W4A8 with MXFP8 activations (W4A8MX) and MXFP4 weights with bf16 activations (MXW4A16)
// share W4A8's prepacked weights (MXFP4); only the activation operand differs.
// FP8B: block-scaled FP8 W8A8 (e4m3 weights with an fp32 scale per 128 x 128 block, e4m3
// activations with an fp32 scale per (row, 128 k)); its codes use W8A8's 64-k units.
// W8A16 / F8A16: INT8 / FP8 e4m3 weights with a per-channel fp32 scale and bf16 activations.
// WNA2 / WNA3: 2-bit / 3-bit WnA16 (UINT2 / UINT3 codes with zero-points, the WNA16 scale and
// zero layout).
enum Family { FAM_WNA16 = 0, FAM_W8A8 = 1, FAM_W4A8 = 2, FAM_W4A4 = 3, FAM_W4A8MX = 4, FAM_MXW4A16 = 5, FAM_FP8B = 6,
              FAM_W8A16 = 7, FAM_F8A16 = 8, FAM_WNA2 = 9, FAM_WNA3 = 10 };

// Integer group-wise weights with bf16 activations: group scales and zero-points, the offset-128
// operand (WNA16, WNA2).
inline constexpr bool family_int_groups(int f) { return f == FAM_WNA16 || f == FAM_WNA2 || f == FAM_WNA3; }

// 8-bit weight codes in 64-k units
inline constexpr bool family_8bit_weights(int f) {
  return f == FAM_W8A8 || f == FAM_FP8B || f == FAM_W8A16 || f == FAM_F8A16;
}

// bf16 activations (2 bytes per k)
inline constexpr bool family_bf16_act(int f) {
  return f == FAM_WNA16 || f == FAM_MXW4A16 || f == FAM_W8A16 || f == FAM_F8A16 || f == FAM_WNA2 || f == FAM_WNA3;
}

constexpr int kUnitBytes = 1024;
// Bytes of one 16-channel unit of codes (WNA2 / WNA3: 128 k of 2-bit / 3-bit codes).
inline constexpr int family_unit_bytes(int f) { return f == FAM_WNA2 ? 512 : f == FAM_WNA3 ? 768 : kUnitBytes; }
constexpr int kTileN = 16;

inline int family_k_unit(Family f) { return family_8bit_weights(f) ? 64 : 128; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PackedLayout {
  Family fam;
  bool asym;
  int64_t N, K;
  int64_t n_tiles, k_units;
  size_t codes_off, codes_bytes;
  size_t scales_off, scales_bytes;
  size_t zeros_off, zeros_bytes;
  size_t expert_stride;
};

inline PackedLayout make_layout(Family fam, bool asym, int64_t N, int64_t K) {
  PackedLayout L{};
  L.fam = fam;
  L.asym = asym;
  L.N = N;
  L.K = K;
  L.n_tiles = N / kTileN;
  L.k_units = K / family_k_unit(fam);
  L.codes_off = 0;
  L.codes_bytes = size_t(L.n_tiles) * size_t(L.k_units) * family_unit_bytes(fam);
  L.scales_off = align256(L.codes_bytes);
  if (family_int_groups(fam)) {
    L.scales_bytes = size_t(L.n_tiles) * L.k_units * 16 * 2;
  } else if (fam == FAM_W8A8 || fam == FAM_W8A16 || fam == FAM_F8A16) {
    L.scales_bytes = size_t(N) * 4;
  } else if (fam == FAM_FP8B) {
    // per 16-channel tile and 128-k step: the 128 x 128 block's fp32 scale, four copies (one
    // 16-byte copy granule)
    L.scales_bytes = size_t(L.n_tiles) * size_t(K / 128) * 16;
  } else {
    L.scales_bytes = size_t(L.n_tiles) * L.k_units * 64;
  }
  L.zeros_off = align256(L.scales_off + L.scales_bytes);
  L.zeros_bytes = (family_int_groups(fam) && asym) ? size_t(L.n_tiles) * L.k_units * 8 : 0;
  L.expert_stride = align256(L.zeros_off + L.zeros_bytes);
  return L;
}

}  // namespace hq
