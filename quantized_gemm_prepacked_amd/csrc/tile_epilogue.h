// tile_epilogue.h -- the end of a wave's output tile in the LDS-staged GEMM kernels (tiled,
// pipelined, ping-pong): WNA16's offset-term contraction and the scaled bf16 / int32 stores.
//
// A wave owns (16*MW) x (16*NTW) outputs as MW x NTW MFMA tiles; lane l holds rows
// 4*(l>>4)+i (i = 0..3) of each 16-row block and column l&15 of each 16-channel tile. Every
// per-row and per-column factor the stores need (MoE row index, token scale, router weight,
// channel scale) is loaded once per tile, all loads issued together, before any store; the
// per-element arithmetic is the one of `epilogue` in gemm_common.h, in the same order.
#pragma once
#include "gemm_common.h"

namespace hq {

// ---- WNA16 offset term ---------------------------------------------------------------------
// The main loop summed x * (128 + u) per group. What remains is
//   acc[m][n] -= sum_g s[n,g] * (128 + z[n,g]) * S[m][g]      (S: group sums of row m of X)
// a K' = K/128 contraction, run on the bf16 MFMA over operands split into high and low bf16
// halves: hi*hi + hi*lo + lo*hi keeps ~16 significant bits of each product (the fp32 sums in the
// workspace are split to ~2^-17 relative; -s*(128+z) has 16 significant bits and splits
// exactly). Lane l supplies
// row / channel l&15 and groups 32*gb + 8*(l>>4) .. +7 of block gb; groups past G are zero.
// Workspace: per activation row, Gp = ceil(G/32)*32 bf16 high halves then Gp low halves
// (group_sums_split_kernel).
template <int MW, int NTW, bool MOE>
__device__ __forceinline__ void wna16_offset_contraction(const KParams& p, const uint8_t* w,
                                                         f32x4 (&acc)[MW][NTW], int row_base,
                                                         int nt0, int lane) {
  const int G = p.K / 128;
  const int Gp = (G + 31) / 32 * 32;
  const uint16_t* ssplit = reinterpret_cast<const uint16_t*>(p.ws);
  const int h = lane >> 4;
  int srow[MW];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb) {
    const int r = row_base + 16 * mb + (lane & 15);
    if constexpr (MOE) {
      const int id = p.sorted_ids[r];
      srow[mb] = id < p.M ? id / p.topk : 0;      // padding rows: any valid row, never stored
    } else {
      srow[mb] = min(r, p.M - 1);
    }
  }
  for (int gb = 0; gb < Gp / 32; ++gb) {
    u32x4 sh[MW], sl[MW];
#pragma unroll
    for (int mb = 0; mb < MW; ++mb) {
      const uint16_t* src = ssplit + size_t(srow[mb]) * 2 * Gp + 32 * gb + 8 * h;
      sh[mb] = *reinterpret_cast<const u32x4*>(src);
      sl[mb] = *reinterpret_cast<const u32x4*>(src + Gp);
    }
    // -s * (128 + z) of the lane's channel and 8 groups, exact in fp32 (8 x 8 significant
    // bits), split as hi = the value truncated to bf16 and lo = the exact rest (at most 8
    // significant bits, so its fp32 pattern has a zero low half): hi + lo is the value exactly
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const size_t tile_unit = size_t(nt0 + t) * p.k_units;
      const uint8_t* sbase = w + p.scales_off + tile_unit * 32 + 2 * (lane & 15);
      const uint8_t* zbase = w + p.zeros_off + tile_unit * 8 + ((lane & 15) >> 1);
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gj = 32 * gb + 8 * h + j;
        const int g = min(gj, G - 1);
        const float s = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sbase + g * 32));
        const uint32_t zb = p.asym ? uint32_t(zbase[g * 8]) : 0x88u;
        const uint32_t z = (lane & 1) ? (zb >> 4) : (zb & 0xFu);
        const float b = gj < G ? -s * float(128u + z) : 0.0f;
        const uint32_t hi = __float_as_uint(b) & 0xFFFF0000u;
        const uint32_t lo = __float_as_uint(b - __uint_as_float(hi));
        if (j & 1) {
          bh[j >> 1] |= hi;
          bl[j >> 1] |= lo & 0xFFFF0000u;
        } else {
          bh[j >> 1] = hi >> 16;
          bl[j >> 1] = lo >> 16;
        }
      }
      const bf16x8 bhv = __builtin_bit_cast(bf16x8, u32x4{bh[0], bh[1], bh[2], bh[3]});
      const bf16x8 blv = __builtin_bit_cast(bf16x8, u32x4{bl[0], bl[1], bl[2], bl[3]});
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        const bf16x8 shv = __builtin_bit_cast(bf16x8, sh[mb]);
        acc[mb][t] = mfma_bf16(shv, bhv, acc[mb][t]);
        acc[mb][t] = mfma_bf16(shv, blv, acc[mb][t]);
        acc[mb][t] = mfma_bf16(__builtin_bit_cast(bf16x8, sl[mb]), bhv, acc[mb][t]);
      }
    }
  }
}

// ---- stores ------------------------------------------------------------------------------------
// row_base: the wave's first row in the workgroup's row space (dense: m; MoE: position in
// sorted_ids). No K split here (p.split == 1).
// w: the weights of the expert (MoE) or the layer, for the per-channel scales.
template <int FAM, bool MOE, int MW, int NTW>
__device__ __forceinline__ void store_tile(const KParams& p, const uint8_t* w,
                                           const typename AccType<FAM>::type (&acc)[MW][NTW],
                                           int row_base, int nt0, int lane) {
  int orow[MW][4];     // output row, or -1 (not stored)
  float rs[MW][4];     // per-token activation scale (1 for bf16 activations)
  float tw[MW][4];     // router weight (1 for dense)
#pragma unroll
  for (int mb = 0; mb < MW; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row_base + 16 * mb + 4 * (lane >> 4) + i;
      int o, s;
      float wgt = 1.0f;
      if constexpr (MOE) {
        const int id = p.sorted_ids[r];
        o = id < p.M ? id : -1;
        s = id < p.M ? id / p.topk : 0;
        if (p.topk_weights && o >= 0) wgt = p.topk_weights[id];
      } else {
        o = r < p.M ? r : -1;
        s = r < p.M ? r : 0;
      }
      orow[mb][i] = o;
      tw[mb][i] = wgt;
      rs[mb][i] = ((FAM == FAM_W8A8 || FAM == FAM_W4A8) && o >= 0) ? p.a_scale[s] : 1.0f;
    }
  float cs[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int n = (nt0 + t) * 16 + (lane & 15);
    constexpr bool kChannelScale = FAM == FAM_W8A8 || FAM == FAM_W8A16 || FAM == FAM_F8A16;
    cs[t] = (kChannelScale && !p.out_i32) ? reinterpret_cast<const float*>(w + p.scales_off)[n] : 1.0f;
  }
  // One row pointer per output row (the lane's column of the wave's first tile); the tiles of the
  // row are 16 columns apart. bf16 results are rounded two at a time (tiles t, t + 1).
#pragma unroll
  for (int mb = 0; mb < MW; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = orow[mb][i];
      if (o < 0) continue;
      const size_t row_off = size_t(o) * p.N + size_t(nt0) * 16 + (lane & 15);
      if constexpr (FAM == FAM_W8A8) {
        if (p.out_i32) {
          int* yr = reinterpret_cast<int*>(p.y) + row_off;
#pragma unroll
          for (int t = 0; t < NTW; ++t) yr[16 * t] = acc[mb][t][i];
          continue;
        }
      }
      auto value = [&](int t) -> float {
        const auto v = acc[mb][t][i];
        if constexpr (family_int_groups(FAM)) return v * tw[mb][i];
        else if constexpr (FAM == FAM_W8A8) return float(v) * rs[mb][i] * cs[t] * tw[mb][i];
        else if constexpr (FAM == FAM_W8A16 || FAM == FAM_F8A16) return v * cs[t] * tw[mb][i];
        else return v * rs[mb][i] * tw[mb][i];
      };
      uint16_t* yr = reinterpret_cast<uint16_t*>(p.y) + row_off;
#pragma unroll
      for (int t = 0; t + 1 < NTW; t += 2) {
        const uint32_t pk = f32x2_to_bf16x2_rne(value(t), value(t + 1));
        yr[16 * t] = uint16_t(pk);
        yr[16 * (t + 1)] = uint16_t(pk >> 16);
      }
      if constexpr (NTW % 2 == 1) yr[16 * (NTW - 1)] = uint16_t(f32x2_to_bf16x2_rne(value(NTW - 1), 0.0f));
    }
}

}  // namespace hq
