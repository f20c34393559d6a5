// gemm_pingpong.hip -- the large-M fused-dequantization GEMM with eight waves in two ping-pong
// groups.
//
// Same computation as gemm_pipe.hip (the Humming announcement's larger-batch pipeline, section
// "Tuning and JIT compilation per workload"), scheduled so the matrix cores never wait for the
// memory work of their own SIMD:
//   - the workgroup's eight waves form two groups of four, one wave of each group per SIMD;
//   - every K step (128 k) a wave runs a memory phase (issue the direct-to-LDS copies of the step
//     S - 1 ahead, read its operand fragments of this step from LDS into registers) and then a
//     compute phase (dequantization, MFMAs and the group scaling, registers only);
//   - group 1 runs one phase behind group 0, and a workgroup barrier separates the phases, so
//     on each SIMD one wave computes while the other loads;
//   - S LDS slots (S = 3..5, per configuration) hold steps s (being read), s + 1 (landed or
//     landing) and s + 2 .. s + S - 1 (in flight); a wave waits only for its own copies of step
//     s + 1 before the barrier that ends its memory phase of step s, so a copy has about
//     2 S - 3 phases to land (more slots hide a longer HBM / L2 latency where the LDS allows).
// WNA16 keeps the offset-128 operand of the other kernels; the offset term is removed at the end
// (tile_epilogue.h).
//
// MoE grouped GEMM (WNA16): a workgroup's BM rows are one block of the token sort's output, all
// routed to one expert (block_m == BM); the rows are gathered through sorted_ids (token =
// id / topk), the expert's weights are read at its stride, and the stores scatter to the flat ids
// with the router weight. Blocks past the sorted rows carry expert -1 and exit at once.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "device_ops.h"
#include "gemm_common.h"
#include "internal.h"
#include "tile_epilogue.h"

namespace hq {

namespace {

template <int FAM>
struct PPTraits;
// kRowBytes: activation bytes per row per step of 128 k; kAScaleBytes: activation block-scale
// bytes per row per step (MXFP4 activations: one e8m0 byte per 32 k).
template <>
struct PPTraits<FAM_WNA16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 32;   // 16 bf16 group scales
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_WNA2> {   // 2-bit codes: 512 bytes per tile and step (half a unit)
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 32;   // 16 bf16 group scales
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_WNA3> {   // 3-bit codes: 768 bytes per tile and step, three 4-byte-per-lane copies
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 32;   // 16 bf16 group scales
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_W8A8> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 2;
  static constexpr int kMetaPerTile = 0;
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_FP8B> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 2;
  static constexpr int kMetaPerTile = 16;   // the block's fp32 weight scale, four copies
  static constexpr int kAScaleBytes = 4;    // fp32 activation scale of the row's 128-k block
};
template <>
struct PPTraits<FAM_W4A8> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 64;   // one e8m0 byte per lane
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_MXW4A16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 64;   // one e8m0 byte per lane
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_W8A16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 2;
  static constexpr int kMetaPerTile = 0;
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_F8A16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 2;
  static constexpr int kMetaPerTile = 0;
  static constexpr int kAScaleBytes = 0;
};
template <>
struct PPTraits<FAM_W4A8MX> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 64;
  static constexpr int kAScaleBytes = 4;
};
template <>
struct PPTraits<FAM_W4A4> {
  static constexpr int kRowBytes = 64;
  static constexpr int kUnitsPerStep = 1;
  static constexpr int kMetaPerTile = 64;
  static constexpr int kAScaleBytes = 4;
};

// Workgroup barrier that the instruction scheduler may not move work across: the phases around
// it must stay where they are for the two groups to alternate.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int FAM, int MW, int NTW, int WM, int WN, int STAGES>
struct PPShape {
  static_assert(WM * WN == 8, "eight waves");
  static_assert(STAGES >= 3 && STAGES <= 5, "three to five LDS slots");
  static constexpr int kStages = STAGES;
  static constexpr int BM = 16 * MW * WM;
  static constexpr int BN = 16 * NTW * WN;
  static constexpr int RB = PPTraits<FAM>::kRowBytes;  // activation bytes per row per step
  static constexpr int CPR = RB / 16;
  static constexpr int A_BYTES = BM * RB;
  static constexpr int NT = BN / 16;
  static constexpr int UPS = PPTraits<FAM>::kUnitsPerStep;
  static constexpr int TILE_STEP_BYTES = UPS * family_unit_bytes(FAM);   // weight bytes per tile and step
  // LDS bytes per tile and step: 3-bit units (768 bytes) each take a 1 KiB slot
  static constexpr int B_SLOT = FAM == FAM_WNA3 ? 1024 : TILE_STEP_BYTES;
  static constexpr int B_BYTES = NT * B_SLOT;
  static constexpr int MPT = PPTraits<FAM>::kMetaPerTile;
  static constexpr int META_BYTES = NT * MPT;
  static constexpr int META_PER_WAVE = META_BYTES / 8;
  static constexpr int META_LANES = META_PER_WAVE / 16;
  // activation block scales (MXFP4 activations): BM rows x 4 bytes, each wave copies BM / 8 rows
  static constexpr int ASC_BYTES = BM * PPTraits<FAM>::kAScaleBytes;
  static constexpr int STAGE = (A_BYTES + B_BYTES + META_BYTES + ASC_BYTES + 1023) / 1024 * 1024;
  static constexpr int LDS = kStages * STAGE;
  static constexpr int A_INSTR = A_BYTES / 1024 / 8;
  static constexpr int B_INSTR = FAM == FAM_WNA3 ? 3 * NT / 8 : B_BYTES / 1024 / 8;
  static constexpr int INSTR = A_INSTR + B_INSTR + (META_BYTES ? 1 : 0) + (ASC_BYTES ? 1 : 0);
  // the copies split evenly over the eight waves (shapes that do not are never launched)
  // the copies split evenly over the eight waves (shapes that do not are never launched), and
  // the copies of S - 2 steps in flight fit the 6-bit vmcnt
  static constexpr bool kValid = A_BYTES % (1024 * 8) == 0 && B_BYTES % (1024 * 8) == 0 &&
                                 META_BYTES % (16 * 8) == 0 && META_LANES <= 64 &&
                                 (ASC_BYTES == 0 || (BM % 8 == 0 && BM / 8 <= 64)) &&
                                 (kStages - 2) * INSTR < 64;
  static constexpr int LDS_OR_NONE = kValid ? LDS : 1 << 30;
};

template <int FAM, bool MOE, int MW, int NTW, int WM, int WN, int STAGES>
__global__ __launch_bounds__(512) void pp_gemm_kernel(KParams p, int tiles_m, int tiles_n) {
  using Sh = PPShape<FAM, MW, NTW, WM, WN, STAGES>;
  static_assert(Sh::kValid, "copies must split over the eight waves");
  using Acc = typename AccType<FAM>::type;
  constexpr int BM = Sh::BM, RB = Sh::RB, CPR = Sh::CPR, NT = Sh::NT, UPS = Sh::UPS;
  constexpr int S = Sh::kStages;
  extern __shared__ __align__(1024) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int group = wave >> 2;   // waves w and w + 4 share a SIMD
  const int wm = wave / WN;
  const int wn = wave % WN;

  // Dense: XCD-aware tile order (blocks are dealt to the eight XCDs round robin), then groups
  // of eight M tiles per N tile so that concurrently running workgroups share operands in L2.
  // MoE: block-major order. Only the first num_padded / BM blocks have work and the rest exit at
  // once, so the live tiles must be the first ones dealt, spread over every XCD; with tiles_n a
  // multiple of 8, an N tile then always lands on the same XCD, whose L2 keeps its slice of the
  // expert's weights for all of the expert's blocks.
  const int nwg = gridDim.x;
  const int pid = blockIdx.x;
  int mt, ntile;
  if constexpr (MOE) {
    mt = pid / tiles_n;
    ntile = pid % tiles_n;
  } else {
    const int lid = (nwg % 8 == 0) ? (pid % 8) * (nwg / 8) + pid / 8 : pid;
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int first_m = (lid / per_group) * GM;
    const int gm = min(GM, tiles_m - first_m);
    const int in_group = lid % per_group;
    mt = first_m + in_group % gm;
    ntile = in_group / gm;
  }
  const int row0 = mt * BM;
  const int nt_wg = ntile * NT;
  const int nt0 = nt_wg + wn * NTW;
  const uint8_t* w = p.w;
  // MoE: this wave's 16-row blocks up to the last one holding a routed row. The token sort puts
  // an expert's routed rows first in its blocks and the padding after them, so in a lightly
  // loaded expert's block the later row blocks are padding only: their MFMAs (and operand
  // reads) are skipped, their rows are never stored.
  int nlive = MW;
  if constexpr (MOE) {
    const int e = p.block_expert[mt];
    if (e < 0 || e >= p.E) return;     // the whole workgroup, before any barrier
    w += size_t(e) * p.expert_stride;
    nlive = 0;
#pragma unroll
    for (int mb = 0; mb < MW; ++mb) {
      const int id = p.sorted_ids[row0 + wm * 16 * MW + 16 * mb + (lane & 15)];
      if (__builtin_amdgcn_ballot_w64(id < p.M) != 0) nlive = mb + 1;
    }
  }

  // ---- per-lane sources of the stage copies (constant over K) ----
  uint32_t a_off[Sh::A_INSTR];
#pragma unroll
  for (int j = 0; j < Sh::A_INSTR; ++j) {
    const int q = (wave * Sh::A_INSTR + j) * 64 + lane;
    const int r = q / CPR;
    const int c = lds_chunk_swizzle(r, q % CPR, CPR);
    int src_row;   // rows past M (dense) and padding rows (MoE) are computed, never stored
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      src_row = id < p.M ? id / p.topk : 0;
    } else {
      src_row = min(row0 + r, p.M - 1);
    }
    a_off[j] = uint32_t(src_row) * uint32_t(p.K / 128 * RB) + uint32_t(c * 16);
  }
  // MoE: wave w copies rows [w * RPW, (w + 1) * RPW) of the block's activations. A block holds its
  // routed rows first and its padding after them, so when the first of these rows is padding all
  // of them are: the wave then issues no activation copies at all (lightly loaded experts' blocks
  // move only their routed rows). Nothing reads those rows: the row blocks after the last routed
  // row are never computed. Such a wave's stages have INSTR - A_INSTR copies each.
  bool a_skip = false;
  if constexpr (MOE) {
    constexpr int RPW = Sh::A_INSTR * 64 / CPR;   // rows per wave
    a_skip = __builtin_amdgcn_readfirstlane(p.sorted_ids[row0 + wave * RPW]) >= p.M;   // wave-uniform
  }
  // MXFP4 activations: lane i < BM / 8 of wave w copies the step's 4 scale bytes of row
  // w * BM / 8 + i
  const uint8_t* asc_src = nullptr;
  if constexpr (Sh::ASC_BYTES > 0) {
    const int r = wave * (BM / 8) + min(lane, BM / 8 - 1);
    int src_row;   // MoE: the row's token
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      src_row = id < p.M ? id / p.topk : 0;
    } else {
      src_row = min(row0 + r, p.M - 1);
    }
    asc_src = reinterpret_cast<const uint8_t*>(p.a_scale) + size_t(src_row) * (p.K / 32);
  }
  // metadata: this wave copies bytes [wave * META_PER_WAVE, +META_PER_WAVE) of the stage's
  // [tile][MPT] block, 16 per lane
  int meta_tile = 0, meta_byte = 0;
  if constexpr (Sh::META_BYTES > 0) {
    const int b = wave * Sh::META_PER_WAVE + 16 * min(lane, Sh::META_LANES - 1);
    meta_tile = b / Sh::MPT;
    meta_byte = b % Sh::MPT;
  }

  auto issue_stage = [&](int ks) {
    uint8_t* st = smem + (ks % S) * Sh::STAGE;
    if (!a_skip) {
#pragma unroll
      for (int j = 0; j < Sh::A_INSTR; ++j)
        lds_dma16(p.a + a_off[j] + size_t(ks) * RB, st + (wave * Sh::A_INSTR + j) * 1024);
    }
    uint8_t* sb = st + Sh::A_BYTES;
#pragma unroll
    for (int j = 0; j < Sh::B_INSTR; ++j) {
      const int u = wave * Sh::B_INSTR + j;
      if constexpr (FAM == FAM_WNA2) {
        // one copy moves the step's 512 bytes of tiles 2u (lanes 0-31) and 2u + 1 (lanes 32-63)
        const size_t unit = size_t(nt_wg + 2 * u + (lane >> 5)) * p.k_units + size_t(ks);
        lds_dma16(w + unit * 512 + 16 * (lane & 31), sb + u * 1024);
      } else if constexpr (FAM == FAM_WNA3) {
        // tile tl's 768-byte unit of the step in three 256-byte pieces (4 bytes per lane), an
        // exact image at the start of the tile's 1 KiB slot
        const int tl = wave * (Sh::NT / 8) + j / 3, c = j % 3;
        const size_t unit = size_t(nt_wg + tl) * p.k_units + size_t(ks);
        lds_dma4(w + unit * 768 + 256 * c + 4 * lane, sb + tl * 1024 + 256 * c);
      } else {
        const size_t unit = size_t(nt_wg + u / UPS) * p.k_units + size_t(ks) * UPS + (u % UPS);
        lds_dma16(w + unit * kUnitBytes + 16 * lane, sb + u * 1024);
      }
    }
    if constexpr (Sh::META_BYTES > 0) {
      // lanes past META_LANES skip the copy (a direct-to-LDS load writes lane i at base + 16 i);
      // the instruction still counts once in this wave's vmcnt
      const size_t unit = size_t(nt_wg + meta_tile) * (p.k_units / UPS) + ks;
      if (lane < Sh::META_LANES)
        lds_dma16(w + p.scales_off + unit * Sh::MPT + meta_byte, sb + Sh::B_BYTES + wave * Sh::META_PER_WAVE);
    }
    if constexpr (Sh::ASC_BYTES > 0) {
      if (lane < BM / 8)
        lds_dma4(asc_src + 4 * ks, sb + Sh::B_BYTES + Sh::META_BYTES + wave * (BM / 8) * 4);
    }
  };

  auto read_a = [&](const uint8_t* st, int mb, int chunk) -> u32x4 {
    const int r = wm * 16 * MW + 16 * mb + (lane & 15);
    return *reinterpret_cast<const u32x4*>(st + r * RB + lds_chunk_swizzle(r, chunk, CPR) * 16);
  };
  auto read_b = [&](const uint8_t* st, int t, int q) -> u32x4 {
    if constexpr (FAM == FAM_WNA2) {   // 8 bytes per lane of the tile's 512
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = *reinterpret_cast<const u32x2*>(st + Sh::A_BYTES + (wn * NTW + t) * 512 + 8 * lane);
      return u32x4{v[0], v[1], 0u, 0u};
    } else if constexpr (FAM == FAM_WNA3) {   // low bits: 8 bytes per lane; high bits: 4
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const uint8_t* b = st + Sh::A_BYTES + (wn * NTW + t) * 1024;
      const u32x2 v = *reinterpret_cast<const u32x2*>(b + 8 * lane);
      return u32x4{v[0], v[1], *reinterpret_cast<const uint32_t*>(b + 512 + 4 * lane), 0u};
    } else {
      const int u = (wn * NTW + t) * UPS + q;
      return *reinterpret_cast<const u32x4*>(st + Sh::A_BYTES + u * 1024 + 16 * lane);
    }
  };

  Acc acc[MW][NTW];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mb][t] = Acc{0, 0, 0, 0};

  // Operand fragments of one step, filled by the memory phase and used by the compute phase.
  constexpr bool BF16A = family_bf16_act(FAM);   // bf16 activations
  constexpr int NA = BF16A ? 4 : (FAM == FAM_W4A4 ? 1 : 2);   // activation fragments per row block
  constexpr int NB = family_8bit_weights(FAM) ? 2 : 1;    // packed weight fragments per channel tile
  u32x4 af[MW][NA];
  u32x4 bq[NTW][NB];
  uint32_t meta[NTW];
  int asf[MW];   // MXFP4 activations: this lane's row block scale
  float asr[MW][4];   // block-scaled FP8: the activation scale of each output row of the lane

  auto memory_phase = [&](int ks, auto nmb) {
    constexpr int NMB = decltype(nmb)::value;   // row blocks with routed rows (MoE) or MW
    const uint8_t* st = smem + (ks % S) * Sh::STAGE;
    const uint8_t* sm = st + Sh::A_BYTES + Sh::B_BYTES;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int d = 0; d < NA; ++d) {
        // WNA16: lane group g holds k 32g..32g+31 of the step (chunks 4g..4g+3); 8-bit
        // activations: MFMA d takes chunk 4d + g (W8A8: k 64d + 16g..; W4A8: the two halves)
        const int chunk = BF16A ? 4 * (lane >> 4) + d : 4 * d + (lane >> 4);
        af[mb][d] = read_a(st, mb, chunk);
      }
    if constexpr (FAM == FAM_FP8B) {
      const float* sa = reinterpret_cast<const float*>(sm + Sh::META_BYTES);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) asr[mb][i] = sa[wm * 16 * MW + 16 * mb + 4 * (lane >> 4) + i];
    } else if constexpr (Sh::ASC_BYTES > 0) {
      const uint8_t* sa = sm + Sh::META_BYTES;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        asf[mb] = sa[(wm * 16 * MW + 16 * mb + (lane & 15)) * 4 + (lane >> 4)];
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
#pragma unroll
      for (int q = 0; q < NB; ++q) bq[t][q] = read_b(st, t, q);
      const int tw = wn * NTW + t;
      if constexpr (family_int_groups(FAM))
        meta[t] = *reinterpret_cast<const uint16_t*>(sm + tw * 32 + 2 * (lane & 15));
      else if constexpr (FAM == FAM_W4A8 || FAM == FAM_W4A4 || FAM == FAM_W4A8MX || FAM == FAM_MXW4A16)
        meta[t] = sm[tw * 64 + lane];
      else if constexpr (FAM == FAM_FP8B)
        meta[t] = *reinterpret_cast<const uint32_t*>(sm + tw * 16);
    }
  };

  auto compute_phase = [&](auto nmb) {
    constexpr int NMB = decltype(nmb)::value;
    if constexpr (family_int_groups(FAM)) {
      // Software-pipelined over the channel tiles: while the MFMAs of tile t run, the VALU
      // dequantizes tile t + 1 and applies the group scale to tile t - 1's partial sums.
      bf16x8 bw[2][4];
      f32x4 part[2][MW];
#pragma unroll
      for (int d = 0; d < 4; ++d) bw[0][d] = dequant_offset128<FAM>(bq[0][0], d);
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int cur = t & 1;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            part[cur][mb] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), bw[cur][d],
                                      d == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[cur][mb]);
        if (t + 1 < NTW) {
#pragma unroll
          for (int d = 0; d < 4; ++d) bw[cur ^ 1][d] = dequant_offset128<FAM>(bq[t + 1][0], d);
        }
        if (t > 0) {
          const float s = __uint_as_float(meta[t - 1] << 16);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) acc[mb][t - 1] += part[cur ^ 1][mb] * s;
        }
      }
      {
        const float s = __uint_as_float(meta[NTW - 1] << 16);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb][NTW - 1] += part[(NTW - 1) & 1][mb] * s;
      }
      // issue order: one MFMA, then up to three VALU instructions
#pragma unroll
      for (int i = 0; i < 4 * NMB * NTW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    } else if constexpr (FAM == FAM_MXW4A16) {
      // the lane's 32 weights of a tile share k block (lane >> 4): its scale is folded into the
      // conversion, and the MFMAs accumulate straight into the tile
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float s = e8m0_to_f32(meta[t]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_fp4x8_scaled(bq[t][0][d], s);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) acc[mb][t] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), bv, acc[mb][t]);
        }
      }
    } else if constexpr (FAM == FAM_W8A16 || FAM == FAM_F8A16) {
      // 8-bit codes of the step's two units -> bf16, MFMA d taking unit d >> 1; the per-channel
      // scale is applied in the epilogue
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_w8_step<FAM == FAM_F8A16>(bq[t][0], bq[t][NB - 1], d);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) acc[mb][t] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), bv, acc[mb][t]);
        }
    } else if constexpr (FAM == FAM_FP8B) {
      // A wave's NTW tiles (NTW divides 8, first tile a multiple of NTW) lie in one 128-channel
      // scale block, so one factor per output row serves all of them. All MFMAs of the step
      // first, then the scaled accumulation of their partial sums.
      const float sw = __uint_as_float(meta[0]);
      float c[MW][4];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) c[mb][i] = asr[mb][i] * sw;
      f32x4 part[MW][NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          part[mb][t] = mfma_fp8_fp8(af[mb][0], af[mb][1], bq[t][0], bq[t][1], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][t][i] += part[mb][t][i] * c[mb][i];
    } else if constexpr (FAM == FAM_W8A8) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) acc[mb][t] = mfma_i8(af[mb][q], bq[t][q], acc[mb][t]);
    } else if constexpr (FAM == FAM_W4A4) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb][t] = mfma_fp4_fp4(af[mb][0], asf[mb], bq[t][0], int(meta[t]), acc[mb][t]);
    } else if constexpr (FAM == FAM_W4A8MX) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb][t] = mfma_fp8_fp4(af[mb][0], af[mb][1], bq[t][0], int(meta[t]), acc[mb][t], asf[mb]);
    } else {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb][t] = mfma_fp8_fp4(af[mb][0], af[mb][1], bq[t][0], int(meta[t]), acc[mb][t]);
    }
  };

  const int nks = p.K / 128;
  // Wait until this wave's copies of every step up to `step` have landed, given that the copies
  // of the steps after it, up to min(step + S - 2, nks - 1), may still be in flight (I copies per
  // stage: INSTR, or INSTR - A_INSTR for a wave that skips its activation copies).
  auto wait_step_n = [&](int step, auto instr) __attribute__((always_inline)) {
    constexpr int I = decltype(instr)::value;
    const int after = min(S - 2, nks - 1 - step);
    if (after >= 3) wait_vmcnt<(S >= 5 ? 3 : 0) * I>();
    else if (after == 2) wait_vmcnt<(S >= 4 ? 2 : 0) * I>();
    else if (after == 1) wait_vmcnt<I>();
    else wait_vmcnt<0>();
  };
  auto wait_step = [&](int step) __attribute__((always_inline)) {
    if (MOE && a_skip) wait_step_n(step, std::integral_constant<int, Sh::INSTR - Sh::A_INSTR>{});
    else wait_step_n(step, std::integral_constant<int, Sh::INSTR>{});
  };

#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < nks) issue_stage(j);
  wait_step(0);
  phase_barrier();
  if (group == 1) phase_barrier();   // group 1 runs one phase behind

  // The main loop over row blocks 0 .. NMB - 1 (MoE: all of them, only the first, or none, and
  // with four row blocks per wave every count; each count a loop of its own so that each keeps
  // its own register allocation).
  auto main_loop = [&](auto nmb) {
    for (int ks = 0; ks < nks; ++ks) {
      // memory phase of step ks: the slot of step ks + S - 1 held step ks - 1, which both groups
      // finished reading before the barrier that opened this phase
      if (ks + S - 1 < nks) issue_stage(ks + S - 1);
      if constexpr (decltype(nmb)::value > 0) memory_phase(ks, nmb);
      wait_step(ks + 1);   // own copies of step ks + 1 have landed
      wait_lgkm0();
      phase_barrier();
      if constexpr (decltype(nmb)::value > 0) compute_phase(nmb);
      // group 1's last compute phase needs no closing barrier; the counts of the groups match
      if (!(group == 1 && ks == nks - 1)) phase_barrier();
    }
  };
  if constexpr (!MOE) {
    main_loop(std::integral_constant<int, MW>{});
  } else if constexpr (MW == 4) {   // 128-row blocks: every count of live row blocks
    if (nlive == 4) main_loop(std::integral_constant<int, 4>{});
    else if (nlive == 3) main_loop(std::integral_constant<int, 3>{});
    else if (nlive == 2) main_loop(std::integral_constant<int, 2>{});
    else if (nlive == 1) main_loop(std::integral_constant<int, 1>{});
    else main_loop(std::integral_constant<int, 0>{});
  } else {
    if (nlive == MW || nlive > 1) main_loop(std::integral_constant<int, MW>{});
    else if (nlive == 1) main_loop(std::integral_constant<int, 1>{});
    else main_loop(std::integral_constant<int, 0>{});
  }

  const int row_base = row0 + wm * 16 * MW;
  if constexpr (family_int_groups(FAM)) wna16_offset_contraction<MW, NTW, MOE>(p, w, acc, row_base, nt0, lane);
  store_tile<FAM, MOE, MW, NTW>(p, w, acc, row_base, nt0, lane);
}

// Group sums of bf16 activation rows over 128-k groups, split into bf16 high and low halves:
// ws[row][0][g] = hi, ws[row][1][g] = lo with hi + lo = the fp32 sum to about 16 bits; groups
// G..Gp-1 are zero. One wave per (row, four groups): lane l loads 16 bytes (8 values) of group
// 4 q + (l >> 4), the 16 lanes of a group add their partial sums in a fixed butterfly, and the
// group's first lane writes it. One load per lane, so the pass is a single memory round trip.
__global__ __launch_bounds__(256) void group_sums_split_kernel(const uint8_t* __restrict__ a, int rows,
                                                               int K, uint16_t* __restrict__ ws) {
  const int G = K / 128;
  const int Gp = (G + 31) / 32 * 32;
  const int per_row = Gp / 4;   // waves per row
  const long wid = (long(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wid >= long(rows) * per_row) return;   // whole waves
  const long r = wid / per_row;
  const int g = int(wid % per_row) * 4 + (lane >> 4);
  float sum = 0.0f;
  if (g < G) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(a + (size_t(r) * K + size_t(g) * 128) * 2 + 16 * (lane & 15));
#pragma unroll
    for (int j = 0; j < 4; ++j) sum += __uint_as_float(v[j] << 16) + __uint_as_float(v[j] & 0xFFFF0000u);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
  if ((lane & 15) == 0) {
    const uint16_t hi = f32_to_bf16_rne(sum);
    const uint16_t lo = f32_to_bf16_rne(sum - __uint_as_float(uint32_t(hi) << 16));
    ws[size_t(r) * 2 * Gp + g] = hi;
    ws[size_t(r) * 2 * Gp + Gp + g] = lo;
  }
}

}  // namespace

static constexpr PPCfg kPP[] = {
    {4, 4, 2, 4},  // 0: 128 x 256, waves of 64 x 64
    {4, 4, 4, 2},  // 1: 256 x 128, waves of 64 x 64
    {2, 4, 4, 2},  // 2: 128 x 128, waves of 32 x 64
    {4, 2, 2, 4},  // 3: 128 x 128, waves of 64 x 32
    {2, 4, 2, 4},  // 4: 64 x 256, waves of 32 x 64 (MoE blocks of 64 rows)
    {2, 8, 2, 4},  // 5: 64 x 512, waves of 32 x 128
    {1, 8, 2, 4},  // 6: 32 x 512, waves of 16 x 128 (MoE blocks of 32 rows)
    {1, 4, 2, 4},  // 7: 32 x 256, waves of 16 x 64
    // deeper pipelines (more steps in flight) where the LDS allows
    {4, 4, 2, 4, 4},  // 8: as 0, four slots (8- and 4-bit activations)
    {4, 4, 2, 4, 5},  // 9: as 0, five slots (4-bit activations)
    {2, 4, 4, 2, 4},  // 10: as 2, four slots
    {4, 2, 2, 4, 4},  // 11: as 3, four slots
    {4, 4, 4, 2, 4},  // 12: as 1, four slots
    {2, 4, 2, 4, 4},  // 13: as 4, four slots
    // 256 x 256 tiles, waves of 64 x 128 (fewer LDS bytes per MFMA; 4- and 8-bit operands only)
    {4, 8, 4, 2, 3},  // 14: three slots
    {4, 8, 4, 2, 4},  // 15: four slots
};

const PPCfg* pp_configs(int* count) {
  *count = int(sizeof(kPP) / sizeof(kPP[0]));
  return kPP;
}

template <int FAM, int I>
constexpr int pp_lds_of() {
  return PPShape<FAM, kPP[I].mw, kPP[I].ntw, kPP[I].wm, kPP[I].wn, kPP[I].stages>::LDS_OR_NONE;
}

template <int FAM, int... I>
int pp_lds_table(int cfg, std::integer_sequence<int, I...>) {
  static const int t[] = {pp_lds_of<FAM, I>()...};
  return t[cfg];
}

int pp_lds_bytes(int fam, int cfg) {
  constexpr int n = int(sizeof(kPP) / sizeof(kPP[0]));
  if (cfg < 0 || cfg >= n) return 1 << 30;
  auto seq = std::make_integer_sequence<int, n>{};
  if (fam == FAM_WNA16) return pp_lds_table<FAM_WNA16>(cfg, seq);
  if (fam == FAM_WNA2) return pp_lds_table<FAM_WNA2>(cfg, seq);
  if (fam == FAM_WNA3) return pp_lds_table<FAM_WNA3>(cfg, seq);
  if (fam == FAM_W8A8) return pp_lds_table<FAM_W8A8>(cfg, seq);
  if (fam == FAM_W4A4) return pp_lds_table<FAM_W4A4>(cfg, seq);
  if (fam == FAM_W4A8MX) return pp_lds_table<FAM_W4A8MX>(cfg, seq);
  if (fam == FAM_MXW4A16) return pp_lds_table<FAM_MXW4A16>(cfg, seq);
  if (fam == FAM_FP8B) return pp_lds_table<FAM_FP8B>(cfg, seq);
  if (fam == FAM_W8A16) return pp_lds_table<FAM_W8A16>(cfg, seq);
  if (fam == FAM_F8A16) return pp_lds_table<FAM_F8A16>(cfg, seq);
  return pp_lds_table<FAM_W4A8>(cfg, seq);
}

template <int FAM, bool MOE, int I>
static hipError_t launch_pp_one(const KParams& p, dim3 grid, int tiles_m, int tiles_n, hipStream_t s) {
  constexpr PPCfg C = kPP[I];
  using Sh = PPShape<FAM, C.mw, C.ntw, C.wm, C.wn, C.stages>;
  // (MoE instantiations exist for every format: activation scales, where there are any, are
  // gathered per routed row from its token's row)
  // (MoE blocks have at most 128 rows: no MoE instantiation of the 256-row tiles)
  if constexpr (Sh::kValid && Sh::LDS <= 160 * 1024 && !(MOE && Sh::BM > 128)) {
    auto kern = pp_gemm_kernel<FAM, MOE, C.mw, C.ntw, C.wm, C.wn, C.stages>;
    if (Sh::LDS > 65536)
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    hipLaunchKernelGGL(kern, grid, dim3(512), Sh::LDS, s, p, tiles_m, tiles_n);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int FAM, bool MOE, int... I>
static hipError_t launch_pp_fam(const KParams& p, int cfg, dim3 grid, int tiles_m, int tiles_n,
                                hipStream_t s, std::integer_sequence<int, I...>) {
  using Fn = hipError_t (*)(const KParams&, dim3, int, int, hipStream_t);
  static const Fn table[] = {&launch_pp_one<FAM, MOE, I>...};
  return table[cfg](p, grid, tiles_m, tiles_n, s);
}

hipError_t launch_pingpong(const KParams& p, int fam, bool moe, int cfg, dim3 grid, int tiles_m,
                           int tiles_n, hipStream_t s) {
  constexpr int n = int(sizeof(kPP) / sizeof(kPP[0]));
  if (cfg < 0 || cfg >= n) return hipErrorInvalidValue;
  auto seq = std::make_integer_sequence<int, n>{};
  if (moe) {
    if (fam == FAM_WNA16) return launch_pp_fam<FAM_WNA16, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_WNA2) return launch_pp_fam<FAM_WNA2, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_WNA3) return launch_pp_fam<FAM_WNA3, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_MXW4A16) return launch_pp_fam<FAM_MXW4A16, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_W8A8) return launch_pp_fam<FAM_W8A8, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_W4A8) return launch_pp_fam<FAM_W4A8, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_FP8B) return launch_pp_fam<FAM_FP8B, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_W8A16) return launch_pp_fam<FAM_W8A16, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_F8A16) return launch_pp_fam<FAM_F8A16, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_W4A4) return launch_pp_fam<FAM_W4A4, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    if (fam == FAM_W4A8MX) return launch_pp_fam<FAM_W4A8MX, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
    return hipErrorInvalidValue;
  }
  if (fam == FAM_WNA16) return launch_pp_fam<FAM_WNA16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_WNA2) return launch_pp_fam<FAM_WNA2, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_WNA3) return launch_pp_fam<FAM_WNA3, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W8A8) return launch_pp_fam<FAM_W8A8, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W4A4) return launch_pp_fam<FAM_W4A4, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W4A8MX) return launch_pp_fam<FAM_W4A8MX, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_MXW4A16) return launch_pp_fam<FAM_MXW4A16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_FP8B) return launch_pp_fam<FAM_FP8B, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W8A16) return launch_pp_fam<FAM_W8A16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_F8A16) return launch_pp_fam<FAM_F8A16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  return launch_pp_fam<FAM_W4A8, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
}

size_t group_sums_split_bytes(int64_t rows, int64_t K) {
  const int64_t G = K / 128;
  return size_t(rows) * size_t((G + 31) / 32 * 32) * 4;
}

hipError_t launch_group_sums_split(const uint8_t* a, int rows, int K, void* ws, hipStream_t s) {
  const int G = K / 128;
  const long waves = long(rows) * ((G + 31) / 32 * 32 / 4);   // four waves per 256-thread block
  hipLaunchKernelGGL(group_sums_split_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, s, a,
                     rows, K, static_cast<uint16_t*>(ws));
  return hipGetLastError();
}

}  // namespace hq
