// gemm_pipe.hip -- the large-M fused-dequantization GEMM with an asynchronous multi-stage
// global -> LDS pipeline (gfx950 global_load_lds_dwordx4).
//
// Same computation as gemm_tiled.hip (the Humming announcement's larger-batch pipeline, section
// "Tuning and JIT compilation per workload"), organised for latency hiding:
//   - every operand of a K step (activation tile, packed weight units, group scales and zeros)
//     is copied global -> LDS by direct-to-LDS loads, so no registers hold in-flight data;
//   - STAGES K steps are in flight in an LDS ring; a thread waits only for its own loads of the
//     step it is about to use (an exact vmcnt), then one workgroup barrier publishes the step
//     and, in the same place, retires the slot that the next loads overwrite;
//   - the weight units of a step are loaded once per workgroup and read by every wave that
//     needs them (no duplicate HBM/L2 traffic between waves along M).
// The activation tile is stored with a 16-byte chunk XOR swizzle (lds_chunk_swizzle) so MFMA
// operand reads are bank-conflict free; a direct-to-LDS load writes lane-contiguous chunks, so each lane
// fetches the global chunk that belongs at its swizzled position.
#include <hip/hip_runtime.h>

#include <utility>

#include "device_ops.h"
#include "gemm_common.h"
#include "internal.h"
#include "tile_epilogue.h"

namespace hq {

namespace {

template <int FAM>
struct PipeTraits;
template <>
struct PipeTraits<FAM_WNA16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 1;
};
template <>
struct PipeTraits<FAM_W8A8> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 2;
};
template <>
struct PipeTraits<FAM_W4A8> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 1;
};
template <>
struct PipeTraits<FAM_FP8B> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 2;
};
template <>
struct PipeTraits<FAM_MXW4A16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 1;
};
template <>
struct PipeTraits<FAM_W4A4> {
  static constexpr int kRowBytes = 64;
  static constexpr int kUnitsPerStep = 1;
};
template <>
struct PipeTraits<FAM_W4A8MX> {
  static constexpr int kRowBytes = 128;
  static constexpr int kUnitsPerStep = 1;
};
template <>
struct PipeTraits<FAM_W8A16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 2;
};
template <>
struct PipeTraits<FAM_F8A16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kUnitsPerStep = 2;
};

__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_barrier();
}

template <int FAM, int MW, int NTW, int WM, int WN, int STAGES, bool MOE>
struct PipeShape {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 16 * MW * WM;
  static constexpr int BN = 16 * NTW * WN;
  static constexpr int RB = PipeTraits<FAM>::kRowBytes;   // activation bytes per row per K step
  static constexpr int CPR = RB / 16;
  static constexpr int A_BYTES = BM * RB;
  static constexpr int NT = BN / 16;               // channel tiles per workgroup
  static constexpr int UPS = PipeTraits<FAM>::kUnitsPerStep;
  static constexpr int B_BYTES = NT * UPS * kUnitBytes;
  // weight scales per tile and step: WNA16 16 bf16 group scales, MXFP4 weights (W4A8, W4A4,
  // W4A8-MXFP8, W4A16-MXFP4) 64 e8m0 block scales, block-scaled FP8 the 128 x 128 block's fp32 scale four times
  static constexpr int SC_BYTES =
      FAM == FAM_WNA16 ? NT * 32
                       : ((FAM == FAM_W4A8 || FAM == FAM_MXW4A16 || FAM == FAM_W4A4 || FAM == FAM_W4A8MX) ? NT * 64 : (FAM == FAM_FP8B ? NT * 16 : 0));
  static constexpr int Z_BYTES = FAM == FAM_WNA16 ? NT * 8 : 0;
  // activation scales per row and step: block-scaled FP8 the fp32 scale of the row's 128-k block,
  // MX activations (W4A4, W4A8-MXFP8) the four e8m0 scales of its 32-k blocks
  static constexpr int ASC_BYTES = (FAM == FAM_FP8B || FAM == FAM_W4A4 || FAM == FAM_W4A8MX) ? BM * 4 : 0;
  static constexpr int ASC_ROWS = ASC_BYTES ? BM / kWaves : 0;   // rows whose scales a wave copies
  // scales @0, zeros or activation scales @1024
  static constexpr int META_BYTES = (SC_BYTES || Z_BYTES || ASC_BYTES) ? 2048 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + META_BYTES;
  static constexpr int LDS = STAGES * STAGE;
  // wave-wide 16-byte loads per stage, per wave
  static constexpr int A_INSTR = A_BYTES / 1024 / kWaves;
  static constexpr int B_INSTR = (NT * UPS) / kWaves;
  static constexpr int META_INSTR = (SC_BYTES ? 1 : 0) + (Z_BYTES ? 1 : 0) + (ASC_BYTES ? 1 : 0);
  static constexpr int INSTR = A_INSTR + B_INSTR + META_INSTR;
  // the copies split evenly over the waves (shapes that do not are never launched)
  static constexpr bool kValid = A_BYTES % (1024 * kWaves) == 0 && (NT * UPS) % kWaves == 0 &&
                                 (ASC_BYTES == 0 || BM % kWaves == 0);
  static constexpr int LDS_OR_NONE = kValid ? LDS : 1 << 30;
  static_assert(SC_BYTES <= 1024 && Z_BYTES <= 256, "metadata fits one masked load");
  static_assert(ASC_BYTES <= 1024 && ASC_ROWS <= 64, "activation scales: one masked load per wave");
  // block-scaled FP8: a wave's NTW tiles lie in one 128-channel scale block
  static_assert(FAM != FAM_FP8B || 8 % NTW == 0, "a wave's tiles share one weight scale block");
};

template <int FAM, int MW, int NTW, int WM, int WN, int STAGES, bool MOE>
__global__ __launch_bounds__(64 * WM * WN) void pipe_gemm_kernel(KParams p, int tiles_m, int tiles_n) {
  using Sh = PipeShape<FAM, MW, NTW, WM, WN, STAGES, MOE>;
  static_assert(Sh::kValid, "copies must split over the waves");
  using Acc = typename AccType<FAM>::type;
  constexpr int BM = Sh::BM, RB = Sh::RB, CPR = Sh::CPR, NT = Sh::NT, UPS = Sh::UPS;
  extern __shared__ __align__(1024) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  int mt, ntile, row0;
  const uint8_t* w = p.w;
  if constexpr (MOE) {
    mt = blockIdx.y;
    ntile = blockIdx.x;
    row0 = mt * BM;
    if (row0 >= *p.num_padded) return;
    const int expert = p.block_expert[mt];
    if (expert < 0 || expert >= p.E) return;   // a block past the sorted rows
    w += size_t(expert) * p.expert_stride;
  } else {
    const int nwg = gridDim.x;
    const int pid = blockIdx.x;
    const int lid = (nwg % 8 == 0) ? (pid % 8) * (nwg / 8) + pid / 8 : pid;
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = lid / per_group;
    const int first_m = group * GM;
    const int gm = min(GM, tiles_m - first_m);
    const int in_group = lid % per_group;
    mt = first_m + in_group % gm;
    ntile = in_group / gm;
    row0 = mt * BM;
  }
  const int nt_wg = ntile * NT;                    // first channel tile of the workgroup
  const int nt0 = nt_wg + wn * NTW;                // first channel tile of this wave

  // ---- per-thread sources of the stage loads (constant over K) ----
  // Activation: load j of this wave covers stage chunk positions q = (wave*A_INSTR + j)*64 + lane.
  uint32_t a_off[Sh::A_INSTR];
#pragma unroll
  for (int j = 0; j < Sh::A_INSTR; ++j) {
    const int q = (wave * Sh::A_INSTR + j) * 64 + lane;
    const int r = q / CPR;
    const int c = lds_chunk_swizzle(r, q % CPR, CPR);
    int src_row;
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      src_row = id < p.M ? id / p.topk : 0;        // padding rows read token 0, never stored
    } else {
      src_row = min(row0 + r, p.M - 1);            // rows past M are computed, never stored
    }
    a_off[j] = uint32_t(src_row) * uint32_t(p.K / 128 * RB) + uint32_t(c * 16);
  }
  // Block-scaled FP8: lane i < ASC_ROWS of wave w copies the step's fp32 scale of row
  // w * ASC_ROWS + i (MoE: of the row's token; rows past M and padding rows read a valid row's
  // and are never stored).
  const uint8_t* asc_src = nullptr;
  if constexpr (Sh::ASC_BYTES > 0) {
    const int r = wave * Sh::ASC_ROWS + min(lane, Sh::ASC_ROWS - 1);
    int src_row;
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      src_row = id < p.M ? id / p.topk : 0;
    } else {
      src_row = min(row0 + r, p.M - 1);
    }
    asc_src = reinterpret_cast<const uint8_t*>(p.a_scale) + size_t(src_row) * (p.K / 32);
  }

  auto issue_stage = [&](int ks) {
    uint8_t* st = smem + (ks % STAGES) * Sh::STAGE;
#pragma unroll
    for (int j = 0; j < Sh::A_INSTR; ++j)
      lds_dma16(p.a + a_off[j] + size_t(ks) * RB, st + (wave * Sh::A_INSTR + j) * 1024);
    uint8_t* sb = st + Sh::A_BYTES;
#pragma unroll
    for (int j = 0; j < Sh::B_INSTR; ++j) {
      const int u = wave * Sh::B_INSTR + j;        // unit index within the stage: tile u/UPS
      const size_t unit = size_t(nt_wg + u / UPS) * p.k_units + size_t(ks) * UPS + (u % UPS);
      lds_dma16(w + unit * kUnitBytes + 16 * lane, sb + u * 1024);
    }
    uint8_t* sm = sb + Sh::B_BYTES;
    // Metadata: only the lanes that carry bytes run the load (a direct-to-LDS load writes lane
    // i's bytes at base + size*i, so idle lanes must not execute it). Each load instruction still
    // counts once in this wave's vmcnt whatever its mask.
    if constexpr (FAM == FAM_WNA16) {
      // scales: NT tiles x 32 bytes = 2 lanes x 16 per tile; zeros: NT x 8 bytes = 2 lanes x 4
      const int t = lane >> 1;
      const size_t unit = size_t(nt_wg + min(t, NT - 1)) * p.k_units + ks;
      if (lane < 2 * NT) lds_dma16(w + p.scales_off + unit * 32 + 16 * (lane & 1), sm);
      const uint8_t* zsrc = p.asym ? w + p.zeros_off + unit * 8 + 4 * (lane & 1)
                                   : w + p.scales_off + unit * 32;   // unused for symmetric weights
      if (lane < 2 * NT) lds_dma4(zsrc, sm + 1024);
    } else if constexpr (FAM == FAM_W4A8 || FAM == FAM_MXW4A16 || FAM == FAM_W4A4 || FAM == FAM_W4A8MX) {
      const int t = lane >> 2;
      const size_t unit = size_t(nt_wg + min(t, NT - 1)) * p.k_units + ks;
      if (lane < 4 * NT) lds_dma16(w + p.scales_off + unit * 64 + 16 * (lane & 3), sm);
      if constexpr (Sh::ASC_BYTES > 0) {   // MX activations: this wave's rows' e8m0 scales
        if (lane < Sh::ASC_ROWS) lds_dma4(asc_src + 4 * ks, sm + 1024 + wave * Sh::ASC_ROWS * 4);
      }
    } else if constexpr (FAM == FAM_FP8B) {
      // weight scales: lane t < NT copies tile t's 16-byte granule of the step (two 64-k units
      // per step, one granule per step); activation scales: this wave's rows
      const size_t unit = size_t(nt_wg + min(lane, NT - 1)) * (p.k_units / UPS) + ks;
      if (lane < NT) lds_dma16(w + p.scales_off + unit * 16, sm);
      if (lane < Sh::ASC_ROWS) lds_dma4(asc_src + 4 * ks, sm + 1024 + wave * Sh::ASC_ROWS * 4);
    }
  };

  auto read_a = [&](const uint8_t* st, int mb, int chunk) -> u32x4 {
    const int r = wm * 16 * MW + 16 * mb + (lane & 15);
    return *reinterpret_cast<const u32x4*>(st + r * RB + (lds_chunk_swizzle(r, chunk, CPR) * 16));
  };
  auto read_b = [&](const uint8_t* st, int t, int q) -> u32x4 {
    const int u = (wn * NTW + t) * UPS + q;
    return *reinterpret_cast<const u32x4*>(st + Sh::A_BYTES + u * 1024 + 16 * lane);
  };

  Acc acc[MW][NTW];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mb][t] = Acc{0, 0, 0, 0};

  const int nks = p.K / 128;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nks) issue_stage(s);

  for (int ks = 0; ks < nks; ++ks) {
    // Own loads of step ks are done once at most (STAGES - 2) newer stages are outstanding.
    const int newer = min(STAGES - 2, nks - 1 - ks);
    if (newer >= 2) wait_vmcnt<2 * Sh::INSTR>();
    else if (newer == 1) wait_vmcnt<Sh::INSTR>();
    else wait_vmcnt<0>();
    wait_lgkm0();  // this wave's LDS reads of the old slot are done
    block_barrier();
    if (ks + STAGES - 1 < nks) issue_stage(ks + STAGES - 1);
    const uint8_t* st = smem + (ks % STAGES) * Sh::STAGE;
    const uint8_t* sm = st + Sh::A_BYTES + Sh::B_BYTES;

    if constexpr (FAM == FAM_WNA16) {
      bf16x8 af[MW][4];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          af[mb][d] = __builtin_bit_cast(bf16x8, read_a(st, mb, 4 * (lane >> 4) + d));
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int tw = wn * NTW + t;
        // one dword holds the scales of channels 2i, 2i+1: read it whole, pick the half
        const uint32_t s2 = *reinterpret_cast<const uint32_t*>(sm + tw * 32 + 4 * ((lane & 15) >> 1));
        const float s = __uint_as_float((lane & 1) ? (s2 & 0xFFFF0000u) : (s2 << 16));
        const u32x4 bq = read_b(st, t, 0);
        bf16x8 bw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = dequant_int4x8_offset128(bq[d]);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) {
          f32x4 part = mfma_bf16(af[mb][0], bw[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int d = 1; d < 4; ++d) part = mfma_bf16(af[mb][d], bw[d], part);
          acc[mb][t] += part * s;
        }
      }
    } else if constexpr (FAM == FAM_W8A8) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 af[MW];
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) af[mb] = read_a(st, mb, 4 * q + (lane >> 4));
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const u32x4 bq = read_b(st, t, q);
#pragma unroll
          for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_i8(af[mb], bq, acc[mb][t]);
        }
      }
    } else if constexpr (FAM == FAM_MXW4A16) {
      // the lane's 32 weights of a tile share k block (lane >> 4): its e8m0 scale is folded into
      // the conversion to bf16, and the MFMAs accumulate straight into the tile
      bf16x8 af[MW][4];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          af[mb][d] = __builtin_bit_cast(bf16x8, read_a(st, mb, 4 * (lane >> 4) + d));
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float sc = e8m0_to_f32(sm[(wn * NTW + t) * 64 + lane]);
        const u32x4 bq = read_b(st, t, 0);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_fp4x8_scaled(bq[d], sc);
#pragma unroll
          for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_bf16(af[mb][d], bv, acc[mb][t]);
        }
      }
    } else if constexpr (FAM == FAM_W8A16 || FAM == FAM_F8A16) {
      // 8-bit codes of the step's two units -> bf16, MFMA d taking unit d >> 1; the per-channel
      // scale is applied in the epilogue
      bf16x8 af[MW][4];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          af[mb][d] = __builtin_bit_cast(bf16x8, read_a(st, mb, 4 * (lane >> 4) + d));
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const u32x4 b0 = read_b(st, t, 0), b1 = read_b(st, t, 1);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_w8_step<FAM == FAM_F8A16>(b0, b1, d);
#pragma unroll
          for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_bf16(af[mb][d], bv, acc[mb][t]);
        }
      }
    } else if constexpr (FAM == FAM_FP8B) {
      // One 128-k step is one scale block: each tile's fp8 partial of the step, times (row
      // scale x the wave's weight block scale), is added to the tile in fp32. The row scale is
      // per output row (rows 4 (lane >> 4) + i of each 16-row block).
      const float* sa = reinterpret_cast<const float*>(sm + 1024);
      const float sw = *reinterpret_cast<const float*>(sm + wn * NTW * 16);
      u32x4 alo[MW], ahi[MW];
      float c[MW][4];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        alo[mb] = read_a(st, mb, lane >> 4);
        ahi[mb] = read_a(st, mb, 4 + (lane >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) c[mb][i] = sa[wm * 16 * MW + 16 * mb + 4 * (lane >> 4) + i] * sw;
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const u32x4 b0 = read_b(st, t, 0), b1 = read_b(st, t, 1);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) {
          const f32x4 part = mfma_fp8_fp8(alo[mb], ahi[mb], b0, b1, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][t][i] += part[i] * c[mb][i];
        }
      }
    } else if constexpr (FAM == FAM_W4A4) {
      // fp4 A operand: lane group g holds the row's k 32g..32g+31 (chunk g) and that block's
      // e8m0 scale; the weights' scale of the same block rides with the weights
      u32x4 av[MW];
      int sa[MW];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        av[mb] = read_a(st, mb, lane >> 4);
        sa[mb] = sm[1024 + (wm * 16 * MW + 16 * mb + (lane & 15)) * 4 + (lane >> 4)];
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int sb = sm[(wn * NTW + t) * 64 + lane];
        const u32x4 bq = read_b(st, t, 0);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_fp4_fp4(av[mb], sa[mb], bq, sb, acc[mb][t]);
      }
    } else if constexpr (FAM == FAM_W4A8MX) {
      // 8-bit A operand (chunks g and 4 + g) with the row's e8m0 scale of k block g
      u32x4 alo[MW], ahi[MW];
      int sa[MW];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        alo[mb] = read_a(st, mb, lane >> 4);
        ahi[mb] = read_a(st, mb, 4 + (lane >> 4));
        sa[mb] = sm[1024 + (wm * 16 * MW + 16 * mb + (lane & 15)) * 4 + (lane >> 4)];
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int sb = sm[(wn * NTW + t) * 64 + lane];
        const u32x4 bq = read_b(st, t, 0);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_fp8_fp4(alo[mb], ahi[mb], bq, sb, acc[mb][t], sa[mb]);
      }
    } else {
      u32x4 alo[MW], ahi[MW];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        alo[mb] = read_a(st, mb, lane >> 4);
        ahi[mb] = read_a(st, mb, 4 + (lane >> 4));
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int tw = wn * NTW + t;
        const int sc = sm[tw * 64 + lane];
        const u32x4 bq = read_b(st, t, 0);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_fp8_fp4(alo[mb], ahi[mb], bq, sc, acc[mb][t]);
      }
    }
  }

  const int row_base = row0 + wm * 16 * MW;
  if constexpr (FAM == FAM_WNA16) wna16_offset_contraction<MW, NTW, MOE>(p, w, acc, row_base, nt0, lane);
  store_tile<FAM, MOE, MW, NTW>(p, w, acc, row_base, nt0, lane);
}

}  // namespace

static constexpr PipeCfg kPipe[] = {
    {4, 4, 2, 2, 3},  // 0: 128 x 128, 4 waves of 64 x 64, 3 stages
    {4, 4, 2, 2, 4},  // 1: as 0, 4 stages (8-bit activations)
    {2, 4, 2, 2, 4},  // 2: 64 x 128
    {2, 2, 2, 2, 4},  // 3: 64 x 64 (MoE blocks of 64)
    {8, 4, 2, 2, 2},  // 4: 256 x 128, 4 waves of 128 x 64, 2 stages
    {8, 4, 2, 2, 3},  // 5: as 4, 3 stages (8-bit activations)
    {4, 8, 2, 2, 3},  // 6: 128 x 256, 4 waves of 64 x 128
    {4, 4, 4, 2, 2},  // 7: 256 x 128, 8 waves of 64 x 64, 2 stages
    {8, 4, 2, 4, 2},  // 8: 256 x 256, 8 waves of 128 x 64, 2 stages
    {8, 4, 2, 4, 3},  // 9: as 8, 3 stages (fp4 weights)
    {4, 4, 4, 2, 3},  // 10: as 7, 3 stages (8-bit activations)
    {4, 8, 4, 2, 2},  // 11: 256 x 256, 8 waves of 64 x 128
    {4, 4, 2, 4, 2},  // 12: 128 x 256, 8 waves of 64 x 64, 2 stages
    {4, 4, 2, 4, 3},  // 13: as 12, 3 stages
    {2, 8, 4, 2, 3},  // 14: 128 x 256, 8 waves of 32 x 128, 3 stages
    {4, 2, 1, 4, 4},  // 15: 64 x 128, 4 waves of 64 x 32 (every wave on all rows), 4 stages
};

const PipeCfg* pipe_configs(int* count) {
  *count = int(sizeof(kPipe) / sizeof(kPipe[0]));
  return kPipe;
}

template <int FAM, int I>
constexpr int pipe_lds_of() {
  return PipeShape<FAM, kPipe[I].mw, kPipe[I].ntw, kPipe[I].wm, kPipe[I].wn, kPipe[I].stages, false>::LDS_OR_NONE;
}

template <int FAM, int... I>
int pipe_lds_table(int cfg, std::integer_sequence<int, I...>) {
  static const int t[] = {pipe_lds_of<FAM, I>()...};
  return t[cfg];
}

int pipe_lds_bytes(int fam, int cfg) {
  constexpr int n = int(sizeof(kPipe) / sizeof(kPipe[0]));
  if (cfg < 0 || cfg >= n) return 1 << 30;
  auto seq = std::make_integer_sequence<int, n>{};
  if (fam == FAM_WNA16) return pipe_lds_table<FAM_WNA16>(cfg, seq);
  if (fam == FAM_W8A8) return pipe_lds_table<FAM_W8A8>(cfg, seq);
  if (fam == FAM_W4A8) return pipe_lds_table<FAM_W4A8>(cfg, seq);
  if (fam == FAM_FP8B) return pipe_lds_table<FAM_FP8B>(cfg, seq);
  if (fam == FAM_MXW4A16) return pipe_lds_table<FAM_MXW4A16>(cfg, seq);
  if (fam == FAM_W4A4) return pipe_lds_table<FAM_W4A4>(cfg, seq);
  if (fam == FAM_W4A8MX) return pipe_lds_table<FAM_W4A8MX>(cfg, seq);
  if (fam == FAM_W8A16) return pipe_lds_table<FAM_W8A16>(cfg, seq);
  if (fam == FAM_F8A16) return pipe_lds_table<FAM_F8A16>(cfg, seq);
  return 1 << 30;   // no instantiation for the other families
}

template <int FAM, bool MOE, int I>
static hipError_t launch_pipe_one(const KParams& p, dim3 grid, int tiles_m, int tiles_n, hipStream_t s) {
  constexpr PipeCfg C = kPipe[I];
  using Sh = PipeShape<FAM, C.mw, C.ntw, C.wm, C.wn, C.stages, MOE>;
  if constexpr (Sh::kValid && Sh::LDS <= 160 * 1024) {
    auto kern = pipe_gemm_kernel<FAM, C.mw, C.ntw, C.wm, C.wn, C.stages, MOE>;
    if (Sh::LDS > 65536)
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    hipLaunchKernelGGL(kern, grid, dim3(Sh::kThreads), Sh::LDS, s, p, tiles_m, tiles_n);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int FAM, bool MOE, int... I>
static hipError_t launch_pipe_fam(const KParams& p, int cfg, dim3 grid, int tiles_m, int tiles_n,
                                  hipStream_t s, std::integer_sequence<int, I...>) {
  using Fn = hipError_t (*)(const KParams&, dim3, int, int, hipStream_t);
  static const Fn table[] = {&launch_pipe_one<FAM, MOE, I>...};
  return table[cfg](p, grid, tiles_m, tiles_n, s);
}

hipError_t launch_pipe(const KParams& p, int fam, bool moe, int cfg, dim3 grid, int tiles_m,
                       int tiles_n, hipStream_t s) {
  constexpr int n = int(sizeof(kPipe) / sizeof(kPipe[0]));
  if (cfg < 0 || cfg >= n) return hipErrorInvalidValue;
  auto seq = std::make_integer_sequence<int, n>{};
  if (fam == FAM_WNA16) return moe ? launch_pipe_fam<FAM_WNA16, true>(p, cfg, grid, tiles_m, tiles_n, s, seq)
                                   : launch_pipe_fam<FAM_WNA16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_FP8B && moe) return launch_pipe_fam<FAM_FP8B, true>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (moe) return hipErrorInvalidValue;
  if (fam == FAM_W8A8) return launch_pipe_fam<FAM_W8A8, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W4A8) return launch_pipe_fam<FAM_W4A8, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_FP8B) return launch_pipe_fam<FAM_FP8B, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_MXW4A16) return launch_pipe_fam<FAM_MXW4A16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W4A4) return launch_pipe_fam<FAM_W4A4, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W4A8MX) return launch_pipe_fam<FAM_W4A8MX, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_W8A16) return launch_pipe_fam<FAM_W8A16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  if (fam == FAM_F8A16) return launch_pipe_fam<FAM_F8A16, false>(p, cfg, grid, tiles_m, tiles_n, s, seq);
  return hipErrorInvalidValue;
}

}  // namespace hq
