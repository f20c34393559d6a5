// gemm_skinny.hip -- the small-M ("decode") fused-dequantization GEMM for gfx950.
//
// At small M the time is the stream of packed weights from HBM (the Humming announcement,
// section "Tuning and JIT compilation per workload", picks a different pipeline per input-size
// range; at small batch the winner is the one that keeps many asynchronous loads in flight).
// Here a workgroup owns NTW channel tiles (16 channels each) and one block of 16*MB rows, and
// its NW waves split the K units between them. Per unit a wave
//   - loads the packed weights of its NTW tiles with one 128-bit load per lane (registers;
//     every weight byte is used by exactly one wave),
//   - copies the unit's activation rows and the tiles' scales (and zero points) into its own LDS
//     slot with direct-to-LDS copies: whole rows per instruction, so a copy touches the fewest
//     cache lines (the MFMA operand layout read straight from global memory would touch four
//     times as many), rows XOR-swizzled for conflict-free operand reads,
//   - dequantizes in registers and feeds the MFMA.
// Units go in batches of UNR; with PP two batch buffers alternate so the next batch is in
// flight while the current one is computed. The waves' partial tiles are summed through LDS in a
// fixed order, so the result is deterministic. Optionally the K units are also split across
// workgroups (grid.z); then fp32/int32 partials go to the workspace and a second kernel sums
// them in split order and applies the epilogue.
#include <hip/hip_runtime.h>

#include <utility>

#include "device_ops.h"
#include "gemm_common.h"
#include "internal.h"

namespace hq {

namespace {

template <int FAM>
struct SkTraits;
// kRowBytes: activation bytes per row per unit of kUnitK k; kAScaleBytes: activation block-scale
// bytes per row per unit (MXFP4 activations: one e8m0 byte per 32 k; block-scaled FP8: one fp32);
// kWLoads: 1 KB weight units per kernel unit (8-bit weights other than W8A8's: two 64-k units per
// 128-k step).
template <int FAM>
struct SkWLoads {
  static constexpr int value = (FAM == FAM_FP8B || FAM == FAM_W8A16 || FAM == FAM_F8A16) ? 2 : 1;
};
template <>
struct SkTraits<FAM_WNA16> {
  static constexpr int kRowBytes = 256, kUnitK = 128, kScaleBytes = 32, kZeroBytes = 8, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_WNA3> {
  static constexpr int kRowBytes = 256, kUnitK = 128, kScaleBytes = 32, kZeroBytes = 8, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_WNA2> {
  static constexpr int kRowBytes = 256, kUnitK = 128, kScaleBytes = 32, kZeroBytes = 8, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_W8A8> {
  static constexpr int kRowBytes = 64, kUnitK = 64, kScaleBytes = 0, kZeroBytes = 0, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_FP8B> {
  static constexpr int kRowBytes = 128, kUnitK = 128, kScaleBytes = 16, kZeroBytes = 0, kAScaleBytes = 4;
};
template <>
struct SkTraits<FAM_W4A8> {
  static constexpr int kRowBytes = 128, kUnitK = 128, kScaleBytes = 64, kZeroBytes = 0, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_MXW4A16> {
  static constexpr int kRowBytes = 256, kUnitK = 128, kScaleBytes = 64, kZeroBytes = 0, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_W8A16> {
  static constexpr int kRowBytes = 256, kUnitK = 128, kScaleBytes = 0, kZeroBytes = 0, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_F8A16> {
  static constexpr int kRowBytes = 256, kUnitK = 128, kScaleBytes = 0, kZeroBytes = 0, kAScaleBytes = 0;
};
template <>
struct SkTraits<FAM_W4A8MX> {
  static constexpr int kRowBytes = 128, kUnitK = 128, kScaleBytes = 64, kZeroBytes = 0, kAScaleBytes = 4;
};
template <>
struct SkTraits<FAM_W4A4> {
  static constexpr int kRowBytes = 64, kUnitK = 128, kScaleBytes = 64, kZeroBytes = 0, kAScaleBytes = 4;
};

template <int FAM, int MB, int NTW, int NW, int UNR, bool PP, bool FEW = false>
struct SkShape {
  using T = SkTraits<FAM>;
  static constexpr int ROWB = T::kRowBytes;              // activation bytes per row per unit
  static constexpr int CPR = ROWB / 16;
  // FEW: the rows one 1 KiB copy holds (4 .. 16) are the live ones
  static constexpr int LIVE = FEW ? (1024 / ROWB < 16 ? 1024 / ROWB : 16) : 16 * MB;
  static constexpr int A_UNIT = LIVE * ROWB;
  static constexpr int A_INSTR = A_UNIT / 1024;         // copies of a unit's activation rows
  static constexpr int SC = NTW * T::kScaleBytes;       // per unit, all tiles
  static constexpr int ZB = NTW * T::kZeroBytes;
  static constexpr int ASC = 16 * MB * T::kAScaleBytes;   // activation block scales per unit
  static constexpr int META_INSTR = (SC ? 1 : 0) + (ZB ? 1 : 0) + (ASC ? 1 : 0);
  static constexpr int UNIT_LDS = (A_UNIT + SC + ZB + ASC + 15) / 16 * 16;
  static constexpr int NBUF = PP ? 2 : 1;
  static constexpr int WAVE_LDS = NBUF * UNR * UNIT_LDS;
  static constexpr int RED = NW * MB * NTW * 4 * 64 * 4; // epilogue reduction (aliases the slots)
  static constexpr int LDS = (NW * WAVE_LDS > RED ? NW * WAVE_LDS : RED);
  static constexpr int WL = SkWLoads<FAM>::value;
  static constexpr int WI = FAM == FAM_WNA3 ? 2 : WL;   // weight loads per tile and unit
  static constexpr int UNIT_INSTR = A_INSTR + NTW * WI + META_INSTR;   // vector-memory ops per unit
  static_assert(A_UNIT % 1024 == 0, "whole-wave activation copies");
  static_assert(SC / 16 <= 64 && ZB / 4 <= 64 && ASC / 4 <= 64, "metadata copies fit one instruction each");
  static_assert(UNR * UNIT_INSTR < 64, "vmcnt range");
  static_assert(!FEW || (MB == 1 && LIVE >= kFewRows), "few-row form: one 16-row block");
};

template <int FAM, int MB, int NTW, int NW, int UNR, bool PP, bool MOE, bool FEW, bool SK = false>
__global__ __launch_bounds__(NW * 64) void skinny_gemm_kernel(KParams p) {
  using Sh = SkShape<FAM, MB, NTW, NW, UNR, PP, FEW>;
  using Acc = typename AccType<FAM>::type;
  using Elem = typename AccType<FAM>::elem;
  using T = SkTraits<FAM>;
  constexpr int ROWB = Sh::ROWB, CPR = Sh::CPR;
  extern __shared__ __align__(16) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int nt0 = SK ? 0 : blockIdx.x * NTW;   // Stream-K: the tile group of the current segment
  const int rb = SK ? 0 : blockIdx.y;
  const int row0 = rb * 16 * MB;

  const uint8_t* w = p.w;
  if constexpr (MOE) {
    if (row0 >= *p.num_padded) return;
    const int expert = p.block_expert[rb];
    if (expert < 0 || expert >= p.E) return;   // a block past the sorted rows
    w += size_t(expert) * p.expert_stride;
  }

  // Activation copy sources: copy j of a unit moves LDS positions q = 64 j + lane of the unit's
  // [16*MB rows][CPR chunks] block; position (r, slot) holds source chunk swizzle(r, slot). Rows
  // past M (MoE: padding) read a valid row and are never stored, so every lane copies.
  const uint8_t* asrc[Sh::A_INSTR];
  const size_t a_row_bytes = size_t(p.K) / T::kUnitK * ROWB;
#pragma unroll
  for (int j = 0; j < Sh::A_INSTR; ++j) {
    const int q = 64 * j + lane;
    const int r = q / CPR;
    const int c = lds_chunk_swizzle(r, q % CPR, CPR);
    int src_row;
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      src_row = id < p.M ? id / p.topk : 0;
    } else {
      src_row = min(row0 + r, p.M - 1);
    }
    asrc[j] = p.a + size_t(src_row) * a_row_bytes + 16 * c;
  }
  // Activation block scales (MXFP4 / MXFP8: 4 e8m0 bytes per unit; block-scaled FP8: one fp32):
  // lane r < 16*MB copies those of row r for each unit (MoE: of the row's token)
  const uint8_t* ascale_src = nullptr;
  if constexpr (Sh::ASC > 0) {
    const int r = min(lane, 16 * MB - 1);
    int src_row;
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      src_row = id < p.M ? id / p.topk : 0;
    } else {
      src_row = min(row0 + r, p.M - 1);
    }
    ascale_src = reinterpret_cast<const uint8_t*>(p.a_scale) + size_t(src_row) * (p.K / 32);
  }

  // Stream-K (one row block): the (tile group, K unit) items, tile groups outermost, are cut into
  // gridDim.x equal contiguous ranges, one per workgroup, so every workgroup streams the same
  // number of weight units. A range covers whole tile groups and at most two partial ones; each
  // piece of a group is a segment. A whole group is stored directly; the pieces of a split group
  // leave fp32 (int32) partial tiles in the workspace, and the workgroup that contributes last
  // (an arrival counter per group) sums them in piece order and stores the result, then sets the
  // counter back to zero for the next call. No workgroup waits for another, and no fence writes
  // back or invalidates a whole cache: the partial tiles and the counters are accessed at device
  // scope, item by item.
  const int k_units = p.k_units / Sh::WL;             // kernel units (steps of kUnitK k)
  long long sk_item = 0, sk_end = 0;
  if constexpr (SK) {
    sk_item = (long long)blockIdx.x * p.sk_items / gridDim.x;
    sk_end = (long long)(blockIdx.x + 1) * p.sk_items / gridDim.x;
  }
  for (;;) {
  int ubeg, uend, sk_g = 0;
  if constexpr (SK) {
    if (sk_item >= sk_end) break;
    sk_g = int(sk_item / k_units);
    ubeg = int(sk_item - (long long)sk_g * k_units);
    uend = int(sk_end - (long long)sk_g * k_units < k_units ? sk_end - (long long)sk_g * k_units : k_units);
    sk_item += uend - ubeg;
    nt0 = sk_g * NTW;
    __syncthreads();   // the previous segment's reads of the reduction buffer are done
  } else {
    ubeg = blockIdx.z * p.units_per_split;
    uend = min(k_units, ubeg + p.units_per_split);
  }

  Acc acc[MB][NTW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mb][t] = Acc{0, 0, 0, 0};

  uint8_t* wlds = smem + wave * Sh::WAVE_LDS;
  u32x4 bw[Sh::NBUF][UNR][NTW];   // packed weights of the batches in flight
  u32x4 bw2[Sh::NBUF][UNR][Sh::WL == 2 ? NTW : 1];   // block-scaled FP8: the step's second unit

  // Issue every copy and load of unit u into slot (buf, r).
  auto issue_unit = [&](int buf, int r, int u) __attribute__((always_inline)) {
    uint8_t* slot = wlds + (buf * UNR + r) * Sh::UNIT_LDS;
#pragma unroll
    for (int j = 0; j < Sh::A_INSTR; ++j) lds_dma16(asrc[j] + size_t(u) * ROWB, slot + 1024 * j);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const size_t unit = (size_t(nt0 + t) * k_units + u) * Sh::WL;
      if constexpr (FAM == FAM_WNA2) {
        bw[buf][r][t] = ldg8_stream(w + unit * 512 + 8 * lane);
      } else if constexpr (FAM == FAM_WNA3) {
        bw[buf][r][t] = ldg8_stream(w + unit * 768 + 8 * lane);
        bw[buf][r][t][2] = ldg4_stream(w + unit * 768 + 512 + 4 * lane);
      } else {
        bw[buf][r][t] = ldg16_stream(w + unit * kUnitBytes + 16 * lane);
      }
      if constexpr (Sh::WL == 2) bw2[buf][r][t] = ldg16_stream(w + (unit + 1) * kUnitBytes + 16 * lane);
    }
    if constexpr (Sh::SC > 0) {
      // the NTW tiles' scale blocks of this unit, T::kScaleBytes each, 16 bytes per lane
      constexpr int per_tile = T::kScaleBytes / 16;
      const int t = min(lane / per_tile, NTW - 1);
      const size_t unit = size_t(nt0 + t) * k_units + u;
      if (lane < Sh::SC / 16)
        lds_dma16(w + p.scales_off + unit * T::kScaleBytes + 16 * (lane % per_tile), slot + Sh::A_UNIT);
    }
    if constexpr (Sh::ZB > 0) {
      // zero points (8 bytes per tile), 4 bytes per lane; symmetric weights have none and copy
      // scale bytes instead, which are never read
      const int t = min(lane >> 1, NTW - 1);
      const size_t unit = size_t(nt0 + t) * k_units + u;
      const uint8_t* src = p.asym ? w + p.zeros_off + unit * 8 + 4 * (lane & 1)
                                  : w + p.scales_off + unit * T::kScaleBytes;
      if (lane < Sh::ZB / 4) lds_dma4(src, slot + Sh::A_UNIT + Sh::SC);
    }
    if constexpr (Sh::ASC > 0) {
      if (lane < 16 * MB) lds_dma4(ascale_src + 4 * u, slot + Sh::A_UNIT + Sh::SC + Sh::ZB);
    }
  };

  // Operand reads from the slot and the MFMAs of one unit.
  auto compute_unit = [&](int buf, int r) __attribute__((always_inline)) {
    const uint8_t* slot = wlds + (buf * UNR + r) * Sh::UNIT_LDS;
    auto read_a = [&](int mb, int chunk) __attribute__((always_inline)) -> u32x4 {
      const int row = FEW ? (lane & (Sh::LIVE - 1)) : 16 * mb + (lane & 15);
      return *reinterpret_cast<const u32x4*>(slot + row * ROWB + 16 * lds_chunk_swizzle(row, chunk, CPR));
    };
    if constexpr (family_int_groups(FAM)) {
      // The group's partial sum_k x*(u - z) is formed as sum_k x*(128 + u) (the offset-128
      // operand costs one bit-select per weight pair) minus (128 + z) * sum_k x; the row sums
      // come from one MFMA against an all-ones operand, shared by the NTW tiles.
      u32x4 af[MB][4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d) af[mb][d] = read_a(mb, 4 * (lane >> 4) + d);
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      f32x4 rsum[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        rsum[mb] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][0]), ones, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int d = 1; d < 4; ++d) rsum[mb] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), ones, rsum[mb]);
      }
      const uint8_t* sc = slot + Sh::A_UNIT;
      const uint8_t* zp = sc + Sh::SC;
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float s = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sc + t * 32 + 2 * (lane & 15)));
        uint32_t z = 8;
        if (p.asym) {
          const uint32_t zb = zp[t * 8 + ((lane & 15) >> 1)];
          z = (lane & 1) ? (zb >> 4) : (zb & 0xFu);
        }
        const float c = -s * float(128u + z);
        f32x4 part[MB];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_offset128<FAM>(bw[buf][r][t], d);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            part[mb] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), bv,
                                 d == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][t] += part[mb] * s + rsum[mb] * c;
      }
    } else if constexpr (FAM == FAM_MXW4A16) {
      // bf16 activations in the WNA16 chunk order; the lane's 32 weights all belong to k block
      // (lane >> 4) of the unit, so one scale per lane and tile is folded into the conversion
      u32x4 af[MB][4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d) af[mb][d] = read_a(mb, 4 * (lane >> 4) + d);
      const uint8_t* sc = slot + Sh::A_UNIT;
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float s = e8m0_to_f32(sc[t * 64 + lane]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_fp4x8_scaled(bw[buf][r][t][d], s);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][t] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), bv, acc[mb][t]);
        }
      }
    } else if constexpr (FAM == FAM_W8A16 || FAM == FAM_F8A16) {
      // bf16 activations in the WNA16 chunk order; the step's two weight units hold the lane
      // group's 32 k, MFMA d taking 8 of them from unit d >> 1. The per-channel scale is applied
      // in the epilogue.
      u32x4 af[MB][4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d) af[mb][d] = read_a(mb, 4 * (lane >> 4) + d);
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 bv = dequant_w8_step<FAM == FAM_F8A16>(bw[buf][r][t], bw2[buf][r][Sh::WL == 2 ? t : 0], d);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][t] = mfma_bf16(__builtin_bit_cast(bf16x8, af[mb][d]), bv, acc[mb][t]);
        }
    } else if constexpr (FAM == FAM_FP8B) {
      // one 128-k step = one scale block: the fp8 MFMA's partial, times (row scale x block
      // scale), into the tile; the row scale is per output row (D rows 4 (lane >> 4) + i)
      const uint8_t* sc = slot + Sh::A_UNIT;
      const float* asc = reinterpret_cast<const float*>(sc + Sh::SC + Sh::ZB);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 alo = read_a(mb, lane >> 4);
        const u32x4 ahi = read_a(mb, 4 + (lane >> 4));
        float sa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = asc[16 * mb + 4 * (lane >> 4) + i];
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const float sw = *reinterpret_cast<const float*>(sc + t * 16);
          const f32x4 part = mfma_fp8_fp8(alo, ahi, bw[buf][r][t], bw2[buf][r][Sh::WL == 2 ? t : 0],
                                          f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][t][i] += part[i] * (sa[i] * sw);
        }
      }
    } else if constexpr (FAM == FAM_W8A8) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 av = read_a(mb, lane >> 4);
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[mb][t] = mfma_i8(av, bw[buf][r][t], acc[mb][t]);
      }
    } else if constexpr (FAM == FAM_W4A4) {
      // fp4 A operand: lane group g holds the row's k 32g..32g+31 (chunk g) and that block's
      // e8m0 scale
      const uint8_t* sc = slot + Sh::A_UNIT;
      const uint8_t* asc = sc + Sh::SC + Sh::ZB;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 av = read_a(mb, lane >> 4);
        const int sa = asc[(16 * mb + (lane & 15)) * 4 + (lane >> 4)];
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          acc[mb][t] = mfma_fp4_fp4(av, sa, bw[buf][r][t], int(sc[t * 64 + lane]), acc[mb][t]);
      }
    } else {
      // 8-bit A operand of the scaled MFMA: lane group g holds chunks g and 4 + g; the scale of
      // k block b comes from lane group b (MXFP8 activations: the row's block scale; per-token
      // FP8: 2^0, the token scale is applied in the epilogue)
      const uint8_t* sc = slot + Sh::A_UNIT;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 alo = read_a(mb, lane >> 4);
        const u32x4 ahi = read_a(mb, 4 + (lane >> 4));
        int sa = 127;
        if constexpr (Sh::ASC > 0) sa = sc[Sh::SC + Sh::ZB + (16 * mb + (lane & 15)) * 4 + (lane >> 4)];
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          acc[mb][t] = mfma_fp8_fp4(alo, ahi, bw[buf][r][t], int(sc[t * 64 + lane]), acc[mb][t], sa);
      }
    }
  };

  // This wave's units are u0, u0 + NW, ... < uend, in batches of UNR; a remainder below UNR is
  // taken one unit at a time.
  const int u0 = ubeg + wave;
  const int nunits = u0 < uend ? (uend - u0 + NW - 1) / NW : 0;
  const int nbatch = nunits / UNR;
  auto issue_batch = [&](int buf, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < UNR; ++r) issue_unit(buf, r, u0 + (b * UNR + r) * NW);
  };
  auto compute_batch = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < UNR; ++r) compute_unit(buf, r);
  };
  if constexpr (PP) {
    // Written out for both buffers so that every register index is a constant. Before a buffer
    // is refilled, the operand reads of the batch that used it last have completed.
    if (nbatch > 0) issue_batch(0, 0);
    for (int b = 0; b < nbatch; b += 2) {
      wait_lgkm0();
      if (b + 1 < nbatch) {
        issue_batch(1, b + 1);
        wait_vmcnt<UNR * Sh::UNIT_INSTR>();
      } else {
        wait_vmcnt<0>();
      }
      compute_batch(0);
      if (b + 1 < nbatch) {
        wait_lgkm0();
        if (b + 2 < nbatch) {
          issue_batch(0, b + 2);
          wait_vmcnt<UNR * Sh::UNIT_INSTR>();
        } else {
          wait_vmcnt<0>();
        }
        compute_batch(1);
      }
    }
  } else {
    for (int b = 0; b < nbatch; ++b) {
      wait_lgkm0();
      issue_batch(0, b);
      wait_vmcnt<0>();
      compute_batch(0);
    }
  }
  for (int i = nbatch * UNR; i < nunits; ++i) {
    wait_lgkm0();
    issue_unit(0, 0, u0 + i * NW);
    wait_vmcnt<0>();
    compute_unit(0, 0);
  }

  // Sum the waves' tiles through LDS (fixed order: wave 0, 1, ...), then the epilogue. The
  // reduction buffer aliases the unit slots: every wave has finished with its slot first.
  // Output rows 4 (lane >> 4) + j: in the few-row form only lane groups below LIVE / 4 hold live
  // rows.
  constexpr int kVals = MB * NTW * 4;
  Elem(*red)[kVals][64] = reinterpret_cast<Elem(*)[kVals][64]>(smem);
  __syncthreads();
  if (!FEW || (lane >> 4) < Sh::LIVE / 4) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][(mb * NTW + t) * 4 + j][lane] = acc[mb][t][j];
  }
  __syncthreads();
  static_assert(NW > 1, "the epilogue reads the waves' tiles from LDS");
  for (int v = threadIdx.x; v < kVals * 64; v += NW * 64) {
    const int le = v & 63;
    if (FEW && (le >> 4) >= Sh::LIVE / 4) continue;
    const int q = v >> 6;
    const int j = q & 3;
    const int t = (q >> 2) % NTW;
    const int mb = (q >> 2) / NTW;
    Elem sum = red[0][q][le];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww][q][le];
    const int ib = 16 * mb + 4 * (le >> 4) + j;
    const int n = (nt0 + t) * 16 + (le & 15);
    if (!SK || (ubeg == 0 && uend == k_units)) {
      store_result<FAM, MOE>(p, w, row0 + ib, n, sum, blockIdx.z);
    } else {
      // partial tile of this piece: slot = this workgroup's place among the group's contributors
      const long long first = ((long long)sk_g * k_units + 1) * gridDim.x - 1;
      const int slot = int(blockIdx.x - first / p.sk_items);
      // written at device (agent) scope: through to the point where every CU's loads see it
      __hip_atomic_store(reinterpret_cast<Elem*>(p.ws) + (size_t(sk_g) * p.sk_slots + slot) * (kVals * 64) + v,
                         sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (SK) {
    if (!(ubeg == 0 && uend == k_units)) {
      const long long gi = (long long)sk_g * k_units;
      const int w_first = int(((gi + 1) * gridDim.x - 1) / p.sk_items);
      const int w_last = int(((gi + k_units) * gridDim.x - 1) / p.sk_items);
      // Ordering without whole-cache fences: every partial store above has completed (its wait
      // count is zero) before the workgroup barrier, and the arrival is counted after the barrier;
      // the partial tiles are read back below with device-scope loads, which bypass the
      // non-coherent cache path.
      wait_vmcnt<0>();
      __syncthreads();   // every thread's partial stores are complete; the reduction buffer is free
      int* flag = reinterpret_cast<int*>(smem);
      if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(p.sk_counters + sk_g, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        *flag = int(old) + 1 == w_last - w_first + 1;
      }
      __syncthreads();
      if (*flag) {
        Elem* part = reinterpret_cast<Elem*>(p.ws) + size_t(sk_g) * p.sk_slots * (kVals * 64);
        for (int v = threadIdx.x; v < kVals * 64; v += NW * 64) {
          const int le = v & 63;
          if (FEW && (le >> 4) >= Sh::LIVE / 4) continue;
          Elem sum = __hip_atomic_load(part + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int sl = 1; sl <= w_last - w_first; ++sl)
            sum += __hip_atomic_load(part + size_t(sl) * (kVals * 64) + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int q = v >> 6;
          const int j = q & 3;
          const int t = (q >> 2) % NTW;
          const int mb = (q >> 2) / NTW;
          store_result<FAM, MOE>(p, w, row0 + 16 * mb + 4 * (le >> 4) + j, (nt0 + t) * 16 + (le & 15), sum, 0);
        }
        if (threadIdx.x == 0)   // ready for the next call
          __hip_atomic_store(p.sk_counters + sk_g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if constexpr (!SK) break;
  }   // segments
}

}  // namespace

// ---- launch table --------------------------------------------------------------------------

// Index = plan.cfg. Keep in sync with skinny_configs() below.
static constexpr SkinnyCfg kSkinny[] = {
    // mb ntw nw unr pp
    {1, 4, 8, 2, 0},   // 0: M <= 16, wide N
    {1, 2, 8, 2, 0},   // 1: M <= 16, N/16 not a multiple of 4
    {1, 1, 8, 2, 0},   // 2: M <= 16, odd channel tiles
    {2, 4, 4, 2, 0},   // 3: M <= 32
    {4, 4, 4, 1, 0},   // 4: M <= 64
    {4, 2, 4, 1, 0},   // 5: M <= 64, N/16 even only
    {4, 1, 4, 1, 0},   // 6: M <= 64, any N
    {2, 2, 4, 2, 0},   // 7: M <= 32, N/16 even only
    {2, 1, 4, 2, 0},   // 8: M <= 32, any N
    {1, 2, 8, 4, 0},   // 9: M <= 16, 4 units in flight per wave
    {1, 1, 8, 4, 0},   // 10
    {1, 1, 16, 2, 0},  // 11
    {1, 2, 16, 2, 0},  // 12
    {1, 4, 8, 1, 1},   // 13: ping-pong, one unit per buffer
    {1, 1, 4, 4, 0},   // 14
    {2, 2, 8, 2, 0},   // 15: M <= 32
    {2, 1, 8, 4, 0},   // 16
    {1, 4, 8, 2, 1},   // 17: ping-pong
    {1, 2, 8, 2, 1},   // 18
    {1, 1, 8, 2, 1},   // 19
    {1, 2, 16, 1, 1},  // 20
    {1, 1, 16, 1, 1},  // 21
    {2, 4, 4, 1, 1},   // 22: M <= 32, ping-pong
    {2, 2, 8, 1, 1},   // 23
    {1, 4, 8, 4, 0},   // 24: M <= 16, all of a wave's units in flight at once (K = 4096)
    {1, 4, 4, 4, 0},   // 25
    {1, 2, 8, 4, 1},   // 26
    {1, 4, 16, 2, 0},  // 27: M <= 16, 16 waves
    {1, 4, 16, 1, 1},  // 28
    {2, 4, 8, 2, 0},   // 29: M <= 32, 8 waves
    {1, 4, 16, 1, 1, 1},  // 30: M <= 4, the few-row forms of 28, 27, 13, 0, 20
    {1, 4, 16, 2, 0, 1},  // 31
    {1, 4, 8, 1, 1, 1},   // 32
    {1, 4, 8, 2, 0, 1},   // 33
    {1, 2, 16, 1, 1, 1},  // 34
};

const SkinnyCfg* skinny_configs(int* count) {
  *count = int(sizeof(kSkinny) / sizeof(kSkinny[0]));
  return kSkinny;
}

template <int FAM, int... I>
static int skinny_lds_table(int cfg, std::integer_sequence<int, I...>) {
  static const int t[] = {SkShape<FAM, kSkinny[I].mb, kSkinny[I].ntw, kSkinny[I].nw, kSkinny[I].unr,
                                  kSkinny[I].pp != 0, kSkinny[I].few != 0>::LDS...};
  return t[cfg];
}

int skinny_lds_bytes(int fam, int cfg) {
  constexpr int n = int(sizeof(kSkinny) / sizeof(kSkinny[0]));
  if (cfg < 0 || cfg >= n) return 1 << 30;
  auto seq = std::make_integer_sequence<int, n>{};
  if (fam == FAM_WNA16) return skinny_lds_table<FAM_WNA16>(cfg, seq);
  if (fam == FAM_WNA2) return skinny_lds_table<FAM_WNA2>(cfg, seq);
  if (fam == FAM_WNA3) return skinny_lds_table<FAM_WNA3>(cfg, seq);
  if (fam == FAM_W8A8) return skinny_lds_table<FAM_W8A8>(cfg, seq);
  if (fam == FAM_W4A4) return skinny_lds_table<FAM_W4A4>(cfg, seq);
  if (fam == FAM_W4A8MX) return skinny_lds_table<FAM_W4A8MX>(cfg, seq);
  if (fam == FAM_MXW4A16) return skinny_lds_table<FAM_MXW4A16>(cfg, seq);
  if (fam == FAM_FP8B) return skinny_lds_table<FAM_FP8B>(cfg, seq);
  if (fam == FAM_W8A16) return skinny_lds_table<FAM_W8A16>(cfg, seq);
  if (fam == FAM_F8A16) return skinny_lds_table<FAM_F8A16>(cfg, seq);
  return skinny_lds_table<FAM_W4A8>(cfg, seq);
}

template <int FAM, int MB, int NTW, int NW, int UNR, bool PP, bool MOE, bool FEW>
static hipError_t launch_skinny_one(const KParams& p, dim3 grid, hipStream_t s) {
  constexpr int lds = SkShape<FAM, MB, NTW, NW, UNR, PP, FEW>::LDS;
  if constexpr (lds > 160 * 1024 || (MOE && FEW)) {   // MoE row blocks are always whole
    return hipErrorInvalidValue;
  } else {
    if (FEW && p.M > kFewRows) return hipErrorInvalidValue;
    auto kern = skinny_gemm_kernel<FAM, MB, NTW, NW, UNR, PP, MOE, FEW>;
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, p);
    return hipGetLastError();
  }
}

template <int FAM, bool MOE>
static hipError_t launch_skinny_fam(const KParams& p, int cfg, dim3 grid, hipStream_t s) {
#define HQ_SK(I)                                                                           \
  case I:                                                                                  \
    return launch_skinny_one<FAM, kSkinny[I].mb, kSkinny[I].ntw, kSkinny[I].nw,            \
                             kSkinny[I].unr, kSkinny[I].pp != 0, MOE, kSkinny[I].few != 0>(p, grid, s);
  switch (cfg) {
    HQ_SK(0) HQ_SK(1) HQ_SK(2) HQ_SK(3) HQ_SK(4) HQ_SK(5) HQ_SK(6) HQ_SK(7) HQ_SK(8) HQ_SK(9)
    HQ_SK(10) HQ_SK(11) HQ_SK(12) HQ_SK(13) HQ_SK(14) HQ_SK(15) HQ_SK(16) HQ_SK(17) HQ_SK(18)
    HQ_SK(19) HQ_SK(20) HQ_SK(21) HQ_SK(22) HQ_SK(23) HQ_SK(24) HQ_SK(25) HQ_SK(26) HQ_SK(27) HQ_SK(28) HQ_SK(29)
    HQ_SK(30) HQ_SK(31) HQ_SK(32) HQ_SK(33) HQ_SK(34)
    default:
      return hipErrorInvalidValue;
  }
#undef HQ_SK
}

// ---- Stream-K launches (dense, one row block) ------------------------------------------------
static constexpr int kSkCfgs[] = {0, 1, 2, 11, 12, 13, 20, 21, 27, 28, 30, 31, 32, 33};

bool skinny_stream_k_cfg(int cfg) {
  for (int c : kSkCfgs)
    if (c == cfg) return true;
  return false;
}

template <int FAM, int I>
static hipError_t launch_sk_one(const KParams& p, int wgs, hipStream_t s) {
  constexpr SkinnyCfg C = kSkinny[I];
  constexpr int lds = SkShape<FAM, C.mb, C.ntw, C.nw, C.unr, C.pp != 0, C.few != 0>::LDS;
  if constexpr (lds > 160 * 1024) {
    return hipErrorInvalidValue;
  } else {
    if (C.few && p.M > kFewRows) return hipErrorInvalidValue;
    auto kern = skinny_gemm_kernel<FAM, C.mb, C.ntw, C.nw, C.unr, C.pp != 0, false, C.few != 0, true>;
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    hipLaunchKernelGGL(kern, dim3(unsigned(wgs)), dim3(C.nw * 64), lds, s, p);
    return hipGetLastError();
  }
}

template <int FAM>
static hipError_t launch_sk_fam(const KParams& p, int cfg, int wgs, hipStream_t s) {
  switch (cfg) {
    case 0: return launch_sk_one<FAM, 0>(p, wgs, s);
    case 1: return launch_sk_one<FAM, 1>(p, wgs, s);
    case 2: return launch_sk_one<FAM, 2>(p, wgs, s);
    case 11: return launch_sk_one<FAM, 11>(p, wgs, s);
    case 12: return launch_sk_one<FAM, 12>(p, wgs, s);
    case 13: return launch_sk_one<FAM, 13>(p, wgs, s);
    case 20: return launch_sk_one<FAM, 20>(p, wgs, s);
    case 21: return launch_sk_one<FAM, 21>(p, wgs, s);
    case 27: return launch_sk_one<FAM, 27>(p, wgs, s);
    case 28: return launch_sk_one<FAM, 28>(p, wgs, s);
    case 30: return launch_sk_one<FAM, 30>(p, wgs, s);
    case 31: return launch_sk_one<FAM, 31>(p, wgs, s);
    case 32: return launch_sk_one<FAM, 32>(p, wgs, s);
    case 33: return launch_sk_one<FAM, 33>(p, wgs, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_skinny_stream_k(const KParams& p, int fam, int cfg, int wgs, hipStream_t s) {
  switch (fam) {
    case FAM_WNA16: return launch_sk_fam<FAM_WNA16>(p, cfg, wgs, s);
    case FAM_WNA2: return launch_sk_fam<FAM_WNA2>(p, cfg, wgs, s);
    case FAM_WNA3: return launch_sk_fam<FAM_WNA3>(p, cfg, wgs, s);
    case FAM_MXW4A16: return launch_sk_fam<FAM_MXW4A16>(p, cfg, wgs, s);
    case FAM_W8A8: return launch_sk_fam<FAM_W8A8>(p, cfg, wgs, s);
    case FAM_W4A8: return launch_sk_fam<FAM_W4A8>(p, cfg, wgs, s);
    case FAM_W4A4: return launch_sk_fam<FAM_W4A4>(p, cfg, wgs, s);
    case FAM_W4A8MX: return launch_sk_fam<FAM_W4A8MX>(p, cfg, wgs, s);
    case FAM_FP8B: return launch_sk_fam<FAM_FP8B>(p, cfg, wgs, s);
    case FAM_W8A16: return launch_sk_fam<FAM_W8A16>(p, cfg, wgs, s);
    case FAM_F8A16: return launch_sk_fam<FAM_F8A16>(p, cfg, wgs, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_skinny(const KParams& p, int fam, bool moe, int cfg, dim3 grid,
                         hipStream_t s) {
  if (fam == FAM_WNA16) return moe ? launch_skinny_fam<FAM_WNA16, true>(p, cfg, grid, s)
                                   : launch_skinny_fam<FAM_WNA16, false>(p, cfg, grid, s);
  if (fam == FAM_WNA2) return moe ? launch_skinny_fam<FAM_WNA2, true>(p, cfg, grid, s)
                                  : launch_skinny_fam<FAM_WNA2, false>(p, cfg, grid, s);
  if (fam == FAM_WNA3) return moe ? launch_skinny_fam<FAM_WNA3, true>(p, cfg, grid, s)
                                  : launch_skinny_fam<FAM_WNA3, false>(p, cfg, grid, s);
  if (fam == FAM_MXW4A16) return moe ? launch_skinny_fam<FAM_MXW4A16, true>(p, cfg, grid, s)
                                     : launch_skinny_fam<FAM_MXW4A16, false>(p, cfg, grid, s);
  if (moe && fam == FAM_W8A8) return launch_skinny_fam<FAM_W8A8, true>(p, cfg, grid, s);
  if (moe && fam == FAM_W4A8) return launch_skinny_fam<FAM_W4A8, true>(p, cfg, grid, s);
  if (moe && fam == FAM_FP8B) return launch_skinny_fam<FAM_FP8B, true>(p, cfg, grid, s);
  if (moe && fam == FAM_W8A16) return launch_skinny_fam<FAM_W8A16, true>(p, cfg, grid, s);
  if (moe && fam == FAM_F8A16) return launch_skinny_fam<FAM_F8A16, true>(p, cfg, grid, s);
  if (moe && fam == FAM_W4A4) return launch_skinny_fam<FAM_W4A4, true>(p, cfg, grid, s);
  if (moe && fam == FAM_W4A8MX) return launch_skinny_fam<FAM_W4A8MX, true>(p, cfg, grid, s);
  if (moe) return hipErrorInvalidValue;
  if (fam == FAM_W8A8) return launch_skinny_fam<FAM_W8A8, false>(p, cfg, grid, s);
  if (fam == FAM_W4A4) return launch_skinny_fam<FAM_W4A4, false>(p, cfg, grid, s);
  if (fam == FAM_W4A8MX) return launch_skinny_fam<FAM_W4A8MX, false>(p, cfg, grid, s);
  if (fam == FAM_FP8B) return launch_skinny_fam<FAM_FP8B, false>(p, cfg, grid, s);
  if (fam == FAM_W8A16) return launch_skinny_fam<FAM_W8A16, false>(p, cfg, grid, s);
  if (fam == FAM_F8A16) return launch_skinny_fam<FAM_F8A16, false>(p, cfg, grid, s);
  return launch_skinny_fam<FAM_W4A8, false>(p, cfg, grid, s);
}

}  // namespace hq
