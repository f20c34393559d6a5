// gemm_skinny.hip -- the small-M ("decode") fused-dequantization GEMM for gfx950.
//
// At small M the time is the stream of packed weights from HBM (the Humming announcement,
// section "Tuning and JIT compilation per workload", picks a different pipeline per input-size
// range; at small batch the winner is the one that keeps many asynchronous loads in flight).
// Here a workgroup owns NTW channel tiles (16 channels each) and one block of 16*MB rows, and
// its NW waves split the K units between them: each wave streams whole 1 KiB weight units with
// one 128-bit load per lane (no LDS staging: every weight byte is used by exactly one wave),
// dequantizes them in registers and feeds the MFMA. The waves' partial tiles are summed through
// LDS in a fixed order, so the result is deterministic. Optionally the K units are also split
// across workgroups (grid.z); then fp32/int32 partials go to the workspace and a second kernel
// sums them in split order and applies the epilogue.
#include <hip/hip_runtime.h>

#include "device_ops.h"
#include "gemm_common.h"
#include "internal.h"

namespace hq {

template <int FAM, int MB, int NTW>
struct SkinnyFrag;

// WNA16: one unit = 16 channels x 128 k (one group) = 4 MFMA k-steps of 32.
template <int MB, int NTW>
struct SkinnyFrag<FAM_WNA16, MB, NTW> {
  u32x4 b[NTW];
  uint32_t s_bits[NTW];
  uint32_t zb[NTW];
  u32x4 a[MB][4];

  __device__ __forceinline__ void load(const KParams& p, const uint8_t* w, int nt0, int u,
                                       int lane, const uint8_t* const* arow) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const size_t unit = size_t(nt0 + t) * p.k_units + u;
      b[t] = ldg16_stream(w + unit * kUnitBytes + 16 * lane);
      s_bits[t] = *reinterpret_cast<const uint16_t*>(w + p.scales_off + unit * 32 + 2 * (lane & 15));
      zb[t] = p.asym ? uint32_t(w[p.zeros_off + unit * 8 + ((lane & 15) >> 1)]) : 0u;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (arow[mb]) {
        const uint8_t* src = arow[mb] + (size_t(u) * 128 + 32 * (lane >> 4)) * 2;
#pragma unroll
        for (int d = 0; d < 4; ++d) a[mb][d] = ldg16(src + 16 * d);
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) a[mb][d] = u32x4{0, 0, 0, 0};
      }
    }
  }

  // The group's partial sum_k x*(u - z) is formed on the MFMA as sum_k x*(128 + u) plus
  // sum_k x*(-(128 + z)): the first operand costs one bit-select per weight pair, the second is
  // a per-channel constant. At small M the MFMA has cycles to spare; the VALU does not.
  __device__ __forceinline__ void compute(const KParams& p, int lane, f32x4 (*acc)[NTW]) const {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const uint32_t z = p.asym ? ((lane & 1) ? (zb[t] >> 4) : (zb[t] & 0xFu)) : 8u;
      const float s = bf16_bits_to_f32(s_bits[t]);
      const bf16x8 bneg = neg_offset_bf16x8(z);
      f32x4 part[MB];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 bw = dequant_int4x8_offset128(b[t][d]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, a[mb][d]);
          part[mb] = mfma_bf16(av, bw, d == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[mb]);
          part[mb] = mfma_bf16(av, bneg, part[mb]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][t] += part[mb] * s;
    }
  }
};

// W8A8: one unit = 16 channels x 64 k = one int8 MFMA.
template <int MB, int NTW>
struct SkinnyFrag<FAM_W8A8, MB, NTW> {
  u32x4 b[NTW];
  u32x4 a[MB];

  __device__ __forceinline__ void load(const KParams& p, const uint8_t* w, int nt0, int u,
                                       int lane, const uint8_t* const* arow) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const size_t unit = size_t(nt0 + t) * p.k_units + u;
      b[t] = ldg16_stream(w + unit * kUnitBytes + 16 * lane);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      a[mb] = arow[mb] ? ldg16(arow[mb] + size_t(u) * 64 + 16 * (lane >> 4)) : u32x4{0, 0, 0, 0};
  }

  __device__ __forceinline__ void compute(const KParams&, int, i32x4 (*acc)[NTW]) const {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][t] = mfma_i8(a[mb], b[t], acc[mb][t]);
  }
};

// W4A8: one unit = 16 channels x 128 k = four MX blocks = one scaled fp8 x fp4 MFMA.
template <int MB, int NTW>
struct SkinnyFrag<FAM_W4A8, MB, NTW> {
  u32x4 b[NTW];
  uint32_t sc[NTW];
  u32x4 a[MB][2];

  __device__ __forceinline__ void load(const KParams& p, const uint8_t* w, int nt0, int u,
                                       int lane, const uint8_t* const* arow) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const size_t unit = size_t(nt0 + t) * p.k_units + u;
      b[t] = ldg16_stream(w + unit * kUnitBytes + 16 * lane);
      sc[t] = w[p.scales_off + unit * 64 + lane];
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (arow[mb]) {
        // 8-bit A operand of the scaled MFMA: lane group g holds k = 16g..16g+15 in bytes 0..15
        // and k = 64+16g..64+16g+15 in bytes 16..31.
        const uint8_t* src = arow[mb] + size_t(u) * 128 + 16 * (lane >> 4);
        a[mb][0] = ldg16(src);
        a[mb][1] = ldg16(src + 64);
      } else {
        a[mb][0] = u32x4{0, 0, 0, 0};
        a[mb][1] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ __forceinline__ void compute(const KParams&, int, f32x4 (*acc)[NTW]) const {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb][t] = mfma_fp8_fp4(a[mb][0], a[mb][1], b[t], int(sc[t]), acc[mb][t]);
  }
};

template <int FAM, int MB, int NTW, int NW, int UNR, bool PP, bool MOE>
__global__ __launch_bounds__(NW * 64) void skinny_gemm_kernel(KParams p) {
  using Acc = typename AccType<FAM>::type;
  using Elem = typename AccType<FAM>::elem;
  constexpr int ABYTES = FAM == FAM_WNA16 ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nt0 = blockIdx.x * NTW;
  const int rb = blockIdx.y;
  const int row0 = rb * 16 * MB;

  const uint8_t* w = p.w;
  if constexpr (MOE) {
    if (row0 >= *p.num_padded) return;
    w += size_t(p.block_expert[rb]) * p.expert_stride;
  }

  const uint8_t* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = row0 + 16 * mb + (lane & 15);
    if constexpr (MOE) {
      const int id = p.sorted_ids[i];
      arow[mb] = id < p.M ? p.a + size_t(id / p.topk) * p.K * ABYTES : nullptr;
    } else {
      arow[mb] = i < p.M ? p.a + size_t(i) * p.K * ABYTES : nullptr;
    }
  }

  Acc acc[MB][NTW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mb][t] = Acc{0, 0, 0, 0};

  // This wave's units are u0, u0 + NW, ... < uend, taken in batches of UNR. Two register
  // buffers alternate so that batch b+1 is in flight while batch b is dequantized and
  // multiplied (written as an explicit ping-pong: no register copies between the buffers).
  const int ubeg = blockIdx.z * p.units_per_split;
  const int uend = min(p.k_units, ubeg + p.units_per_split);
  const int u0 = ubeg + wave;
  const int nunits = u0 < uend ? (uend - u0 + NW - 1) / NW : 0;
  const int nbatch = nunits / UNR;
  using Frag = SkinnyFrag<FAM, MB, NTW>;
  Frag fa[UNR];
  [[maybe_unused]] Frag fb[PP ? UNR : 1];
  auto load_batch = [&](Frag* f, int b) {
#pragma unroll
    for (int r = 0; r < UNR; ++r) f[r].load(p, w, nt0, u0 + (b * UNR + r) * NW, lane, arow);
  };
  auto compute_batch = [&](const Frag* f) {
#pragma unroll
    for (int r = 0; r < UNR; ++r) f[r].compute(p, lane, acc);
  };
  if constexpr (PP) {
    if (nbatch > 0) load_batch(fa, 0);
    for (int b = 0; b < nbatch; b += 2) {
      if (b + 1 < nbatch) load_batch(fb, b + 1);
      compute_batch(fa);
      if (b + 2 < nbatch) load_batch(fa, b + 2);
      if (b + 1 < nbatch) compute_batch(fb);
    }
  } else {
    for (int b = 0; b < nbatch; ++b) {
      load_batch(fa, b);
      compute_batch(fa);
    }
  }
  for (int i = nbatch * UNR; i < nunits; ++i) {
    Frag f;
    f.load(p, w, nt0, u0 + i * NW, lane, arow);
    f.compute(p, lane, acc);
  }

  // Sum the waves' tiles through LDS (fixed order: wave 0, 1, ...), then the epilogue.
  constexpr int kVals = MB * NTW * 4;
  __shared__ Elem red[NW][kVals][64];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][(mb * NTW + t) * 4 + j][lane] = acc[mb][t][j];
  __syncthreads();
  static_assert(NW > 1, "the epilogue reads the waves' tiles from LDS");
  for (int v = threadIdx.x; v < kVals * 64; v += NW * 64) {
    const int le = v & 63;
    const int q = v >> 6;
    const int j = q & 3;
    const int t = (q >> 2) % NTW;
    const int mb = (q >> 2) / NTW;
    Elem sum = red[0][q][le];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww][q][le];
    const int ib = 16 * mb + 4 * (le >> 4) + j;
    const int n = (nt0 + t) * 16 + (le & 15);
    store_result<FAM, MOE>(p, row0 + ib, n, sum, blockIdx.z);
  }
}

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
};

const SkinnyCfg* skinny_configs(int* count) {
  *count = int(sizeof(kSkinny) / sizeof(kSkinny[0]));
  return kSkinny;
}

template <int FAM, bool MOE>
static hipError_t launch_skinny_fam(const KParams& p, int cfg, dim3 grid, hipStream_t s) {
#define HQ_SK(I)                                                                           \
  case I:                                                                                  \
    hipLaunchKernelGGL((skinny_gemm_kernel<FAM, kSkinny[I].mb, kSkinny[I].ntw, kSkinny[I].nw, \
                                           kSkinny[I].unr, kSkinny[I].pp != 0, MOE>),      \
                       grid, dim3(kSkinny[I].nw * 64), 0, s, p);                           \
    break;
  switch (cfg) {
    HQ_SK(0) HQ_SK(1) HQ_SK(2) HQ_SK(3) HQ_SK(4) HQ_SK(5) HQ_SK(6) HQ_SK(7) HQ_SK(8) HQ_SK(9)
    HQ_SK(10) HQ_SK(11) HQ_SK(12) HQ_SK(13) HQ_SK(14) HQ_SK(15) HQ_SK(16) HQ_SK(17) HQ_SK(18)
    HQ_SK(19) HQ_SK(20) HQ_SK(21) HQ_SK(22) HQ_SK(23)
    default:
      return hipErrorInvalidValue;
  }
#undef HQ_SK
  return hipGetLastError();
}

hipError_t launch_skinny(const KParams& p, int fam, bool moe, int cfg, dim3 grid,
                         hipStream_t s) {
  if (fam == FAM_WNA16) return moe ? launch_skinny_fam<FAM_WNA16, true>(p, cfg, grid, s)
                                   : launch_skinny_fam<FAM_WNA16, false>(p, cfg, grid, s);
  if (moe) return hipErrorInvalidValue;
  if (fam == FAM_W8A8) return launch_skinny_fam<FAM_W8A8, false>(p, cfg, grid, s);
  return launch_skinny_fam<FAM_W4A8, false>(p, cfg, grid, s);
}

}  // namespace hq
