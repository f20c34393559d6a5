// gemm_tiled.hip -- the large-M ("prefill") fused-dequantization GEMM for gfx950.
//
// At large M the work is MFMA-bound (the Humming announcement, section "Tuning and JIT
// compilation per workload", switches to a different pipeline at larger batch sizes). A
// workgroup computes a BM x BN output tile with WM x WN waves; each wave owns an (16*MW) x
// (16*NTW) sub-tile. Per K step of 128:
//   - the activation tile (BM rows x 128 k) is staged through LDS, double-buffered, in 16-byte
//     chunks XOR-swizzled by row so that the MFMA operand reads are bank-conflict free; all
//     waves read their rows from it;
//   - each wave streams the packed weight units of its own channel tiles straight from HBM into
//     registers one step ahead (1 KiB per unit, one 128-bit load per lane), dequantizes them in
//     registers and feeds the MFMA;
//   - WNA16 feeds the MFMA the exact bf16 value 128 + u of each code (one bit-select per pair of
//     weights), forms each 128-k group's fp32 partial with four MFMAs and applies the group scale
//     with one fp32 FMA per accumulator; the offset term sum_g s*(128 + z)*rowsum_g(x) is removed
//     once at the end by a K/128-deep fp32 MFMA contraction (exact enough: fp32 throughout).
// Workgroups are ordered so that each XCD (workgroup id mod 8) gets a contiguous band of tiles
// grouped along M, which keeps the shared weight and activation tiles in that XCD's L2.
#include <hip/hip_runtime.h>

#include "device_ops.h"
#include "gemm_common.h"
#include "internal.h"
#include "tile_epilogue.h"

namespace hq {

namespace {

template <int FAM>
struct TiledTraits;
template <>
struct TiledTraits<FAM_WNA16> {
  static constexpr int kABytes = 2;      // bf16 activations
  static constexpr int kUnitsPerStep = 1;
};
template <>
struct TiledTraits<FAM_W8A8> {
  static constexpr int kABytes = 1;
  static constexpr int kUnitsPerStep = 2;  // two 64-k units per 128-k step
};
template <>
struct TiledTraits<FAM_W4A8> {
  static constexpr int kABytes = 1;
  static constexpr int kUnitsPerStep = 1;
};

// Weight registers of one K step for NTW channel tiles.
template <int FAM, int NTW>
struct BStep {
  u32x4 b[NTW][TiledTraits<FAM>::kUnitsPerStep];
  uint32_t s[NTW];  // WNA16: bf16 scale bits; W4A8: e8m0 byte
  uint32_t z[NTW];  // WNA16 asym: packed zero byte

  __device__ __forceinline__ void load(const KParams& p, const uint8_t* w, int nt0, int ks, int lane) {
    constexpr int UPS = TiledTraits<FAM>::kUnitsPerStep;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
#pragma unroll
      for (int q = 0; q < UPS; ++q) {
        const size_t unit = size_t(nt0 + t) * p.k_units + size_t(ks) * UPS + q;
        b[t][q] = ldg16_stream(w + unit * kUnitBytes + 16 * lane);
      }
      const size_t unit = size_t(nt0 + t) * p.k_units + size_t(ks) * UPS;
      if constexpr (FAM == FAM_WNA16) {
        s[t] = *reinterpret_cast<const uint16_t*>(w + p.scales_off + unit * 32 + 2 * (lane & 15));
        z[t] = p.asym ? uint32_t(w[p.zeros_off + unit * 8 + ((lane & 15) >> 1)]) : 0u;
      } else if constexpr (FAM == FAM_W4A8) {
        s[t] = w[p.scales_off + unit * 64 + lane];
      }
    }
  }
};

template <int FAM, int MW, int NTW, int WM, int WN, int OCC, bool MOE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void tiled_gemm_kernel(KParams p, int tiles_m, int tiles_n) {
  using Acc = typename AccType<FAM>::type;
  constexpr int kThreads = 64 * WM * WN;
  constexpr int BM = 16 * MW * WM;
  constexpr int AB = TiledTraits<FAM>::kABytes;
  constexpr int RB = 128 * AB;              // bytes of one activation row per K step
  constexpr int CPR = RB / 16;              // 16-byte chunks per row
  constexpr int kChunks = BM * CPR;
  static_assert(kChunks % kThreads == 0, "activation tile must split evenly over threads");
  constexpr int CH = kChunks / kThreads;    // chunks each thread moves per K step
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile coordinates ----
  int mt, ntile;
  const uint8_t* w = p.w;
  int row0;
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
    // XCD-aware: the hardware deals workgroups round-robin over 8 XCDs; give each XCD a
    // contiguous range of logical tiles, then walk them in groups of 8 m-tiles.
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
  const int nt0 = ntile * NTW * WN + wn * NTW;   // first 16-channel tile of this wave

  // ---- per-thread activation source rows (constant over K) ----
  const uint8_t* asrc[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int ci = tid + j * kThreads;
    const int r = ci / CPR;
    const int c = ci % CPR;
    const uint8_t* base = nullptr;
    if constexpr (MOE) {
      const int id = p.sorted_ids[row0 + r];
      if (id < p.M) base = p.a + size_t(id / p.topk) * p.K * AB;
    } else {
      if (row0 + r < p.M) base = p.a + size_t(row0 + r) * p.K * AB;
    }
    asrc[j] = base ? base + c * 16 : nullptr;
  }

  auto load_a = [&](int ks, u32x4* regs) {
#pragma unroll
    for (int j = 0; j < CH; ++j)
      regs[j] = asrc[j] ? ldg16(asrc[j] + size_t(ks) * RB) : u32x4{0, 0, 0, 0};
  };
  auto store_a = [&](int stage, const u32x4* regs) {
    uint8_t* sbase = smem + stage * (BM * RB);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int ci = tid + j * kThreads;
      const int r = ci / CPR;
      const int c = ci % CPR;
      *reinterpret_cast<u32x4*>(sbase + r * RB + lds_chunk_swizzle(r, c, CPR) * 16) = regs[j];
    }
  };
  auto read_frag = [&](int stage, int mb, int chunk) -> u32x4 {
    const int r = wm * 16 * MW + 16 * mb + (lane & 15);
    return *reinterpret_cast<const u32x4*>(smem + stage * (BM * RB) + r * RB + lds_chunk_swizzle(r, chunk, CPR) * 16);
  };

  Acc acc[MW][NTW];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mb][t] = Acc{0, 0, 0, 0};

  const int nks = p.K / 128;
  u32x4 areg[CH];
  load_a(0, areg);
  store_a(0, areg);
  BStep<FAM, NTW> bcur, bnext;
  bcur.load(p, w, nt0, 0, lane);
  __syncthreads();

  for (int ks = 0; ks < nks; ++ks) {
    const int stage = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) {
      load_a(ks + 1, areg);
      bnext.load(p, w, nt0, ks + 1, lane);
    }
    if constexpr (FAM == FAM_WNA16) {
      bf16x8 af[MW][4];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          af[mb][d] = __builtin_bit_cast(bf16x8, read_frag(stage, mb, 4 * (lane >> 4) + d));
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float s = bf16_bits_to_f32(bcur.s[t]);
        bf16x8 bw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = dequant_int4x8_offset128(bcur.b[t][0][d]);
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
        for (int mb = 0; mb < MW; ++mb) af[mb] = read_frag(stage, mb, 4 * q + (lane >> 4));
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int mb = 0; mb < MW; ++mb) acc[mb][t] = mfma_i8(af[mb], bcur.b[t][q], acc[mb][t]);
      }
    } else {
      u32x4 alo[MW], ahi[MW];
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        alo[mb] = read_frag(stage, mb, lane >> 4);
        ahi[mb] = read_frag(stage, mb, 4 + (lane >> 4));
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mb = 0; mb < MW; ++mb)
          acc[mb][t] = mfma_fp8_fp4(alo[mb], ahi[mb], bcur.b[t][0], int(bcur.s[t]), acc[mb][t]);
    }
    if (more) {
      store_a(stage ^ 1, areg);
      bcur = bnext;
    }
    __syncthreads();
  }

  const int row_base = row0 + wm * 16 * MW;
  if constexpr (FAM == FAM_WNA16) wna16_offset_contraction<MW, NTW, MOE>(p, w, acc, row_base, nt0, lane);
  store_tile<FAM, MOE, MW, NTW>(p, w, acc, row_base, nt0, lane);
}

}  // namespace


static constexpr TiledCfg kTiled[] = {
    {4, 4, 2, 2, 1},  // 0: 128 x 128 tile, 64 x 64 per wave
    {4, 2, 2, 2, 1},  // 1: 128 x 64 (N/16 even)
    {4, 1, 2, 2, 2},  // 2: 128 x 32 (any N)
    {2, 4, 2, 2, 2},  // 3: 64 x 128 (MoE block 64)
    {2, 4, 2, 2, 1},  // 4: 64 x 128
    {4, 2, 2, 4, 2},  // 5: 128 x 128, 8 waves of 64 x 32
};

const TiledCfg* tiled_configs(int* count) {
  *count = int(sizeof(kTiled) / sizeof(kTiled[0]));
  return kTiled;
}

template <int FAM, bool MOE>
static hipError_t launch_tiled_fam(const KParams& p, int cfg, dim3 grid, int tiles_m, int tiles_n,
                                   hipStream_t s) {
#define HQ_TL(I)                                                                                    \
  case I: {                                                                                         \
    constexpr TiledCfg C = kTiled[I];                                                               \
    constexpr int kSmem = 2 * 16 * C.mw * C.wm * 128 * TiledTraits<FAM>::kABytes;                   \
    auto kern = tiled_gemm_kernel<FAM, C.mw, C.ntw, C.wm, C.wn, C.occ, MOE>;                               \
    if (kSmem > 65536) (void)hipFuncSetAttribute((const void*)kern,                                     \
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);     \
    hipLaunchKernelGGL(kern, grid, dim3(64 * C.wm * C.wn), kSmem, s, p, tiles_m, tiles_n);          \
    break;                                                                                          \
  }
  switch (cfg) {
    HQ_TL(0) HQ_TL(1) HQ_TL(2) HQ_TL(3) HQ_TL(4) HQ_TL(5)
    default:
      return hipErrorInvalidValue;
  }
#undef HQ_TL
  return hipGetLastError();
}

hipError_t launch_tiled(const KParams& p, int fam, bool moe, int cfg, dim3 grid, int tiles_m,
                        int tiles_n, hipStream_t s) {
  if (fam == FAM_WNA16) return moe ? launch_tiled_fam<FAM_WNA16, true>(p, cfg, grid, tiles_m, tiles_n, s)
                                   : launch_tiled_fam<FAM_WNA16, false>(p, cfg, grid, tiles_m, tiles_n, s);
  if (moe) return hipErrorInvalidValue;
  if (fam == FAM_W8A8) return launch_tiled_fam<FAM_W8A8, false>(p, cfg, grid, tiles_m, tiles_n, s);
  if (fam == FAM_W4A8) return launch_tiled_fam<FAM_W4A8, false>(p, cfg, grid, tiles_m, tiles_n, s);
  return hipErrorInvalidValue;   // W4A4 runs on the skinny and ping-pong kernels only
}

}  // namespace hq
