// gemm_common.h -- kernel parameters and the output epilogue shared by the GEMM kernels.
//
// The epilogue is where the Humming announcement (section "Shared CUDA components across
// formats and architectures") fuses scaling into the output stage: per-token and per-channel
// scales, the MoE router weight, bf16 rounding and the MoE row scatter happen here, once per
// output element.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_ops.h"
#include "layout.h"

namespace hq {

struct KParams {
  const uint8_t* a;         // activations [rows, K] (bf16 / int8 / e4m3)
  const float* a_scale;     // per-token scale [rows] (INT8 / FP8 activations)
  const uint8_t* w;         // prepacked weights, expert 0
  void* y;                  // output [M, N] bf16 or int32
  void* ws;                 // split-K partials [split][M][N] (fp32 or int32)
  int M;                    // dense: rows of A and y; MoE: T * topk (flat routed rows)
  int N, K;
  int k_units;              // K / K unit
  int units_per_split;
  int split;
  int asym, out_i32;
  size_t expert_stride, scales_off, zeros_off;
  const int32_t* sorted_ids;    // MoE only
  const int32_t* block_expert;
  const int32_t* num_padded;
  const float* topk_weights;
  int topk;
  int E;                    // MoE experts (block_expert entries outside [0, E) are skipped)
  // Stream-K (skinny kernel, one row block): (tile group, K unit) items in all, partial-tile
  // slots per tile group in the workspace, and the per-group arrival counters (zero between calls)
  long long sk_items;
  int sk_slots;
  uint32_t* sk_counters;
};

template <int FAM>
struct AccType {
  typedef f32x4 type;
  typedef float elem;
};
template <>
struct AccType<FAM_W8A8> {
  typedef i32x4 type;
  typedef int elem;
};

// Final value of output (orow, n): `v` is the full K sum; srow indexes the per-token scale.
// w: the weights of the expert (MoE) or the layer, for the per-channel scales (W8A8, W8A16,
// F8A16).
template <int FAM>
__device__ __forceinline__ void epilogue(const KParams& p, const uint8_t* w, int orow, int srow, int n,
                                         typename AccType<FAM>::elem v, float tw) {
  const size_t o = size_t(orow) * p.N + n;
  if constexpr (family_int_groups(FAM)) {
    reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(v * tw);
  } else if constexpr (FAM == FAM_W8A8) {
    if (p.out_i32) {
      reinterpret_cast<int*>(p.y)[o] = v;
    } else {
      const float sch = reinterpret_cast<const float*>(w + p.scales_off)[n];
      reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(float(v) * p.a_scale[srow] * sch * tw);
    }
  } else if constexpr (FAM == FAM_W4A8) {
    reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(v * p.a_scale[srow] * tw);
  } else if constexpr (FAM == FAM_W8A16 || FAM == FAM_F8A16) {
    const float sch = reinterpret_cast<const float*>(w + p.scales_off)[n];
    reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(v * sch * tw);
  } else {   // W4A4, W4A8MX: both block scales were applied by the MFMA
    reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(v * tw);
  }
}

// Row `row` of the workgroup's row space (dense: m; MoE: position in sorted_ids).
template <int FAM, bool MOE>
__device__ __forceinline__ void store_result(const KParams& p, const uint8_t* w, int row, int n,
                                             typename AccType<FAM>::elem v, int z) {
  if constexpr (MOE) {
    const int id = p.sorted_ids[row];
    if (id >= p.M) return;
    const float tw = p.topk_weights ? p.topk_weights[id] : 1.0f;
    epilogue<FAM>(p, w, id, id / p.topk, n, v, tw);
  } else {
    if (row >= p.M) return;
    if (p.split > 1) {
      typedef typename AccType<FAM>::elem E;
      reinterpret_cast<E*>(p.ws)[(size_t(z) * p.M + row) * p.N + n] = v;
      return;
    }
    epilogue<FAM>(p, w, row, row, n, v, 1.0f);
  }
}

// A skinny-kernel instantiation: MB row blocks of 16, NTW channel tiles of 16, NW waves that
// split K, UNR units per batch; pp = 1 double-buffers batches (next batch in flight while the
// current one is computed); few = 1 (MB = 1, dense only, M <= kFewRows): only the first rows of
// the block are copied and reduced -- one 1 KiB activation copy per unit, the other MFMA rows
// repeating them and never stored.
struct SkinnyCfg {
  int mb, ntw, nw, unr, pp;
  int few = 0;
};
constexpr int kFewRows = 4;
const SkinnyCfg* skinny_configs(int* count);
int skinny_lds_bytes(int fam, int cfg);
// Stream-K instantiations exist for these skinny configurations (the ones chosen at M <= 16).
bool skinny_stream_k_cfg(int cfg);
hipError_t launch_skinny_stream_k(const KParams& p, int fam, int cfg, int wgs, hipStream_t s);

// A tiled-kernel instantiation: waves own (16*MW) x (16*NTW) sub-tiles, WM x WN waves per
// workgroup; the workgroup tile is (16*MW*WM) x (16*NTW*WN).
struct TiledCfg {
  int mw, ntw, wm, wn, occ;  // occ: waves per SIMD the register allocation must allow
};
const TiledCfg* tiled_configs(int* count);
hipError_t launch_tiled(const KParams& p, int fam, bool moe, int cfg, dim3 grid, int tiles_m,
                        int tiles_n, hipStream_t s);

// A pipelined-kernel instantiation: WM x WN waves of (16*MW) x (16*NTW), STAGES K steps in flight.
struct PipeCfg {
  int mw, ntw, wm, wn, stages;
};
const PipeCfg* pipe_configs(int* count);
int pipe_lds_bytes(int fam, int cfg);
hipError_t launch_pipe(const KParams& p, int fam, bool moe, int cfg, dim3 grid, int tiles_m,
                       int tiles_n, hipStream_t s);

// A ping-pong-kernel instantiation: eight waves (WM x WN) of (16*MW) x (16*NTW), `stages` LDS
// slots (K steps resident or in flight); the workgroup tile is (16*MW*WM) x (16*NTW*WN).
struct PPCfg {
  int mw, ntw, wm, wn;
  int stages = 3;
};
const PPCfg* pp_configs(int* count);
int pp_lds_bytes(int fam, int cfg);
hipError_t launch_pingpong(const KParams& p, int fam, bool moe, int cfg, dim3 grid, int tiles_m,
                           int tiles_n, hipStream_t s);
// WNA16 group sums for the LDS-staged kernels' offset term: per row, Gp = ceil(K/128 / 32) * 32
// bf16 high halves then Gp low halves.
size_t group_sums_split_bytes(int64_t rows, int64_t K);
hipError_t launch_group_sums_split(const uint8_t* a, int rows, int K, void* ws, hipStream_t s);


hipError_t launch_skinny(const KParams& p, int fam, bool moe, int cfg, dim3 grid, hipStream_t s);
hipError_t launch_splitk_reduce(const KParams& p, int fam, hipStream_t s);

}  // namespace hq
