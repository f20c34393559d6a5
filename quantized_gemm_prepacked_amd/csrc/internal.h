// internal.h -- declarations shared by the C ABI (hq_api.cpp), the host prepack and the HIP
// launchers. Not part of the public interface.
#pragma once
#include <string>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "hq.h"
#include "layout.h"

namespace hq {

// A validated weight/activation/output combination.
struct Combo {
  Family fam;
  bool asym;     // WNA16 with zero-points
  bool out_i32;  // W8A8 raw accumulator output
  bool invariant;  // HQ_COMPUTE_BATCH_INVARIANT: one fixed kernel configuration for every M
  bool stream_k;   // HQ_COMPUTE_STREAM_K: small-M calls balanced over the CUs (Stream-K)
};

size_t prepacked_bytes(const Combo& c, int64_t E, int64_t N, int64_t K);
void prepack(const Combo& c, int64_t E, int64_t N, int64_t K, const void* wq, const void* scales,
             const void* zeros, void* out);

// Kernel choice for one call (see dispatch in gemm_kernels.hip).
struct Plan {
  int kind;    // 0 = skinny (waves split K), 1 = tiled (LDS-staged activations), 2 = pipelined,
               // 3 = ping-pong, 4 = skinny Stream-K (one row block, `split` workgroups)
  int cfg;     // index into the kind's instantiation table
  int split;   // K splits across workgroups (partials in the workspace, then a reduction);
               // Stream-K: the number of workgroups
  size_t ws_bytes;
  long long sk_items = 0;   // Stream-K: (tile group, K unit) items
  int sk_slots = 0;         // Stream-K: partial-tile slots per tile group
};

struct GemmCall {
  Combo c;
  int64_t M, N, K;
  const void* a;
  const float* a_scale;
  const uint8_t* w;
  void* y;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  // MoE (sorted_ids != nullptr)
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  const float* topk_weights;
  int64_t T;
  int32_t topk;
  int32_t E;
  int32_t block_m;
  int64_t max_blocks;
};

Plan plan_dense(const Combo& c, int64_t M, int64_t N, int64_t K);
// Run-time tuning table (tuning_table.cpp): load (path NULL clears), lookup for a dense call.
int load_tuning_table(const char* path, std::string* err);
bool tuning_lookup(const Combo& c, int64_t M, int64_t N, int64_t K, int* kind, int* cfg, int* split);
int kernel_config_count(int kind);
Plan plan_moe(const Combo& c, int64_t T, int32_t topk, int32_t E, int64_t N, int64_t K,
              int32_t block_m);
int32_t moe_block_m(const Combo& c, int64_t T, int32_t topk, int32_t E, int64_t N, int64_t K);
bool moe_block_m_supported(int32_t block_m);
hipError_t launch_gemm(const GemmCall& call, const Plan& plan);
// hq_gemm_noalloc's workspace: a library-owned device array of kNoAllocScratchBytes per GPU; the
// device address of the current device's copy (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(HQ_NOALLOC_SCRATCH_BYTES);
hipError_t noalloc_scratch(void** ptr);

size_t moe_align_ws_bytes(int64_t T, int32_t topk, int32_t E, int32_t block_m);
hipError_t launch_grouped_index(const int32_t* offsets, int64_t R, int32_t E, int32_t bm, int64_t cap,
                                int32_t* sorted, int32_t* block_expert, int32_t* num_padded,
                                hipStream_t stream);
hipError_t launch_silu_mul(int64_t R, int64_t I, const void* gate_up, void* act, hipStream_t s);
hipError_t launch_moe_combine(int64_t T, int32_t topk, int32_t E, int64_t N, const int32_t* topk_ids,
                              const void* y, void* out, hipStream_t s);
hipError_t launch_act_quant(int act_fmt, int64_t M, int64_t K, const void* x, void* xq, float* s_tok,
                            hipStream_t stream);
hipError_t launch_silu_mul_quant(int act_fmt, int64_t R, int64_t I, const void* gate_up, void* act_q,
                                 float* act_scale, hipStream_t stream);
hipError_t launch_moe_align(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                            int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                            int32_t* expert_offsets, int32_t* num_padded, void* ws,
                            hipStream_t stream);

}  // namespace hq
