// hq_api.cpp -- the C ABI (include/hq.h): argument validation, then prepack or kernel launch.
//
// Validation follows the preprocessing contract of the Humming announcement (section "Tuning and
// JIT compilation per workload": parameters are validated before anything runs). Every check
// here happens on the host before any HIP call, so a rejected call has no device side effect.
#include "hq.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.h"
#include "layout.h"

namespace {

thread_local std::string g_last_error;

hq_status fail(hq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hq_status ok() {
  g_last_error.clear();
  return HQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

// Map a description onto a supported combination.
hq_status resolve(const hq_quant_desc* d, hq::Combo* c) {
  if (!d) return fail(HQ_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->struct_size != sizeof(hq_quant_desc))
    return fail(HQ_ERR_INVALID_ARGUMENT, "desc->struct_size %u != %zu", d->struct_size,
                sizeof(hq_quant_desc));
  if (d->out_fmt != HQ_OUT_BF16 && d->out_fmt != HQ_OUT_INT32_ACC)
    return fail(HQ_ERR_INVALID_ARGUMENT, "unknown out_fmt %d", d->out_fmt);
  c->out_i32 = d->out_fmt == HQ_OUT_INT32_ACC;
  c->asym = false;
  if (d->compute_flags & ~int32_t(HQ_COMPUTE_BATCH_INVARIANT | HQ_COMPUTE_STREAM_K))
    return fail(HQ_ERR_INVALID_ARGUMENT, "unknown compute_flags bits 0x%x", unsigned(d->compute_flags));
  c->invariant = (d->compute_flags & HQ_COMPUTE_BATCH_INVARIANT) != 0;
  c->stream_k = !c->invariant && (d->compute_flags & HQ_COMPUTE_STREAM_K) != 0;
  switch (d->weight_fmt) {
    case HQ_W_INT4_SYM:
    case HQ_W_UINT4_ASYM: {
      const bool asym = d->weight_fmt == HQ_W_UINT4_ASYM;
      if (d->group_size != 128 || d->scale_dtype != HQ_SCALE_BF16 ||
          d->has_zero_point != (asym ? 1 : 0) || d->act_fmt != HQ_ACT_BF16 || c->out_i32)
        return fail(HQ_ERR_UNSUPPORTED,
                    "INT4 weights need group_size 128, BF16 scales, has_zero_point %d, BF16 "
                    "activations and bf16 output",
                    asym ? 1 : 0);
      c->fam = hq::FAM_WNA16;
      c->asym = asym;
      return HQ_OK;
    }
    case HQ_W_UINT2_ASYM:
    case HQ_W_UINT3_ASYM:
      if (d->group_size != 128 || d->scale_dtype != HQ_SCALE_BF16 || d->has_zero_point != 1 ||
          d->act_fmt != HQ_ACT_BF16 || c->out_i32)
        return fail(HQ_ERR_UNSUPPORTED,
                    "UINT2 / UINT3 weights need group_size 128, BF16 scales, has_zero_point 1, BF16 "
                    "activations and bf16 output");
      c->fam = d->weight_fmt == HQ_W_UINT2_ASYM ? hq::FAM_WNA2 : hq::FAM_WNA3;
      c->asym = true;
      return HQ_OK;
    case HQ_W_INT8_SYM:
      if (d->act_fmt == HQ_ACT_BF16) {
        if (d->group_size != 0 || d->scale_dtype != HQ_SCALE_FP32 || d->has_zero_point != 0 || c->out_i32)
          return fail(HQ_ERR_UNSUPPORTED,
                      "INT8 weights with BF16 activations need group_size 0 (per channel), FP32 "
                      "scales, no zero-point and bf16 output");
        c->fam = hq::FAM_W8A16;
        return HQ_OK;
      }
      if (d->group_size != 0 || d->scale_dtype != HQ_SCALE_FP32 || d->has_zero_point != 0 ||
          d->act_fmt != HQ_ACT_INT8_PER_TOKEN)
        return fail(HQ_ERR_UNSUPPORTED,
                    "INT8 weights need group_size 0 (per channel), FP32 scales, no zero-point "
                    "and per-token INT8 activations (or BF16 activations, see above)");
      c->fam = hq::FAM_W8A8;
      return HQ_OK;
    case HQ_W_FP4_E2M1:
      if (d->group_size != 32 || d->scale_dtype != HQ_SCALE_E8M0 || d->has_zero_point != 0 ||
          (d->act_fmt != HQ_ACT_FP8E4M3_PER_TOKEN && d->act_fmt != HQ_ACT_MXFP4 &&
           d->act_fmt != HQ_ACT_MXFP8 && d->act_fmt != HQ_ACT_BF16) || c->out_i32)
        return fail(HQ_ERR_UNSUPPORTED,
                    "FP4 weights need group_size 32, E8M0 scales, no zero-point, BF16, per-token FP8 "
                    "e4m3, MXFP8 or MXFP4 activations and bf16 output");
      c->fam = d->act_fmt == HQ_ACT_MXFP4   ? hq::FAM_W4A4
               : d->act_fmt == HQ_ACT_MXFP8 ? hq::FAM_W4A8MX
               : d->act_fmt == HQ_ACT_BF16  ? hq::FAM_MXW4A16
                                            : hq::FAM_W4A8;
      return HQ_OK;
    case HQ_W_FP8_E4M3:
      if (d->act_fmt == HQ_ACT_BF16) {
        if (d->group_size != 0 || d->scale_dtype != HQ_SCALE_FP32 || d->has_zero_point != 0 || c->out_i32)
          return fail(HQ_ERR_UNSUPPORTED,
                      "FP8 weights with BF16 activations need group_size 0 (per channel), FP32 "
                      "scales, no zero-point and bf16 output");
        c->fam = hq::FAM_F8A16;
        return HQ_OK;
      }
      if (d->group_size != 128 || d->scale_dtype != HQ_SCALE_FP32 || d->has_zero_point != 0 ||
          d->act_fmt != HQ_ACT_FP8E4M3_BLOCK128 || c->out_i32)
        return fail(HQ_ERR_UNSUPPORTED,
                    "FP8 weights need group_size 128 (128 x 128 blocks), FP32 scales, no zero-point, "
                    "FP8 activations with 128-k block scales and bf16 output");
      c->fam = hq::FAM_FP8B;
      return HQ_OK;
    default:
      return fail(HQ_ERR_INVALID_ARGUMENT, "unknown weight_fmt %d", d->weight_fmt);
  }
}

hq_status check_shape(const hq::Combo& c, int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "N=%lld K=%lld out of range", (long long)N, (long long)K);
  const int ku = (c.fam == hq::FAM_FP8B || c.fam == hq::FAM_W8A16 || c.fam == hq::FAM_F8A16)
                     ? 128 : hq::family_k_unit(c.fam);
  if (c.fam == hq::FAM_FP8B && N % 128 != 0)
    return fail(HQ_ERR_UNSUPPORTED, "FP8 block-scaled weights need N %% 128 == 0 (N=%lld)", (long long)N);
  if (N % 16 != 0 || K % ku != 0)
    return fail(HQ_ERR_UNSUPPORTED, "N must be a multiple of 16 and K of %d (N=%lld K=%lld)", ku,
                (long long)N, (long long)K);
  return HQ_OK;
}

hq_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* hq_last_error(void) { return g_last_error.c_str(); }

int32_t hq_version(void) { return 101; }

size_t hq_prepacked_bytes(const hq_quant_desc* desc, int64_t E, int64_t N, int64_t K) {
  hq::Combo c{};
  if (resolve(desc, &c) != HQ_OK || E <= 0 || check_shape(c, N, K) != HQ_OK) return 0;
  return hq::prepacked_bytes(c, E, N, K);
}

hq_status hq_prepack_weights(const hq_quant_desc* desc, int64_t E, int64_t N, int64_t K,
                             const void* wq, const void* scales, const void* zeros, void* out,
                             size_t out_bytes) {
  hq::Combo c{};
  hq_status s = resolve(desc, &c);
  if (s != HQ_OK) return s;
  if (E <= 0 || E > 65536) return fail(HQ_ERR_INVALID_ARGUMENT, "E=%lld out of range", (long long)E);
  if ((s = check_shape(c, N, K)) != HQ_OK) return s;
  if (!wq || !scales || !out) return fail(HQ_ERR_INVALID_ARGUMENT, "wq, scales and out must be non-NULL");
  if (c.asym && !zeros) return fail(HQ_ERR_INVALID_ARGUMENT, "zeros must be non-NULL for UINT4_ASYM / UINT3_ASYM / UINT2_ASYM");
  if (!c.asym && zeros) return fail(HQ_ERR_INVALID_ARGUMENT, "zeros must be NULL without zero-points");
  const size_t need = hq::prepacked_bytes(c, E, N, K);
  if (out_bytes < need)
    return fail(HQ_ERR_WORKSPACE, "out_bytes %zu < required %zu", out_bytes, need);
  hq::prepack(c, E, N, K, wq, scales, zeros, out);
  return ok();
}

hq_status hq_load_tuning_table(const char* path) {
  std::string err;
  if (hq::load_tuning_table(path, &err) != 0) return fail(HQ_ERR_INVALID_ARGUMENT, "%s", err.c_str());
  return ok();
}

hq_status hq_gemm_plan(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K, int32_t* kind,
                       int32_t* cfg, int32_t* split) {
  hq::Combo c{};
  hq_status s = resolve(desc, &c);
  if (s != HQ_OK) return s;
  if ((s = check_shape(c, N, K)) != HQ_OK) return s;
  if (M <= 0 || M > kMaxDim) return fail(HQ_ERR_INVALID_ARGUMENT, "M=%lld out of range", (long long)M);
  if (!kind || !cfg || !split) return fail(HQ_ERR_INVALID_ARGUMENT, "kind, cfg and split must be non-NULL");
  const hq::Plan p = hq::plan_dense(c, M, N, K);
  *kind = p.kind;
  *cfg = p.cfg;
  *split = p.split;
  return p.kind < 0 ? fail(HQ_ERR_INVALID_ARGUMENT, "the HQ_TUNE override does not fit this shape") : ok();
}

int32_t hq_kernel_config_count(int32_t kind) { return kind < 0 || kind > 3 ? 0 : hq::kernel_config_count(kind); }

size_t hq_gemm_workspace_bytes(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K) {
  hq::Combo c{};
  if (resolve(desc, &c) != HQ_OK || M <= 0 || M > kMaxDim || check_shape(c, N, K) != HQ_OK) return 0;
  return hq::plan_dense(c, M, N, K).ws_bytes;
}

}  // extern "C"

namespace {

// hq_gemm and hq_gemm_noalloc: validation, plan, launch. noalloc: the workspace is the
// library-owned scratch array of the current device instead of (ws, ws_bytes).
hq_status gemm_entry(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K, const void* a,
                     const float* a_scale, const void* w_packed, void* y, void* ws, size_t ws_bytes,
                     hq_stream_t stream, bool noalloc) {
  hq::Combo c{};
  hq_status s = resolve(desc, &c);
  if (s != HQ_OK) return s;
  if ((s = check_shape(c, N, K)) != HQ_OK) return s;
  if (M < 0 || M > kMaxDim) return fail(HQ_ERR_INVALID_ARGUMENT, "M=%lld out of range", (long long)M);
  if (M * N >= (int64_t(1) << 31) || M * K >= (int64_t(1) << 40))
    return fail(HQ_ERR_UNSUPPORTED, "M*N must stay below 2^31 (M=%lld N=%lld)", (long long)M, (long long)N);
  if (!a || !w_packed || !y) return fail(HQ_ERR_INVALID_ARGUMENT, "a, w_packed and y must be non-NULL");
  if (!aligned16(a) || !aligned16(w_packed) || !aligned16(y))
    return fail(HQ_ERR_INVALID_ARGUMENT, "a, w_packed and y must be 16-byte aligned");
  const bool needs_scale = !hq::family_bf16_act(c.fam);
  if (needs_scale && !a_scale) return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale is required for INT8/FP8 activations");
  if (!needs_scale && a_scale) return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale must be NULL for BF16 activations");
  if (a_scale && (reinterpret_cast<uintptr_t>(a_scale) & 3u))
    return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale must be 4-byte aligned");
  if (M == 0) return ok();
  const hq::Plan plan = hq::plan_dense(c, M, N, K);
  if (plan.kind < 0) return fail(HQ_ERR_INVALID_ARGUMENT, "the HQ_TUNE override does not fit this shape");
  if (noalloc) {
    if (plan.ws_bytes > hq::kNoAllocScratchBytes)
      return fail(HQ_ERR_WORKSPACE,
                  "hq_gemm_noalloc: this call needs %zu bytes of scratch, more than the %zu bytes the "
                  "library holds per GPU (use hq_gemm with a workspace)",
                  plan.ws_bytes, hq::kNoAllocScratchBytes);
    ws_bytes = hq::kNoAllocScratchBytes;
    ws = nullptr;
    if (plan.ws_bytes) {
      const hipError_t e = hq::noalloc_scratch(&ws);
      if (e != hipSuccess) return fail(HQ_ERR_HIP, "hq_gemm_noalloc: scratch address: %s", hipGetErrorString(e));
    }
  } else {
    if (ws_bytes < plan.ws_bytes || (plan.ws_bytes && !ws))
      return fail(HQ_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, plan.ws_bytes);
    if (ws && !aligned16(ws)) return fail(HQ_ERR_INVALID_ARGUMENT, "ws must be 16-byte aligned");
  }
  hq::GemmCall call{};
  call.c = c;
  call.M = M;
  call.N = N;
  call.K = K;
  call.a = a;
  call.a_scale = a_scale;
  call.w = static_cast<const uint8_t*>(w_packed);
  call.y = y;
  call.ws = ws;
  call.ws_bytes = ws_bytes;
  call.stream = static_cast<hipStream_t>(stream);
  return check_hip(hq::launch_gemm(call, plan), noalloc ? "hq_gemm_noalloc launch" : "hq_gemm launch");
}

}  // namespace

extern "C" {

hq_status hq_gemm(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K, const void* a,
                  const float* a_scale, const void* w_packed, void* y, void* ws, size_t ws_bytes,
                  hq_stream_t stream) {
  return gemm_entry(desc, M, N, K, a, a_scale, w_packed, y, ws, ws_bytes, stream, false);
}

hq_status hq_gemm_noalloc(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K, const void* a,
                          const float* a_scale, const void* w_packed, void* y, hq_stream_t stream) {
  return gemm_entry(desc, M, N, K, a, a_scale, w_packed, y, nullptr, 0, stream, true);
}

size_t hq_moe_align_capacity(int64_t T, int32_t topk, int32_t E, int32_t block_m) {
  if (T < 0 || topk <= 0 || E <= 0 || block_m <= 0) return 0;
  const int64_t n_flat = T * topk;
  const int64_t active = std::min<int64_t>(E, n_flat);
  const int64_t cap = n_flat + active * (block_m - 1);
  return size_t((cap + block_m - 1) / block_m * block_m);
}

size_t hq_moe_align_workspace_bytes(int64_t T, int32_t topk, int32_t E, int32_t block_m) {
  return hq::moe_align_ws_bytes(T, topk, E, block_m);
}

hq_status hq_moe_align(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                       int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* expert_offsets, int32_t* num_padded, void* ws, size_t ws_bytes,
                       hq_stream_t stream) {
  if (T < 0 || T * int64_t(topk) > (int64_t(1) << 30))
    return fail(HQ_ERR_INVALID_ARGUMENT, "T=%lld out of range", (long long)T);
  if (topk <= 0 || topk > 64) return fail(HQ_ERR_INVALID_ARGUMENT, "topk=%d out of range", topk);
  if (E <= 0 || E > 512) return fail(HQ_ERR_UNSUPPORTED, "E=%d: 1..512 experts supported", E);
  if (block_m < 16 || block_m > 256 || block_m % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "block_m=%d must be a multiple of 16 in [16, 256]", block_m);
  if (!sorted_ids || !block_expert || !expert_offsets || !num_padded || (T > 0 && !topk_ids))
    return fail(HQ_ERR_INVALID_ARGUMENT, "output pointers and topk_ids must be non-NULL");
  const size_t need = hq::moe_align_ws_bytes(T, topk, E, block_m);
  if (ws_bytes < need) return fail(HQ_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, need);
  return check_hip(hq::launch_moe_align(topk_ids, T, topk, E, block_m, sorted_ids, block_expert,
                                        expert_offsets, num_padded, ws,
                                        static_cast<hipStream_t>(stream)),
                   "hq_moe_align launch");
}

hq_status hq_quantize_activations(int32_t act_fmt, int64_t M, int64_t K, const void* x, void* xq,
                                  float* s_tok, hq_stream_t stream) {
  if (act_fmt != HQ_ACT_INT8_PER_TOKEN && act_fmt != HQ_ACT_FP8E4M3_PER_TOKEN && act_fmt != HQ_ACT_MXFP4 &&
      act_fmt != HQ_ACT_MXFP8 && act_fmt != HQ_ACT_FP8E4M3_BLOCK128)
    return fail(HQ_ERR_UNSUPPORTED, "act_fmt=%d: INT8 or FP8 e4m3 per-token, FP8 per 128-k block, MXFP8 or MXFP4",
                act_fmt);
  if (act_fmt == HQ_ACT_FP8E4M3_BLOCK128 && K % 128 != 0)
    return fail(HQ_ERR_UNSUPPORTED, "K=%lld must be a multiple of 128 for FP8 block scales", (long long)K);
  const bool mx = act_fmt == HQ_ACT_MXFP4 || act_fmt == HQ_ACT_MXFP8;
  if (M < 0 || M > kMaxDim || K <= 0 || K > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "M=%lld K=%lld out of range", (long long)M, (long long)K);
  if (K % 8 != 0) return fail(HQ_ERR_UNSUPPORTED, "K=%lld must be a multiple of 8", (long long)K);
  if (mx && K % 32 != 0)
    return fail(HQ_ERR_UNSUPPORTED, "K=%lld must be a multiple of 32 for MX activations", (long long)K);
  if (mx && M * (K / 32) >= (int64_t(1) << 40))
    return fail(HQ_ERR_UNSUPPORTED, "M*K/32 must stay below 2^40");
  if (M == 0) return ok();
  if (!x || !xq || !s_tok) return fail(HQ_ERR_INVALID_ARGUMENT, "x, xq and s_tok must be non-NULL");
  if (!aligned16(x) || !aligned16(xq) || (reinterpret_cast<uintptr_t>(s_tok) & 3u))
    return fail(HQ_ERR_INVALID_ARGUMENT, "x and xq must be 16-byte aligned, s_tok 4-byte aligned");
  return check_hip(hq::launch_act_quant(act_fmt, M, K, x, xq, s_tok, static_cast<hipStream_t>(stream)),
                   "hq_quantize_activations launch");
}

namespace {
// Workspace of hq_grouped_gemm: the row index (sorted ids, block -> expert table, num_padded),
// then the grouped GEMM's own workspace, each 256-byte aligned.
struct GroupedWs {
  int32_t bm;
  size_t cap, sorted_off, bexp_off, npad_off, gemm_off, gemm_bytes, total;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

GroupedWs grouped_ws(const hq::Combo& c, int64_t R, int32_t E, int64_t N, int64_t K) {
  GroupedWs g{};
  g.bm = hq::moe_block_m(c, R, 1, E, N, K);
  g.cap = hq_moe_align_capacity(R, 1, E, g.bm);
  g.sorted_off = 0;
  g.bexp_off = align256(g.cap * 4);
  g.npad_off = g.bexp_off + align256(std::max<size_t>(g.cap / g.bm, 1) * 4);
  g.gemm_off = g.npad_off + 256;
  g.gemm_bytes = hq::plan_moe(c, R, 1, E, N, K, g.bm).ws_bytes;
  g.total = g.gemm_off + align256(g.gemm_bytes);
  return g;
}
}  // namespace

size_t hq_grouped_gemm_workspace_bytes(const hq_quant_desc* desc, int64_t R, int32_t E, int64_t N, int64_t K) {
  hq::Combo c{};
  if (resolve(desc, &c) != HQ_OK || check_shape(c, N, K) != HQ_OK || R < 0 || E <= 0 || E > 512) return 0;
  return grouped_ws(c, R, E, N, K).total;
}

hq_status hq_grouped_gemm(const hq_quant_desc* desc, int64_t R, int32_t E, int64_t N, int64_t K,
                          const void* a, const float* a_scale, const void* w_packed,
                          const int32_t* expert_offsets, void* y, void* ws, size_t ws_bytes,
                          hq_stream_t stream) {
  hq::Combo c{};
  hq_status s = resolve(desc, &c);
  if (s != HQ_OK) return s;
  const bool per_token = !hq::family_bf16_act(c.fam);   // activation scale rows, one per token
  if ((s = check_shape(c, N, K)) != HQ_OK) return s;
  if (R < 0 || R > kMaxDim || E <= 0 || E > 512)
    return fail(HQ_ERR_INVALID_ARGUMENT, "R=%lld E=%d out of range", (long long)R, E);
  if (R * N >= (int64_t(1) << 31)) return fail(HQ_ERR_UNSUPPORTED, "R*N must stay below 2^31");
  if (per_token && !a_scale)
    return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale ([R], or [R, K/128] for block-scaled FP8) is required for INT8/FP8 activations");
  if (!per_token && a_scale) return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale must be NULL for BF16 activations");
  if (!a || !w_packed || !expert_offsets || !y)
    return fail(HQ_ERR_INVALID_ARGUMENT, "a, w_packed, expert_offsets and y must be non-NULL");
  if (!aligned16(a) || !aligned16(w_packed) || !aligned16(y))
    return fail(HQ_ERR_INVALID_ARGUMENT, "a, w_packed and y must be 16-byte aligned");
  if (R == 0) return ok();
  const GroupedWs g = grouped_ws(c, R, E, N, K);
  if (!ws || ws_bytes < g.total) return fail(HQ_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, g.total);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(HQ_ERR_INVALID_ARGUMENT, "ws must be 256-byte aligned");
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + g.sorted_off);
  int32_t* bexp = reinterpret_cast<int32_t*>(base + g.bexp_off);
  int32_t* npad = reinterpret_cast<int32_t*>(base + g.npad_off);
  if ((s = check_hip(hq::launch_grouped_index(expert_offsets, R, E, g.bm, int64_t(g.cap), sorted, bexp, npad,
                                              static_cast<hipStream_t>(stream)),
                     "hq_grouped_gemm row index launch")) != HQ_OK)
    return s;
  return hq_moe_grouped_gemm(desc, R, 1, E, N, K, a, a_scale, w_packed, sorted, bexp, npad, g.bm, nullptr, y,
                             g.gemm_bytes ? base + g.gemm_off : nullptr, g.gemm_bytes, stream);
}

hq_status hq_moe_silu_mul(int64_t R, int64_t I, const void* gate_up, void* act, hq_stream_t stream) {
  if (R < 0 || R > kMaxDim || I <= 0 || I > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "R=%lld I=%lld out of range", (long long)R, (long long)I);
  if (I % 8 != 0) return fail(HQ_ERR_UNSUPPORTED, "I=%lld must be a multiple of 8", (long long)I);
  if (R * I > (int64_t(1) << 40)) return fail(HQ_ERR_UNSUPPORTED, "R*I must stay below 2^40");
  if (R == 0) return ok();
  if (!gate_up || !act) return fail(HQ_ERR_INVALID_ARGUMENT, "gate_up and act must be non-NULL");
  if (!aligned16(gate_up) || !aligned16(act))
    return fail(HQ_ERR_INVALID_ARGUMENT, "gate_up and act must be 16-byte aligned");
  return check_hip(hq::launch_silu_mul(R, I, gate_up, act, static_cast<hipStream_t>(stream)),
                   "hq_moe_silu_mul launch");
}

hq_status hq_moe_silu_mul_quantize(int32_t act_fmt, int64_t R, int64_t I, const void* gate_up, void* act_q,
                                   float* act_scale, hq_stream_t stream) {
  if (act_fmt != HQ_ACT_INT8_PER_TOKEN && act_fmt != HQ_ACT_FP8E4M3_PER_TOKEN)
    return fail(HQ_ERR_UNSUPPORTED, "act_fmt=%d: INT8 or FP8 e4m3 per token", act_fmt);
  if (R < 0 || R > kMaxDim || I <= 0 || I > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "R=%lld I=%lld out of range", (long long)R, (long long)I);
  if (I % 8 != 0) return fail(HQ_ERR_UNSUPPORTED, "I=%lld must be a multiple of 8", (long long)I);
  if (R * I > (int64_t(1) << 40)) return fail(HQ_ERR_UNSUPPORTED, "R*I must stay below 2^40");
  if (R == 0) return ok();
  if (!gate_up || !act_q || !act_scale)
    return fail(HQ_ERR_INVALID_ARGUMENT, "gate_up, act_q and act_scale must be non-NULL");
  if (!aligned16(gate_up) || !aligned16(act_q) || (reinterpret_cast<uintptr_t>(act_scale) & 3u))
    return fail(HQ_ERR_INVALID_ARGUMENT, "gate_up and act_q must be 16-byte aligned, act_scale 4-byte aligned");
  return check_hip(hq::launch_silu_mul_quant(act_fmt, R, I, gate_up, act_q, act_scale, static_cast<hipStream_t>(stream)),
                   "hq_moe_silu_mul_quantize launch");
}

hq_status hq_moe_combine(int64_t T, int32_t topk, int32_t E, int64_t N, const int32_t* topk_ids,
                         const void* y, void* out, hq_stream_t stream) {
  if (T < 0 || T > kMaxDim || topk <= 0 || topk > 64 || E <= 0 || N <= 0 || N > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "T=%lld topk=%d E=%d N=%lld out of range", (long long)T, topk, E,
                (long long)N);
  if (N % 8 != 0) return fail(HQ_ERR_UNSUPPORTED, "N=%lld must be a multiple of 8", (long long)N);
  if (T * N > (int64_t(1) << 40)) return fail(HQ_ERR_UNSUPPORTED, "T*N must stay below 2^40");
  if (T == 0) return ok();
  if (!topk_ids || !y || !out) return fail(HQ_ERR_INVALID_ARGUMENT, "topk_ids, y and out must be non-NULL");
  if (!aligned16(y) || !aligned16(out)) return fail(HQ_ERR_INVALID_ARGUMENT, "y and out must be 16-byte aligned");
  return check_hip(hq::launch_moe_combine(T, topk, E, N, topk_ids, y, out, static_cast<hipStream_t>(stream)),
                   "hq_moe_combine launch");
}

int32_t hq_moe_block_m(const hq_quant_desc* desc, int64_t T, int32_t topk, int32_t E, int64_t N,
                       int64_t K) {
  hq::Combo c{};
  if (resolve(desc, &c) != HQ_OK || T < 0 || topk <= 0 || E <= 0) return 0;
  return hq::moe_block_m(c, T, topk, E, N, K);
}

size_t hq_moe_gemm_workspace_bytes(const hq_quant_desc* desc, int64_t T, int32_t topk, int32_t E,
                                   int64_t N, int64_t K, int32_t block_m) {
  hq::Combo c{};
  if (resolve(desc, &c) != HQ_OK || check_shape(c, N, K) != HQ_OK) return 0;
  return hq::plan_moe(c, T, topk, E, N, K, block_m).ws_bytes;
}

hq_status hq_moe_grouped_gemm(const hq_quant_desc* desc, int64_t T, int32_t topk, int32_t E,
                              int64_t N, int64_t K, const void* a, const float* a_scale,
                              const void* w_packed, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              int32_t block_m, const float* topk_weights, void* y, void* ws,
                              size_t ws_bytes, hq_stream_t stream) {
  hq::Combo c{};
  hq_status s = resolve(desc, &c);
  if (s != HQ_OK) return s;
  if (c.out_i32) return fail(HQ_ERR_UNSUPPORTED, "MoE grouped GEMM writes bf16 only");
  const bool per_token = !hq::family_bf16_act(c.fam);   // activation scale rows, one per token
  if ((s = check_shape(c, N, K)) != HQ_OK) return s;
  if (T < 0 || topk <= 0 || topk > 64 || E <= 0 || E > 512)
    return fail(HQ_ERR_INVALID_ARGUMENT, "T=%lld topk=%d E=%d out of range", (long long)T, topk, E);
  if (T * topk * N >= (int64_t(1) << 31))
    return fail(HQ_ERR_UNSUPPORTED, "T*topk*N must stay below 2^31");
  if (!hq::moe_block_m_supported(block_m))
    return fail(HQ_ERR_UNSUPPORTED, "block_m=%d: supported values are 16, 32, 64, 128", block_m);
  if (c.invariant && block_m != 32)
    return fail(HQ_ERR_INVALID_ARGUMENT, "block_m=%d: batch-invariant MoE calls use block_m 32", block_m);
  if (per_token && !a_scale)
    return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale ([T], or [T, K/128] for block-scaled FP8) is required for INT8/FP8 activations");
  if (!per_token && a_scale) return fail(HQ_ERR_INVALID_ARGUMENT, "a_scale must be NULL for BF16 activations");
  if (!a || !w_packed || !sorted_ids || !block_expert || !num_padded || !y)
    return fail(HQ_ERR_INVALID_ARGUMENT, "a, w_packed, sorted_ids, block_expert, num_padded and y must be non-NULL");
  if (!aligned16(a) || !aligned16(w_packed) || !aligned16(y))
    return fail(HQ_ERR_INVALID_ARGUMENT, "a, w_packed and y must be 16-byte aligned");
  if (T == 0) return ok();
  const hq::Plan plan = hq::plan_moe(c, T, topk, E, N, K, block_m);
  if (plan.kind < 0)
    return fail(HQ_ERR_UNSUPPORTED, "block_m=%d: no kernel configuration fits N=%lld K=%lld (128-row blocks need K %% 128 == 0 and N %% 128 == 0), or the HQ_TUNE override does not fit",
                block_m, (long long)N, (long long)K);
  if (ws_bytes < plan.ws_bytes || (plan.ws_bytes && !ws))
    return fail(HQ_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, plan.ws_bytes);
  if (ws && !aligned16(ws)) return fail(HQ_ERR_INVALID_ARGUMENT, "ws must be 16-byte aligned");
  hq::GemmCall call{};
  call.c = c;
  call.M = T * topk;
  call.N = N;
  call.K = K;
  call.a = a;
  call.a_scale = a_scale;
  call.w = static_cast<const uint8_t*>(w_packed);
  call.y = y;
  call.ws = ws;
  call.ws_bytes = ws_bytes;
  call.stream = static_cast<hipStream_t>(stream);
  call.sorted_ids = sorted_ids;
  call.block_expert = block_expert;
  call.num_padded = num_padded;
  call.topk_weights = topk_weights;
  call.T = T;
  call.topk = topk;
  call.E = E;
  call.block_m = block_m;
  call.max_blocks = int64_t(hq_moe_align_capacity(T, topk, E, block_m)) / block_m;
  return check_hip(hq::launch_gemm(call, plan), "hq_moe_grouped_gemm launch");
}

}  // extern "C"
