// moe_layer.hip -- the two elementwise stages that turn the grouped GEMMs into an MoE layer:
// the SiLU-gated activation between gate_up and Down, and the top-k combine after Down.
//
// The Humming announcement times MoE layers as gate_up plus Down (section "Results: kernel
// microbenchmarks"); the expert MLP in between is the usual gated one: for each routed row the
// first half of the gate_up output is the gate g, the second half the up projection u, and the
// Down GEMM consumes silu(g) * u. The router weights are applied in the Down GEMM's epilogue, so
// the combine only sums a token's top-k rows.
#include <hip/hip_runtime.h>

#include "device_ops.h"
#include "elementwise_ops.h"
#include "internal.h"

namespace hq {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// act[r, i] = bf16(silu(g) * u), g = gu[r, i], u = gu[r, I + i]; 8 outputs per thread.
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(const uint16_t* __restrict__ gu,
                                                            uint16_t* __restrict__ act, int64_t R,
                                                            int I) {
  const int64_t per_row = I / 8;
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= R * per_row) return;
  const int64_t r = idx / per_row;
  const int c = int(idx % per_row) * 8;
  const u32x4 g = ldg16(gu + r * 2 * I + c);
  const u32x4 u = ldg16(gu + r * 2 * I + I + c);
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float g0 = bf16_lo(g[j]), g1 = bf16_hi(g[j]);
    const float a0 = silu(g0) * bf16_lo(u[j]);
    const float a1 = silu(g1) * bf16_hi(u[j]);
    out[j] = uint32_t(f32_to_bf16_rne(a0)) | (uint32_t(f32_to_bf16_rne(a1)) << 16);
  }
  *reinterpret_cast<u32x4*>(act + r * I + c) = out;
}

// out[t, n] = bf16(sum_k y[t*topk + k, n]) over the k routed to an expert in [0, E), fp32 sum in
// k order; 8 outputs per thread.
__global__ __launch_bounds__(kThreads) void moe_combine_kernel(const uint16_t* __restrict__ y,
                                                               const int32_t* __restrict__ ids,
                                                               uint16_t* __restrict__ out, int64_t T,
                                                               int topk, int E, int N) {
  const int64_t per_row = N / 8;
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int c = int(idx % per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < topk; ++k) {
    const int e = ids[t * topk + k];
    if (e < 0 || e >= E) continue;
    const u32x4 v = ldg16(y + (t * topk + k) * N + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_lo(v[j]);
      acc[2 * j + 1] += bf16_hi(v[j]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = uint32_t(f32_to_bf16_rne(acc[2 * j])) | (uint32_t(f32_to_bf16_rne(acc[2 * j + 1])) << 16);
  *reinterpret_cast<u32x4*>(out + t * N + c) = o;
}

}  // namespace

hipError_t launch_silu_mul(int64_t R, int64_t I, const void* gate_up, void* act, hipStream_t s) {
  const int64_t n = R * (I / 8);
  const dim3 grid{static_cast<unsigned>((n + kThreads - 1) / kThreads)};
  hipLaunchKernelGGL(silu_mul_kernel, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(gate_up),
                     static_cast<uint16_t*>(act), R, int(I));
  return hipGetLastError();
}

hipError_t launch_moe_combine(int64_t T, int32_t topk, int32_t E, int64_t N, const int32_t* topk_ids,
                              const void* y, void* out, hipStream_t s) {
  const int64_t n = T * (N / 8);
  const dim3 grid{static_cast<unsigned>((n + kThreads - 1) / kThreads)};
  hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(y),
                     topk_ids, static_cast<uint16_t*>(out), T, int(topk), int(E), int(N));
  return hipGetLastError();
}

}  // namespace hq
