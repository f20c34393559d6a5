// elementwise_ops.h -- device helpers shared by the MoE layer's elementwise kernels and the
// activation quantizers (the gated activation feeds a quantizer when the Down GEMM takes 8-bit
// activations, and both paths must produce the same bits).
#pragma once
#include <hip/hip_runtime.h>

namespace hq {

// silu(g) = g * sigmoid(g), with sigmoid(g) = 1 / (1 + e) for g >= 0 and e / (1 + e) for g < 0,
// e = exp(-|g|): e never overflows, so a very negative gate keeps its tiny product instead of
// dividing by an infinite exp(-g).
__device__ __forceinline__ float silu(float g) {
  const float e = expf(-fabsf(g));
  return g * ((g >= 0.0f ? 1.0f : e) / (1.0f + e));
}

}  // namespace hq
