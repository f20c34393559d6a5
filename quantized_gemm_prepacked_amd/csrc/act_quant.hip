// act_quant.hip -- per-token dynamic quantization of bf16 activations for the W8A8 and W4A8
// GEMMs: one fp32 scale per row and INT8 or OCP e4m3 codes.
//
// The Humming announcement lists per-token input scales among the compute options (section
// "Tuning and JIT compilation per workload") and attributes its end-to-end gain to tokenwise FP8
// activations (section "End-to-end performance"); the rule here is symmetric absmax scaling:
//   s = fp32(max_k |x| / Q) (Q = 127 or 448; 1 for an all-zero row), v = fp32(x / s) (IEEE
//   binary32 division), INT8 q = clamp(rne(v), -127, 127), e4m3 q = rne_e4m3(clamp(v, +-448)).
// One workgroup per row: a pass for the row maximum (wave then LDS reduction), a pass that
// re-reads the row (from cache) and writes 8 codes per lane per step.
//
// MXFP4 activations (W4A4) follow the OCP Microscaling rule per block of 32 k instead: shared
// exponent e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for a zero block), e8m0 byte
// e + 127, codes = nearest e2m1 to x * 2^-e with ties to even, saturating at 6, sign only on a
// non-zero magnitude. One thread per block; every decision is exact (integer maximum of the bf16
// magnitudes, exponent from the bits, a power-of-two scaling, comparisons with the e2m1
// midpoints), so no denormal mode or rounding mode can change a code.
#include <hip/hip_runtime.h>

#include "device_ops.h"
#include "elementwise_ops.h"
#include "internal.h"

namespace hq {

namespace {

constexpr int kThreads = 256;

// fp32 -> OCP e4m3 ("fn") code, round to nearest even, for |v| <= 448 (the caller clamps). The
// sign is kept, so values that round to zero give +-0 (0x00 / 0x80).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {
    // below 2^-6: subnormal codes m * 2^-9 (m = 8 is the smallest normal, code 0x08); the
    // scaling by 2^9 is exact
    code = uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
  } else {
    // normal: exponent field (fp32 exponent + 7, 1..15) and the top three mantissa bits,
    // rounded on the 20 dropped bits (a carry moves into the exponent)
    const uint32_t e = (a >> 23) - 120u;
    const uint32_t m = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    code = (e << 3) | m;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) code += 1u;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// The eight codes of eight bf16 inputs (four packed pairs) at scale s, as two dwords.
template <int ACT>
__device__ __forceinline__ uint2 quant8(const u32x4& v, float s) {
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t bits = (j & 1) ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16);
    const float q = __uint_as_float(bits) / s;
    uint32_t code;
    if constexpr (ACT == HQ_ACT_INT8_PER_TOKEN) {
      code = uint32_t(int(fminf(fmaxf(__builtin_rintf(q), -127.0f), 127.0f))) & 0xFFu;
    } else {
      code = e4m3_rne(fminf(fmaxf(q, -448.0f), 448.0f));
    }
    out[j >> 2] |= code << (8 * (j & 3));
  }
  return make_uint2(out[0], out[1]);
}

__device__ __forceinline__ float absmax8(float amax, const u32x4& v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = fmaxf(amax, fabsf(__uint_as_float(v[j] << 16)));
    amax = fmaxf(amax, fabsf(__uint_as_float(v[j] & 0xFFFF0000u)));
  }
  return amax;
}

// The row maximum over the workgroup (wave shuffles, then LDS), and the row's scale.
template <int ACT>
__device__ __forceinline__ float row_scale(float amax) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
  float s = amax / (ACT == HQ_ACT_INT8_PER_TOKEN ? 127.0f : 448.0f);
  return s == 0.0f ? 1.0f : s;
}

template <int ACT>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ xq,
                                                             float* __restrict__ s_tok, int K) {
  const int row = blockIdx.x;
  const uint16_t* xr = x + size_t(row) * K;
  uint8_t* qr = xq + size_t(row) * K;
  float amax = 0.0f;
  for (int i = threadIdx.x * 8; i < K; i += kThreads * 8) amax = absmax8(amax, ldg16(xr + i));
  const float s = row_scale<ACT>(amax);
  if (threadIdx.x == 0) s_tok[row] = s;
  for (int i = threadIdx.x * 8; i < K; i += kThreads * 8)
    *reinterpret_cast<uint2*>(qr + i) = quant8<ACT>(ldg16(xr + i), s);
}

// Eight gated activations bf16(silu(g) * u) of a gate_up row [g (I) | u (I)] at column i,
// computed exactly as the SiLU-gated activation kernel of the MoE layer does.
__device__ __forceinline__ u32x4 gated8(const uint16_t* gr, int I, int i) {
  const u32x4 g = ldg16(gr + i);
  const u32x4 u = ldg16(gr + I + i);
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a0 = silu(__uint_as_float(g[j] << 16)) * __uint_as_float(u[j] << 16);
    const float a1 = silu(__uint_as_float(g[j] & 0xFFFF0000u)) * __uint_as_float(u[j] & 0xFFFF0000u);
    out[j] = uint32_t(f32_to_bf16_rne(a0)) | (uint32_t(f32_to_bf16_rne(a1)) << 16);
  }
  return out;
}

// The gated activation of a row quantized per row: the same chunks per thread as act_quant_kernel
// (column tid * 8 + c * 2048), the first kKeep chunks computed once and kept in registers between
// the maximum and the quantization, any further ones (I > 8192) computed again.
template <int ACT>
__global__ __launch_bounds__(kThreads) void silu_quant_kernel(const uint16_t* __restrict__ gu,
                                                              uint8_t* __restrict__ aq,
                                                              float* __restrict__ s_out, int I) {
  constexpr int kKeep = 4;
  const int row = blockIdx.x;
  const uint16_t* gr = gu + size_t(row) * 2 * I;
  uint8_t* qr = aq + size_t(row) * I;
  u32x4 a[kKeep];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kKeep; ++c) {
    const int i = (c * kThreads + threadIdx.x) * 8;
    if (i < I) {
      a[c] = gated8(gr, I, i);
      amax = absmax8(amax, a[c]);
    }
  }
  for (int i = (kKeep * kThreads + threadIdx.x) * 8; i < I; i += kThreads * 8) amax = absmax8(amax, gated8(gr, I, i));
  const float s = row_scale<ACT>(amax);
  if (threadIdx.x == 0) s_out[row] = s;
#pragma unroll
  for (int c = 0; c < kKeep; ++c) {
    const int i = (c * kThreads + threadIdx.x) * 8;
    if (i < I) *reinterpret_cast<uint2*>(qr + i) = quant8<ACT>(a[c], s);
  }
  for (int i = (kKeep * kThreads + threadIdx.x) * 8; i < I; i += kThreads * 8)
    *reinterpret_cast<uint2*>(qr + i) = quant8<ACT>(gated8(gr, I, i), s);
}

// e2m1 magnitude code of a >= 0 (exact binary32), ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
         uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
}

__global__ __launch_bounds__(kThreads) void act_quant_mxfp4_kernel(const uint16_t* __restrict__ x,
                                                                   uint8_t* __restrict__ xq,
                                                                   uint8_t* __restrict__ xs,
                                                                   int64_t n_blocks) {
  const int64_t b = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (b >= n_blocks) return;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ldg16(x + b * 32 + 8 * i);
  uint32_t amax = 0;   // largest |x| as bf16 bits: the bit order of non-negative values
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = max(amax, max(v[i][j] & 0x7FFFu, (v[i][j] >> 16) & 0x7FFFu));
  const int ef = int(amax >> 7);                      // bf16 exponent field (0: zero or subnormal)
  const int e = ef == 0 ? -127 : max(ef - 127 - 2, -127);
  xs[b] = uint8_t(e + 127);
  const float inv = __uint_as_float(uint32_t(127 - e) << 23);   // 2^-e, e in [-127, 125]
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = (v[i][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t mag = h & 0x7FFFu;
      // a subnormal bf16 magnitude is mag * 2^-133, so v = mag * 2^(-133 - e): exact while that
      // power of two is a normal binary32 number (e <= -7); past it v < 2^-120 rounds to zero
      const float a = (mag >> 7) != 0 ? __uint_as_float(mag << 16) * inv
                      : e <= -7      ? float(mag) * __uint_as_float(uint32_t(-6 - e) << 23)
                                     : 0.0f;
      const uint32_t c = e2m1_code(a);
      word |= (c | (((h >> 15) & uint32_t(c != 0u)) << 3)) << (4 * j);
    }
    out[i] = word;
  }
  *reinterpret_cast<u32x4*>(xq + b * 16) = u32x4{out[0], out[1], out[2], out[3]};
}

// MXFP8 activations: the same block rule with e4m3 elements (largest exponent 8), codes by the
// per-token path's e4m3 encoder on clamp(x * 2^-e, -448, 448); the sign is kept (-0 = 0x80).
__global__ __launch_bounds__(kThreads) void act_quant_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                                   uint8_t* __restrict__ xq,
                                                                   uint8_t* __restrict__ xs,
                                                                   int64_t n_blocks) {
  const int64_t b = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (b >= n_blocks) return;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ldg16(x + b * 32 + 8 * i);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = max(amax, max(v[i][j] & 0x7FFFu, (v[i][j] >> 16) & 0x7FFFu));
  const int ef = int(amax >> 7);
  const int e = ef == 0 ? -127 : max(ef - 127 - 8, -127);
  xs[b] = uint8_t(e + 127);
  const float inv = __uint_as_float(uint32_t(127 - e) << 23);   // 2^-e, e in [-127, 119]
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * h2 + j;                      // element k of the 8 in v[i]
        const uint32_t h = (v[i][k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
        const uint32_t mag = h & 0x7FFFu;
        const float a = (mag >> 7) != 0 ? __uint_as_float(mag << 16) * inv
                        : e <= -7      ? float(mag) * __uint_as_float(uint32_t(-6 - e) << 23)
                                       : 0.0f;
        const float sv = __uint_as_float(__float_as_uint(fminf(a, 448.0f)) | ((h & 0x8000u) << 16));
        word |= e4m3_rne(sv) << (8 * j);
      }
      out[2 * i + h2] = word;
    }
  uint32_t* dst = reinterpret_cast<uint32_t*>(xq + b * 32);
  *reinterpret_cast<u32x4*>(dst) = u32x4{out[0], out[1], out[2], out[3]};
  *reinterpret_cast<u32x4*>(dst + 4) = u32x4{out[4], out[5], out[6], out[7]};
}

// FP8 activations with a scale per (row, 128-k block), for the block-scaled FP8 W8A8: the
// per-token rule on each block -- s = fp32(amax / 448) (1 for a zero block), codes = e4m3 of
// clamp(fp32(x / s), +-448). Sixteen lanes per block, eight elements per lane; the block maximum
// by shuffles within the sixteen lanes.
__global__ __launch_bounds__(kThreads) void act_quant_fp8block_kernel(const uint16_t* __restrict__ x,
                                                                      uint8_t* __restrict__ xq,
                                                                      float* __restrict__ xs,
                                                                      int64_t n_groups) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;   // 8-element group index
  const bool live = i < n_groups;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (live) v = ldg16(x + i * 8);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = fmaxf(amax, fabsf(__uint_as_float(v[j] << 16)));
    amax = fmaxf(amax, fabsf(__uint_as_float(v[j] & 0xFFFF0000u)));
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  float s = amax / 448.0f;
  if (s == 0.0f) s = 1.0f;
  if (!live) return;
  if ((i & 15) == 0) xs[i >> 4] = s;
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t bits = (j & 1) ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16);
    const float q = __uint_as_float(bits) / s;
    out[j >> 2] |= e4m3_rne(fminf(fmaxf(q, -448.0f), 448.0f)) << (8 * (j & 3));
  }
  *reinterpret_cast<uint2*>(xq + i * 8) = make_uint2(out[0], out[1]);
}

}  // namespace

hipError_t launch_act_quant(int act_fmt, int64_t M, int64_t K, const void* x, void* xq, float* s_tok,
                            hipStream_t stream) {
  const dim3 grid{static_cast<unsigned>(M)};
  const auto* xin = static_cast<const uint16_t*>(x);
  auto* out = static_cast<uint8_t*>(xq);
  if (act_fmt == HQ_ACT_FP8E4M3_BLOCK128) {
    const int64_t ng = M * (K / 8);   // a multiple of 16: K % 128 == 0
    hipLaunchKernelGGL(act_quant_fp8block_kernel, dim3(unsigned((ng + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, xin, out, s_tok, ng);
    return hipGetLastError();
  }
  if (act_fmt == HQ_ACT_MXFP8) {
    const int64_t nb = M * (K / 32);
    hipLaunchKernelGGL(act_quant_mxfp8_kernel, dim3(unsigned((nb + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, xin, out, reinterpret_cast<uint8_t*>(s_tok), nb);
    return hipGetLastError();
  }
  if (act_fmt == HQ_ACT_MXFP4) {
    const int64_t nb = M * (K / 32);
    hipLaunchKernelGGL(act_quant_mxfp4_kernel, dim3(unsigned((nb + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, xin, out, reinterpret_cast<uint8_t*>(s_tok), nb);
    return hipGetLastError();
  }
  if (act_fmt == HQ_ACT_INT8_PER_TOKEN)
    hipLaunchKernelGGL(act_quant_kernel<HQ_ACT_INT8_PER_TOKEN>, grid, dim3(kThreads), 0, stream, xin, out, s_tok, int(K));
  else
    hipLaunchKernelGGL(act_quant_kernel<HQ_ACT_FP8E4M3_PER_TOKEN>, grid, dim3(kThreads), 0, stream, xin, out, s_tok, int(K));
  return hipGetLastError();
}

hipError_t launch_silu_mul_quant(int act_fmt, int64_t R, int64_t I, const void* gate_up, void* act_q,
                                 float* act_scale, hipStream_t stream) {
  const dim3 grid{static_cast<unsigned>(R)};
  const auto* gu = static_cast<const uint16_t*>(gate_up);
  auto* out = static_cast<uint8_t*>(act_q);
  if (act_fmt == HQ_ACT_INT8_PER_TOKEN)
    hipLaunchKernelGGL(silu_quant_kernel<HQ_ACT_INT8_PER_TOKEN>, grid, dim3(kThreads), 0, stream, gu, out,
                       act_scale, int(I));
  else
    hipLaunchKernelGGL(silu_quant_kernel<HQ_ACT_FP8E4M3_PER_TOKEN>, grid, dim3(kThreads), 0, stream, gu, out,
                       act_scale, int(I));
  return hipGetLastError();
}

}  // namespace hq
