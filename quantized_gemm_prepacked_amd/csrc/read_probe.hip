// read_probe.hip -- a streaming-read kernel that measures how fast one kernel can read a fresh
// buffer from HBM on this GPU: the practical ceiling of a decode (M = 1) GEMM, which must stream
// its packed weights once. Not part of the GEMM library: built into its own libhq_probe.so and
// used by quantized_gemm_prepacked_amd/ceilings.py.
//
// Each thread issues up to 16 independent 16-byte non-temporal loads (grid-stride) before it uses
// any of them, so a launch of a few thousand workgroups has the whole buffer in flight at once,
// and folds them with XOR; one dword per workgroup goes to `sink` so the loads cannot be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int kUnroll = 16;
  uint32_t x = 0;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < int(blockDim.x); ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned device pointer) with `wgs` workgroups of 256
// threads; `sink` receives one dword per workgroup. Returns a hipError_t.
extern "C" int hqp_stream_read(const void* src, size_t bytes, void* sink, int wgs, void* stream) {
  if (!src || !sink || bytes % 16 || wgs <= 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(wgs)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return int(hipGetLastError());
}
