// read_probe.hip -- a streaming-read kernel that measures how fast one kernel can read a fresh
// buffer from HBM on this GPU: the practical ceiling of a decode (M = 1) GEMM, which must stream
// its packed weights once. Not part of the GEMM library: built into its own libhq_probe.so and
// used by quantized_gemm_prepacked_amd/ceilings.py.
//
// Two ways of dealing the buffer's 16-byte chunks to the threads, and a depth L of 1, 4 or 16: a
// thread issues L of its chunks as independent non-temporal loads, then uses them, then the next L
// (L = 1: one load in flight per thread, latency hidden by the number of waves only):
// Workgroups of 256 or 1024 threads.
//   grid-stride  thread i of the grid reads chunks i, i + S, i + 2S, ... (S = the grid's thread
//                count): each round of the grid reads S consecutive chunks;
//   blocked      workgroup b reads its own contiguous share of the buffer (a multiple of 1 KiB),
//                its threads consecutive chunks of it in each round.
// With L = 16 and at least n / (16 * 256) workgroups of 256 the whole buffer is in flight at once. The
// best of these is the figure to quote: more bytes in flight is not always faster. The loaded words
// are folded with XOR (per wave with shuffles, so the fold adds no serial tail) and one dword per
// workgroup goes to `sink`, so the loads cannot be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kBlocked, int kLoads>
__global__ __launch_bounds__(1024) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  size_t first, step, end;
  if constexpr (kBlocked) {
    const size_t share = ((n16 + gridDim.x - 1) / gridDim.x + 63) / 64 * 64;
    first = size_t(blockIdx.x) * share + threadIdx.x;
    end = min(n16, size_t(blockIdx.x + 1) * share);
    step = blockDim.x;
  } else {
    first = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    end = n16;
    step = size_t(gridDim.x) * blockDim.x;
  }
  uint32_t x = 0;
  for (size_t i = first; i < end; i += kLoads * step) {
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const size_t j = i + u * step;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // fold the workgroup's words: across each wave with shuffles, then one word per wave
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t red[16];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

template <bool kBlocked>
void launch(int loads, dim3 grid, dim3 block, hipStream_t st, const u32x4* s16, size_t n16, uint32_t* out) {
  if (loads == 1) hipLaunchKernelGGL((stream_read_kernel<kBlocked, 1>), grid, block, 0, st, s16, n16, out);
  else if (loads == 4) hipLaunchKernelGGL((stream_read_kernel<kBlocked, 4>), grid, block, 0, st, s16, n16, out);
  else hipLaunchKernelGGL((stream_read_kernel<kBlocked, 16>), grid, block, 0, st, s16, n16, out);
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned device pointer) with `wgs` workgroups of
// `threads` (256 or 1024) threads, grid-stride (blocked = 0) or a contiguous share per workgroup (blocked = 1), `loads`
// (1, 4 or 16) loads in flight per thread; `sink` receives one dword per workgroup. Returns a
// hipError_t.
extern "C" int hqp_stream_read(const void* src, size_t bytes, void* sink, int wgs, int threads, int blocked,
                               int loads, void* stream) {
  if (!src || !sink || bytes % 16 || wgs <= 0 || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (threads != 256 && threads != 1024) || (loads != 1 && loads != 4 && loads != 16))
    return int(hipErrorInvalidValue);
  const dim3 grid{unsigned(wgs)}, block{unsigned(threads)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s16 = static_cast<const u32x4*>(src);
  uint32_t* out = static_cast<uint32_t*>(sink);
  if (blocked) launch<true>(loads, grid, block, st, s16, bytes / 16, out);
  else launch<false>(loads, grid, block, st, s16, bytes / 16, out);
  return int(hipGetLastError());
}
