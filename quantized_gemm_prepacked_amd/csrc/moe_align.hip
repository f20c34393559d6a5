// moe_align.hip -- MoE token sort / expert offsets on the device, one launch, no host sync.
//
// Feeds the "Indexed" MoE path (rows gathered through a sorted index) of the Humming
// announcement's section "Results: kernel microbenchmarks". The token sort itself is not
// described there; the contract (stable ascending order per expert, per-expert padding to a
// multiple of block_m with sentinel T*topk) is the library's (hq.h).
//
// Workgroups of 1024 threads, each owning a contiguous range of whole tiles of 1024 entries of the
// flat id list (up to 128 workgroups, so the scatter is spread over the GPU). Every workgroup
// (1) builds the per-expert histogram of the whole list with LDS atomics (order-free), counting
// apart the entries before its own range, (2) scans the padded counts block-wide (wave shuffles,
// then over the wave totals) -- the same offsets in every workgroup, from the same counts --
// (3) scatters its own range stably, one tile at a time: inside a wave, entries of the same
// expert are found with ballots over the expert id bits and ranked by lane; across the 16 waves
// of a tile, per-wave counts are prefix-summed in wave order; across tiles a running count per
// expert carries on, starting from the expert's count before the range. Every position is
// therefore a pure function of the input, independent of scheduling, and the workgroups write
// disjoint positions; the padding slots, the block -> expert table and the offsets are dealt
// out between them the same way. The ids are read in chunks of 8 tiles, each thread issuing its
// 8 loads together and keeping them in registers, so a chunk costs one memory latency rather
// than eight; when the first workgroup's range holds the whole first chunk (8192 entries, e.g.
// 1024 tokens at top-8) it reuses the histogram's registers for its scatter.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "hq.h"
#include "internal.h"

namespace hq {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kIdBits = 11;  // expert ids < 2048; id E marks an unrouted entry
constexpr int kPer = 8;      // ids each thread holds in registers: one chunk = kPer tiles of kThreads

// Entries [c0, c0 + kPer * kThreads) of the flat id list, thread tid holding c0 + j * kThreads + tid
// in e[j] (-1 past the end); all loads issued before any is used.
__device__ void load_chunk(const int32_t* __restrict__ ids, int n_flat, int c0, int (&e)[kPer]) {
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = c0 + j * kThreads + int(threadIdx.x);
    e[j] = i < n_flat ? ids[i] : -1;
  }
}

// Inclusive prefix sum of v over the kThreads threads of the workgroup, in thread order:
// shuffles inside each wave, then over the kWaves wave totals in wave 0. tmp: 2 * kWaves ints of
// LDS, not touched by the caller between the call and its return. Two barriers.
__device__ int block_inclusive_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int t = __shfl_up(w, off, 64);
      if (lane >= off) w += t;
    }
    if (lane < kWaves) tmp[kWaves + lane] = w;   // total of waves 0 .. lane
  }
  __syncthreads();
  return wave > 0 ? v + tmp[kWaves + wave - 1] : v;
}

__global__ __launch_bounds__(kThreads) void moe_align_kernel(const int32_t* __restrict__ ids,
                                                             int n_flat, int E, int bm,
                                                             int32_t* __restrict__ sorted,
                                                             int32_t* __restrict__ block_expert,
                                                             int32_t* __restrict__ offsets_out,
                                                             int32_t* __restrict__ num_padded,
                                                             int max_blocks, int range) {
  extern __shared__ int sm[];
  int* cnt = sm;               // [E]
  int* offs = cnt + E;         // [E + 1]
  int* run = offs + E + 1;     // [E] entries of expert e before the current tile
  int* scan = run + E;         // [2 * kWaves], the scan's wave totals
  int* wc = scan + 2 * kWaves; // [kWaves][E]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wg = blockIdx.x, nwg = gridDim.x;
  // this workgroup's entries: [r0, r1), whole tiles (range is a multiple of kThreads)
  const int r0 = min(n_flat, wg * range);
  const int r1 = min(n_flat, r0 + range);

  for (int e = tid; e < E; e += kThreads) {
    cnt[e] = 0;
    run[e] = 0;
  }
  for (int j = tid; j < kWaves * E; j += kThreads) wc[j] = 0;
  // The first chunk stays in registers for the scatter of the first workgroup when its range
  // holds all of the chunk's entries.
  const bool reuse_first = wg == 0 && r1 >= min(n_flat, kPer * kThreads);
  int ec[kPer];
  load_chunk(ids, n_flat, 0, ec);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (ec[j] >= 0 && ec[j] < E) {
      atomicAdd(&cnt[ec[j]], 1);
      if (j * kThreads + tid < r0) atomicAdd(&run[ec[j]], 1);
    }
  for (int c0 = kPer * kThreads; c0 < n_flat; c0 += kPer * kThreads) {
    int e[kPer];
    load_chunk(ids, n_flat, c0, e);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (e[j] >= 0 && e[j] < E) {
        atomicAdd(&cnt[e[j]], 1);
        if (c0 + j * kThreads + tid < r0) atomicAdd(&run[e[j]], 1);
      }
  }
  __syncthreads();

  // Exclusive scan of padded counts; E <= kThreads is checked on the host, E may be < kThreads.
  const int padded = tid < E ? (cnt[tid] + bm - 1) / bm * bm : 0;
  const int incl = block_inclusive_scan(padded, scan);
  if (tid < E) offs[tid] = incl - padded;
  if (tid == E - 1) offs[E] = incl;
  __syncthreads();
  const int total = offs[E];
  if (wg == 0) {
    for (int e = tid; e <= E; e += kThreads) offsets_out[e] = offs[e];
    if (tid == 0) *num_padded = total;
  }

  // Padding slots (expert e's by workgroup e mod nwg) and the block -> expert table (blocks dealt
  // out round robin).
  for (int e = wg + nwg * tid; e < E; e += nwg * kThreads)
    for (int s = offs[e] + cnt[e]; s < offs[e + 1]; ++s) sorted[s] = n_flat;
  for (int b = wg * kThreads + tid; b * bm < total; b += nwg * kThreads) {
    const int row = b * bm;
    int lo = 0, hi = E - 1;  // last e with offs[e] <= row (offs is non-decreasing)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= row) lo = mid; else hi = mid - 1;
    }
    block_expert[b] = lo;
  }
  // blocks past the sorted rows (up to the capacity) get no expert
  for (int b = (total + bm - 1) / bm + wg * kThreads + tid; b < max_blocks; b += nwg * kThreads)
    block_expert[b] = -1;

  // Stable scatter of [r0, r1), one tile of kThreads entries at a time. wc is zero at the start of
  // every tile: zeroed above, then by the running-count update that reads it.
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = r0; c0 < r1; c0 += kPer * kThreads) {
    if (!(c0 == 0 && reuse_first)) load_chunk(ids, r1, c0, ec);
#pragma unroll
    for (int jt = 0; jt < kPer; ++jt) {
      const int t0 = c0 + jt * kThreads;
      if (t0 >= r1) break;  // the same for every thread
      const int i = t0 + tid;
      const int e = ec[jt];
      const bool valid = e >= 0 && e < E;
      const int key = valid ? e : E;
      uint64_t same = ~0ull;
#pragma unroll
      for (int b = 0; b < kIdBits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
      }
      const int rank = __popcll(same & below);
      if (valid && rank == 0) wc[wave * E + e] = __popcll(same);
      __syncthreads();
      if (valid) {
        int base = run[e];
        for (int w = 0; w < wave; ++w) base += wc[w * E + e];
        sorted[offs[e] + base + rank] = i;
      }
      __syncthreads();
      for (int x = tid; x < E; x += kThreads) {
        int sum = 0;
        for (int w = 0; w < kWaves; ++w) {
          sum += wc[w * E + x];
          wc[w * E + x] = 0;
        }
        run[x] += sum;
      }
      __syncthreads();
    }
  }
}

// The same sort for at most 64 entries (a few tokens): one wave, one entry per lane. Lanes with the
// same expert are found with ballots over the expert id bits and ranked by lane (stable); the
// padded counts go to an LDS table indexed by expert and are prefix-summed by the wave (each lane
// a contiguous run of experts, then shuffles over the run totals); each entry's position is its
// expert's offset plus its rank, the first lane of each expert writes that expert's padding, and
// the block -> expert table is searched in the offsets. A few hundred instructions where the
// workgroup kernel above needs its LDS clears and about ten workgroup barriers.
__global__ __launch_bounds__(64) void moe_align_small_kernel(const int32_t* __restrict__ ids, int n_flat,
                                                              int E, int bm, int32_t* __restrict__ sorted,
                                                              int32_t* __restrict__ block_expert,
                                                              int32_t* __restrict__ offsets_out,
                                                              int32_t* __restrict__ num_padded, int max_blocks) {
  __shared__ int offs[513];   // padded count, then exclusive offset, per expert; offs[E] = total
  const int lane = threadIdx.x;
  const int e = lane < n_flat ? ids[lane] : -1;
  const bool valid = e >= 0 && e < E;
  const int key = valid ? e : E;
  uint64_t same = ~0ull;
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & below);
  const int cnt = __popcll(same);
  for (int x = lane; x <= E; x += 64) offs[x] = 0;
  __syncthreads();
  if (valid && rank == 0) offs[e] = (cnt + bm - 1) / bm * bm;
  __syncthreads();
  // exclusive scan of offs[0..E): lane l owns experts [l * per, (l + 1) * per)
  const int per = (E + 63) / 64;
  const int lo = min(E, lane * per), hi = min(E, lo + per);
  int run = 0;
  for (int x = lo; x < hi; ++x) run += offs[x];
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  const int total = __shfl(incl, 63, 64);
  __syncthreads();
  int acc = incl - run;
  for (int x = lo; x < hi; ++x) {
    const int padded = offs[x];
    offs[x] = acc;
    acc += padded;
  }
  if (lane == 0) offs[E] = total;
  __syncthreads();
  for (int x = lane; x <= E; x += 64) offsets_out[x] = offs[x];
  if (lane == 0) *num_padded = total;
  if (valid) {
    const int base = offs[e];
    sorted[base + rank] = lane;
    if (rank == 0)
      for (int s = base + cnt; s < offs[e + 1]; ++s) sorted[s] = n_flat;
  }
  for (int b = lane; b < max_blocks; b += 64) {
    const int row = b * bm;
    int v = -1;
    if (row < total) {
      int l = 0, h = E - 1;  // last expert with offs <= row (offs is non-decreasing)
      while (l < h) {
        const int mid = (l + h + 1) >> 1;
        if (offs[mid] <= row) l = mid; else h = mid - 1;
      }
      v = l;
    }
    block_expert[b] = v;
  }
}

// Row index of the "Grouped" path (rows already grouped by expert): expert e owns rows
// [offsets[e], offsets[e+1]) clipped to [0, R). The same outputs as the token sort -- each
// expert's rows padded to a multiple of bm with the sentinel R, the block -> expert table, -1
// for blocks past the padded rows, num_padded -- so the grouped GEMM kernels run unchanged with
// every row as its own token. Every workgroup rebuilds the (E <= 1024) padded prefix sum in LDS
// and fills positions [1024 * blockIdx.x, ...) of the capacity; positions never exceed cap, so
// offsets that overlap (outside the contract) give unspecified rows but no access out of bounds.
__global__ __launch_bounds__(kThreads) void grouped_index_kernel(const int32_t* __restrict__ offsets,
                                                                 int R, int E, int bm, int cap,
                                                                 int32_t* __restrict__ sorted,
                                                                 int32_t* __restrict__ block_expert,
                                                                 int32_t* __restrict__ num_padded) {
  __shared__ int lo_s[kThreads], cnt_s[kThreads], scan[kThreads], wtot[2 * kWaves];
  const int tid = threadIdx.x;
  int padded = 0;
  if (tid < E) {
    const int lo = min(max(offsets[tid], 0), R);
    const int hi = min(max(offsets[tid + 1], 0), R);
    lo_s[tid] = lo;
    cnt_s[tid] = max(hi - lo, 0);
    padded = (cnt_s[tid] + bm - 1) / bm * bm;
  }
  scan[tid] = block_inclusive_scan(padded, wtot);
  __syncthreads();
  const int total = min(scan[E - 1], cap);   // inclusive scan: scan[e] = end of expert e's range
  if (blockIdx.x == 0 && tid == 0) *num_padded = total;
  for (int pos = blockIdx.x * kThreads + tid; pos < cap; pos += gridDim.x * kThreads) {
    if (pos < total) {
      int lo = 0, hi = E - 1;   // first e whose range ends past pos
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (scan[mid] > pos) hi = mid; else lo = mid + 1;
      }
      const int i = pos - (scan[lo] - (cnt_s[lo] + bm - 1) / bm * bm);
      sorted[pos] = i < cnt_s[lo] ? lo_s[lo] + i : R;
      if (pos % bm == 0) block_expert[pos / bm] = lo;
    } else {
      sorted[pos] = R;
      if (pos % bm == 0) block_expert[pos / bm] = -1;
    }
  }
}

}  // namespace

hipError_t launch_grouped_index(const int32_t* offsets, int64_t R, int32_t E, int32_t bm, int64_t cap,
                                int32_t* sorted, int32_t* block_expert, int32_t* num_padded,
                                hipStream_t stream) {
  const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>((cap + kThreads - 1) / kThreads, 1024));
  hipLaunchKernelGGL(grouped_index_kernel, dim3(unsigned(wgs)), dim3(kThreads), 0, stream, offsets,
                     int(R), int(E), int(bm), int(cap), sorted, block_expert, num_padded);
  return hipGetLastError();
}

size_t moe_align_ws_bytes(int64_t, int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_moe_align(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                            int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                            int32_t* expert_offsets, int32_t* num_padded, void*,
                            hipStream_t stream) {
  const int64_t n_flat = T * topk;
  const int max_blocks = int(hq_moe_align_capacity(T, topk, E, block_m) / size_t(block_m));
  if (n_flat <= 64) {   // a few tokens: one wave
    hipLaunchKernelGGL(moe_align_small_kernel, dim3(1), dim3(64), 0, stream, topk_ids, int(n_flat), int(E),
                       int(block_m), sorted_ids, block_expert, expert_offsets, num_padded, max_blocks);
    return hipGetLastError();
  }
  const size_t smem = sizeof(int) * (size_t(E) * 3 + 1 + 2 * kWaves + size_t(kWaves) * E);
  // up to 128 workgroups of whole tiles: each counts the whole list, then scatters its own range
  const int64_t tiles = std::max<int64_t>(1, (n_flat + kThreads - 1) / kThreads);
  const int64_t tiles_per_wg = (tiles + 127) / 128;
  const int64_t wgs = (tiles + tiles_per_wg - 1) / tiles_per_wg;
  hipLaunchKernelGGL(moe_align_kernel, dim3(unsigned(wgs)), dim3(kThreads), smem, stream, topk_ids,
                     int(n_flat), int(E), int(block_m), sorted_ids, block_expert,
                     expert_offsets, num_padded, max_blocks, int(tiles_per_wg * kThreads));
  return hipGetLastError();
}

}  // namespace hq
