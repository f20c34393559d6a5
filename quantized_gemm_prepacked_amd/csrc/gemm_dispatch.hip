// gemm_dispatch.hip -- per-M-range kernel choice and launches (the tuning table), plus the
// split-K reduction kernel.
//
// The Humming announcement (section "Tuning and JIT compilation per workload") prepares
// different kernel configurations for ranges of input sizes and dispatches at runtime. Here the
// configurations are compiled ahead of time for gfx950 and chosen by M (or tokens per expert
// for MoE) and by the shape.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "gemm_common.h"
#include "internal.h"

namespace hq {

namespace {

constexpr int kCUs = 256;
// Stream-K arrival counters: up to kSkStreams streams per GPU, kSkMaxGroups tile groups per call.
constexpr int kSkStreams = 16;
constexpr int kSkMaxGroups = 8192;

// K per skinny unit (8-bit weights other than W8A8's step over two 64-k layout units at a time)
int k_unit(const Combo& c) {
  return (c.fam == FAM_FP8B || c.fam == FAM_W8A16 || c.fam == FAM_F8A16) ? 128 : family_k_unit(c.fam);
}

// Families with no LDS-tiled instantiation: the skinny and ping-pong kernels (and, for
// block-scaled FP8, the pipelined one) cover every shape they take.
bool pp_only(const Combo& c) {
  return c.fam == FAM_W4A4 || c.fam == FAM_W4A8MX || c.fam == FAM_MXW4A16 || c.fam == FAM_FP8B ||
         c.fam == FAM_W8A16 || c.fam == FAM_F8A16 || c.fam == FAM_WNA2 || c.fam == FAM_WNA3;
}

// Families with a pipelined-kernel instantiation, dense and MoE.
bool has_pipe(const Combo& c) {
  return c.fam == FAM_WNA16 || c.fam == FAM_W8A8 || c.fam == FAM_W4A8 || c.fam == FAM_FP8B ||
         c.fam == FAM_W8A16 || c.fam == FAM_F8A16 || c.fam == FAM_MXW4A16 || c.fam == FAM_W4A4 ||
         c.fam == FAM_W4A8MX;
}
bool has_pipe_moe(const Combo& c) { return c.fam == FAM_WNA16 || c.fam == FAM_FP8B; }

// Activation bytes per 2 k (bf16: 4; 8-bit: 2; 4-bit: 1): the direct-to-LDS kernels address
// activation rows with 32-bit offsets, so M * K * this / 2 must stay below 2^32.
uint64_t act_bytes_2k(const Combo& c) {
  return family_bf16_act(c.fam) ? 4u : c.fam == FAM_W4A4 ? 1u : 2u;
}

// Pick the skinny configuration for a row block of `rows` rows and N channels (measured on
// MI355X at the benchmark shapes; the first candidate whose channel-tile count divides N/16).
int pick_skinny(const Combo& c, int64_t rows, int64_t N) {
  const int64_t nt = N / 16;
  int n_cfg = 0;
  const SkinnyCfg* cfgs = skinny_configs(&n_cfg);
  auto first_fit = [&](std::initializer_list<int> cands) {
    for (int i : cands)
      if (nt % cfgs[i].ntw == 0 && skinny_lds_bytes(c.fam, i) <= 160 * 1024 &&
          (!cfgs[i].few || rows <= kFewRows))
        return i;
    return 2;  // NTW = 1 always fits (same rows as the candidates' fallback)
  };
  if (rows <= kFewRows) {
    // bf16 activations: the few-row forms (one activation copy per unit instead of four).
    // N=14336 K=4096 M=1, few-row form against the best whole-block one: INT4 9.25 / 9.60 us,
    // MXFP4 8.53 / 8.88, UINT2 8.00 / 8.78, UINT3 10.80 / 11.49, INT8 13.00 / 13.10, FP8 12.07 /
    // 12.32.
    if (c.fam == FAM_WNA16) return first_fit({30, 28, 13, 0, 1, 2});
    if (c.fam == FAM_MXW4A16) return first_fit({32, 30, 28, 13, 0, 1, 2});
    if (c.fam == FAM_WNA2 || c.fam == FAM_WNA3) return first_fit({31, 30, 28, 13, 0, 1, 2});
    if (c.fam == FAM_W8A16) return first_fit({33, 31, 27, 0, 1, 2});
    if (c.fam == FAM_F8A16) return first_fit({30, 31, 27, 0, 1, 2});
    if (c.fam == FAM_FP8B) return first_fit({21, 2});
  }
  if (rows <= 16) {
    if (c.fam == FAM_WNA2 || c.fam == FAM_WNA3) return first_fit({28, 13, 0, 1, 2});
    // 8-bit weights with bf16 activations, N=14336 K=4096: 16 waves of 64 channels, two units in
    // flight (M=1 INT8 / FP8: 13.2 / 12.3 us; the 8-wave form 13.5 / 12.6)
    if (c.fam == FAM_W8A16 || c.fam == FAM_F8A16) return first_fit({27, 0, 1, 2});
    if (c.fam == FAM_MXW4A16) return first_fit({28, 13, 0, 1, 2});
    // 8-bit activations, N=K=8192: block-scaled FP8 M=8 / 16 12.65 / 13.16 us (the form taken
    // below 5 rows: 13.01 / 14.87); W8A8 M=8 12.23 us (the 16-row choice: 13.26)
    if (c.fam == FAM_FP8B) return first_fit({20, 21, 2});
    if (c.fam == FAM_W8A8) return rows <= 8 ? first_fit({2}) : first_fit({1, 11, 2});
    if (c.fam == FAM_W4A8) return first_fit({21, 2});
    if (c.fam == FAM_W4A4 || c.fam == FAM_W4A8MX) return first_fit({21, 2});
    return first_fit({28, 13, 0, 1, 2});
  }
  if (rows <= 32) {
    if (c.fam == FAM_WNA2 || c.fam == FAM_WNA3) return first_fit({29, 22, 3, 7, 8});
    if (c.fam == FAM_W8A16) return first_fit({29, 22, 3, 7, 8});   // M=32: 16.0 us (next 18.9)
    if (c.fam == FAM_F8A16) return first_fit({22, 29, 3, 7, 8});   // M=32: 15.8 us (next 16.3)
    if (c.fam == FAM_MXW4A16) return first_fit({29, 22, 3, 7, 8});
    // M=32: block-scaled FP8 (N=K=8192) 16.0 us against 22.8 for the 32-row 4-tile form; the
    // MXFP4-weight formats (N=4096, K=7168) on two 16-row blocks of 32 channels: W4A8 7.24,
    // W4A4 7.04, MXFP8 activations 7.52 us against 8.50 / 8.25 / 9.35 for one 32-row block
    if (c.fam == FAM_FP8B) return first_fit({23, 15, 8});
    if (c.fam == FAM_W4A8 || c.fam == FAM_W4A4 || c.fam == FAM_W4A8MX) return first_fit({18, 16, 8});
    if (c.fam == FAM_W8A8) return first_fit({23, 15, 8});
    return first_fit({29, 22, 3, 7, 8});
  }
  // 2-bit weights: two 32-row blocks, double-buffered (N=14336, K=4096, M=64 / 128: 20.4 / 37.2
  // us against 22.4 / 39.2 with 64-row blocks)
  if (c.fam == FAM_WNA2 || c.fam == FAM_WNA3) return first_fit({22, 5, 4, 6});
  // INT4 at 33..64 rows: two 32-row blocks of 64 channels, double-buffered (M = 48 / 64: 20.6 /
  // 21.4 us against 21.4 / 21.9 for one 64-row block)
  if (c.fam == FAM_WNA16) return first_fit({22, 5, 4, 6});
  // MXFP4 weights with bf16 activations, M=64: two 32-row blocks of 64 channels 18.7 us (the
  // 64-row form 20.2); M=128: the 64-row form
  if (c.fam == FAM_MXW4A16) return rows <= 64 ? first_fit({3, 5, 4, 6}) : first_fit({4, 5, 6});
  // M=64 (N=4096, K=7168): W4A8 8.96 us against 16.3 for the 64-row form with a K split, W4A4
  // 8.76, MXFP8 activations 9.36 on four 16-row blocks (9.87 on two 32-row ones); W8A8 (N=K=8192)
  // 21.96 us on two 32-row blocks against 25.6 for the pipelined kernel
  if ((c.fam == FAM_W4A4 || c.fam == FAM_W4A8) && rows <= 64) return first_fit({23, 15, 8});   // two 32-row blocks
  if (c.fam == FAM_W4A8MX && rows <= 64) return first_fit({28, 23, 15, 8});
  if (c.fam == FAM_W8A8 && rows <= 64) return first_fit({29, 15, 8});
  // M=128 (N=4096, K=7168): four 32-row blocks of 64 channels, W4A8 / W4A4 / MXFP8 activations
  // 12.4 / 12.0 / 13.6 us against 21.5 / 20.0 / 21.2 for the 64-row form; W4A8 M=256: 32-row
  // blocks of 64 channels, double-buffered, 19.5 against 21.3
  if ((c.fam == FAM_W4A8 || c.fam == FAM_W4A4 || c.fam == FAM_W4A8MX) && rows <= 128)
    return first_fit({29, 4, 5, 6});
  if (c.fam == FAM_W4A8 && rows <= 256) return first_fit({22, 4, 5, 6});
  if (c.fam == FAM_FP8B && rows <= 64) return first_fit({29, 15, 8});   // M=64: 31.9 us vs 40.6
  return first_fit({4, 5, 6});
}

size_t acc_elem_bytes() { return 4; }

// Sweep override for tuning runs: HQ_TUNE="kind=<k>,cfg=<i>,split=<s>" forces the kernel
// family (0 skinny, 1 LDS-tiled, 2 async-pipelined, 3 ping-pong), its configuration and (skinny) the K split for every dense call;
// entries that do not fit the shape are ignored. Read on every call so one process can sweep.
struct TuneOverride {
  int kind = -1, cfg = -1, split = -1;
};

TuneOverride tune_override() {
  TuneOverride o;
  if (const char* e = std::getenv("HQ_TUNE")) {
    std::sscanf(e, "kind=%d,cfg=%d,split=%d", &o.kind, &o.cfg, &o.split);
  }
  return o;
}

template <int FAM>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(KParams p) {
  typedef typename AccType<FAM>::elem E;
  const size_t total = size_t(p.M) * p.N;
  const size_t idx = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const E* ws = reinterpret_cast<const E*>(p.ws);
  E s = ws[idx];
  for (int z = 1; z < p.split; ++z) s += ws[size_t(z) * total + idx];
  const int m = int(idx / p.N);
  const int n = int(idx % p.N);
  epilogue<FAM>(p, p.w, m, m, n, s, 1.0f);
}

}  // namespace

hipError_t launch_splitk_reduce(const KParams& p, int fam, hipStream_t s) {
  const size_t total = size_t(p.M) * p.N;
  dim3 grid(unsigned((total + 255) / 256));
  if (fam == FAM_WNA16)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_WNA16>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_W8A8)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_W8A8>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_W4A4)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_W4A4>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_W4A8MX)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_W4A8MX>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_MXW4A16)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_MXW4A16>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_FP8B)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_FP8B>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_W8A16)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_W8A16>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_WNA2)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_WNA2>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_WNA3)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_WNA3>, grid, dim3(256), 0, s, p);
  else if (fam == FAM_F8A16)
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_F8A16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<FAM_W4A8>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

namespace {

// Tiled configuration for a dense call, or -1 when the shape does not fit one.
int pick_tiled(const Combo&, int64_t N, int64_t K) {
  if (K % 128 != 0) return -1;
  if (N % 128 == 0) return 0;
  if (N % 64 == 0) return 1;
  if (N % 32 == 0) return 2;
  return -1;
}

// The per-M-range table for large M (kinds: 1 = LDS-tiled, 2 = async-pipelined, 3 = ping-pong),
// measured on MI355X at the benchmark shapes: the first entry whose max_m covers M and whose
// tile divides N is used; below the first entry (and when no tile fits) the skinny kernel runs.
struct RangeEntry {
  int64_t max_m;
  int kind, cfg;
};
constexpr int64_t kInf = int64_t(1) << 40;
// WNA16 at N=14336, K=4096: pipelined 64 x 128 with four waves of 64 x 32 at M = 65..128 (every wave
// spans the tile's 64 rows, so each dequantized weight feeds four row blocks: M=128 32.9 us against
// 35.4 for waves of 32 x 64 and 36.1 for eight waves of 32 x 32)
constexpr RangeEntry kWna16Table[] = {{64, 0, 0}, {128, 2, 15}, {256, 3, 3}, {kInf, 3, 0}};
// (M in (256, 512]: ping-pong 128 x 128 with four LDS slots, 57.7 vs 61.3 us with three)
// W8A8 at N=K=8192: pipelined 64 x 64 to M=128 (M = 96 / 128: 23.6 / 24.3 us), then 64 x 128 with
// four waves of 64 x 32 to 256 (M = 160 / 192 / 256: 36.1 / 36.5 / 37.7 us against 36.5 / 38.4 /
// 38.7 for 64 x 64)
constexpr RangeEntry kW8a8Table[] = {{64, 0, 0}, {128, 2, 3}, {256, 2, 15}, {512, 3, 11}, {1024, 3, 1}, {kInf, 2, 8}};
// The MXFP4-weight formats with 8- or 4-bit activations, measured at N=4096, K=7168 (one sweep
// of every pipelined and ping-pong configuration; us at the M values named, the choice's time
// first, the ping-pong kernel's best after the semicolon). Above the skinny range the pipelined
// kernel wins nearly everywhere (one barrier per step, all waves computing); which tile depends
// on how evenly it fills the CUs at this N.
// W4A8 (FP8 activations): skinny to M=256 (19.4 us), pipelined 64 x 64 to 512 (M = 320 / 448 /
// 512: 24.6 / 25.5 / 26.0 us against 27.1 / 26.6 / 27.4 skinny); then, at M = 768 / 1024 / 1536 /
// 2048 / 3072 / 4096 / 8192: 64 x 128 to 1024 (34.4 / 33.2; 38.8 / 39.3), 128 x 128 to 2048
// (45.5 / 52.4; 48.7 / 52.1), 128 x 256 with eight waves of 64 x 64 at 3072 (82.5; 95.0),
// 256 x 256 beyond (91.1 / 176.2; 100.9 / 197.1).
constexpr RangeEntry kW4a8Table[] = {{256, 0, 0}, {512, 2, 3}, {1024, 2, 2}, {2048, 2, 0}, {3072, 2, 12}, {kInf, 2, 11}};
// W4A4 (MXFP4 activations): skinny to M=160 (M=128: 11.9 us), pipelined 64 x 64 to 640 (M = 192 /
// 256 / 320 / 384 / 512: 18.5 / 18.9 / 23.2 / 23.8 / 23.0 us against 19.8 / 19.3 / 32.9 / 31.1 /
// 29.7 for skinny 64-row blocks), 64 x 128 to 1024 (32.4 / 30.7; 38.4 / 39.1), 128 x 256 with eight waves of 64 x 64 and three
// stages to 2048 (45.6 / 47.0; 50.2 / 51.9), 128 x 256 with four waves of 64 x 128 beyond
// (63.8 / 73.3 / 141.1; 69.2 / 75.1 / 146.9).
constexpr RangeEntry kW4a4Table[] = {{160, 0, 0}, {640, 2, 3}, {1024, 2, 2}, {2048, 2, 13}, {kInf, 2, 6}};
// W4A8-MXFP8: skinny to M=256 (21.1 us), pipelined 64 x 64 to 512 (M = 320 / 384 / 512: 25.0 /
// 25.6 / 27.4 us against 35.3 / 33.9 / 35.3 skinny), 64 x 128 to 1024 (37.5 / 36.2; 41.6 / 43.0), ping-pong 128 x 256 with four slots to 2048 (52.5 / 56.1), pipelined
// 256 x 256 beyond (92.1 / 99.5 / 192.2; 104.2 / 110.4 / 214.3).
constexpr RangeEntry kW4a8mxTable[] = {{256, 0, 0}, {512, 2, 3}, {1024, 2, 2}, {2048, 3, 8}, {kInf, 2, 11}};
// MXFP4 weights with bf16 activations: the W4A16 crossovers, ping-pong instead of async-pipelined
// (M = 128, N=14336 K=4096: the small-M kernel 25.7 us against 35.0 for ping-pong 128 x 128)
constexpr RangeEntry kMxW4a16Table[] = {{128, 0, 0}, {256, 3, 3}, {kInf, 3, 0}};
// Block-scaled FP8 W8A8, measured at N=K=8192: the small-M kernel to M=128 (33.1 us; ping-pong
// 58.4), pipelined 64 x 128 to 256 (M = 160 / 192 / 224 / 256: 41.4 / 42.7 / 42.2 / 43.4 us against
// 48.9 / 54.0 / 53.6 / 53.5 for the small-M kernel), ping-pong 128 x 128 with four LDS slots at M=512
// (56.5 us; pipelined 128 x 256 86.9), then the pipelined kernel, whose eight waves compute
// together so that one wave's per-step scaling runs beside the other's MFMAs (ping-pong at
// M = 768 / 1024 / 2048 / 4096: 106.2 / 107.9 / 214.9 / 408.9 us). Its two tiles alternate with
// how evenly they fill the 256 CUs: 128 x 256 (waves of 32 x 128) at M = 768 / 1024 / 3072
// (88.4 / 94.1 / 253.8 us; 256 x 256: 146.4 at 1024, 293.4 at 3072), 256 x 256 (waves of
// 64 x 128) at M = 1536 / 2048 / 4096 (149.9 / 153.6 / 303.2 us; 128 x 256: 162.7 / 169.4 / 338.8).
constexpr RangeEntry kFp8bTable[] = {{128, 0, 0}, {256, 2, 2}, {640, 3, 10}, {1280, 2, 14}, {2048, 2, 11},
                                     {3072, 2, 14}, {kInf, 2, 11}};
// INT8 / FP8 weights with bf16 activations, measured at N=14336, K=4096 (INT8 / FP8): skinny
// 64-row blocks to M=128 (34.5 / 32.5 us; ping-pong 41.7 / 32.1), ping-pong 128 x 128 with waves
// of 64 x 32 at M=256 (38.3 / 35.0 us; the ping-pong 128 x 256 tile's three-slot ring of 64 KiB
// steps exceeds the LDS), then the pipelined 128 x 256 tile with eight waves of 64 x 64 and two
// stages (the dequantization of one wave issues beside the other's MFMAs): M = 384 / 512 / 1024 /
// 8192 at 66.7 / 67.6 / 130.3 / 934.9 and 58.0 / 57.7 / 112.1 / 816.0 us, against 73.6 / 74.8 /
// 145.7 / 1038.9 and 67.6 / 69.4 / 132.2 / 961.5 for ping-pong 128 x 128 — except around M = 768,
// where its 336 tiles fill the CUs unevenly (127.9 / 109.5 us against 112.0 / 102.2).
constexpr RangeEntry kW8a16Table[] = {{128, 0, 0}, {256, 3, 3}, {640, 2, 12}, {896, 3, 3}, {kInf, 2, 12}};
// 2-bit WnA16 on the ping-pong kernel's 256-wide tiles (the only ones whose half-unit weight copies
// split over the eight waves), measured at N=14336, K=4096: skinny to M=128 (36.8 us; ping-pong
// 52.1), 64 x 256 with four slots to 256 (44.2 us; 128 x 256 71.2), 128 x 256 beyond (M = 320 /
// 384 / 512: 65.4 / 66.1 / 68.0 us against 83.2 / 83.4 / 84.8 for 64 x 256; M=1024 / 8192: 133 /
// 916 us, the skinny kernel 242 / 1834)
constexpr RangeEntry kWna2Table[] = {{128, 0, 0}, {256, 3, 13}, {kInf, 3, 0}};
// 3-bit WnA16 (each tile's 768-byte unit of a step lands in a 1 KiB LDS slot, three 4-byte-per-lane
// copies, so every ping-pong tile whose ring fits the LDS works), measured at N=14336, K=4096:
// skinny to M=128 (46.6 us), ping-pong 128 x 128 to 256 (M=192 / 256: 55.2 / 55.6 us against 69.9
// for 64 x 256 with four slots), 128 x 256 beyond (M=512 / 1024 / 2048 / 8192: 89.8 / 172.6 / 337.8
// / 1154.8 us; the best skinny configuration 2342 us at M=8192)
constexpr RangeEntry kWna3Table[] = {{128, 0, 0}, {256, 3, 3}, {kInf, 3, 0}};

int tile_n_of(int kind, int cfg) {
  int n = 0;
  if (kind == 1) {
    const TiledCfg& t = tiled_configs(&n)[cfg];
    return 16 * t.ntw * t.wn;
  }
  if (kind == 3) {
    const PPCfg& t = pp_configs(&n)[cfg];
    return 16 * t.ntw * t.wn;
  }
  const PipeCfg& t = pipe_configs(&n)[cfg];
  return 16 * t.ntw * t.wn;
}

// (kind, cfg) from the table, or kind 0 for the skinny kernel.
RangeEntry pick_range(const Combo& c, int64_t M, int64_t N, int64_t K) {
  if (K % 128 != 0) return {0, 0, 0};
  const RangeEntry* t;
  int n;
  if (c.fam == FAM_WNA16) {
    t = kWna16Table;
    n = int(sizeof(kWna16Table) / sizeof(kWna16Table[0]));
  } else if (c.fam == FAM_W8A8) {
    t = kW8a8Table;
    n = int(sizeof(kW8a8Table) / sizeof(kW8a8Table[0]));
  } else if (c.fam == FAM_FP8B) {
    t = kFp8bTable;
    n = int(sizeof(kFp8bTable) / sizeof(kFp8bTable[0]));
  } else if (c.fam == FAM_MXW4A16) {
    t = kMxW4a16Table;
    n = int(sizeof(kMxW4a16Table) / sizeof(kMxW4a16Table[0]));
  } else if (c.fam == FAM_WNA2) {
    t = kWna2Table;
    n = int(sizeof(kWna2Table) / sizeof(kWna2Table[0]));
  } else if (c.fam == FAM_WNA3) {
    t = kWna3Table;
    n = int(sizeof(kWna3Table) / sizeof(kWna3Table[0]));
  } else if (c.fam == FAM_W8A16 || c.fam == FAM_F8A16) {
    t = kW8a16Table;
    n = int(sizeof(kW8a16Table) / sizeof(kW8a16Table[0]));
  } else if (c.fam == FAM_W4A4) {
    t = kW4a4Table;
    n = int(sizeof(kW4a4Table) / sizeof(kW4a4Table[0]));
  } else if (c.fam == FAM_W4A8MX) {
    t = kW4a8mxTable;
    n = int(sizeof(kW4a8mxTable) / sizeof(kW4a8mxTable[0]));
  } else {
    t = kW4a8Table;
    n = int(sizeof(kW4a8Table) / sizeof(kW4a8Table[0]));
  }
  for (int i = 0; i < n; ++i) {
    if (M > t[i].max_m) continue;
    if (t[i].kind == 0) return t[i];
    if (N % tile_n_of(t[i].kind, t[i].cfg) != 0) break;
    if (t[i].kind == 2 && pipe_lds_bytes(c.fam, t[i].cfg) > 160 * 1024) break;
    if (t[i].kind == 3 && (K % 128 != 0 || pp_lds_bytes(c.fam, t[i].cfg) > 160 * 1024)) break;
    return t[i];
  }
  // Fallbacks when the preferred tile does not divide N.
  if (pp_only(c)) {
    int n_p = 0;
    const PPCfg* pc = pp_configs(&n_p);
    for (int cfg : {10, 3, 2})   // 128 x 128 tiles (four LDS slots where they fit)
      if (M > 256 && N % (16 * pc[cfg].ntw * pc[cfg].wn) == 0 && pp_lds_bytes(c.fam, cfg) <= 160 * 1024)
        return {kInf, 3, cfg};
    return {0, 0, 0};
  }
  const int tc = pick_tiled(c, N, K);
  if (M > 64 && tc >= 0) return {kInf, 1, tc};
  return {0, 0, 0};
}

}  // namespace

namespace {

bool override_fits(const Combo& c, const TuneOverride& o, int64_t M, int64_t N, int64_t K) {
  int n = 0;
  if (o.kind == 0) {
    const SkinnyCfg* cfgs = skinny_configs(&n);
    return o.cfg < 0 || (o.cfg < n && (N / 16) % cfgs[o.cfg].ntw == 0 &&
                         skinny_lds_bytes(c.fam, o.cfg) <= 160 * 1024 &&
                         (!cfgs[o.cfg].few || M <= kFewRows));
  }
  if ((o.kind == 1 && pp_only(c)) || (o.kind == 2 && !has_pipe(c))) return false;
  if (o.kind == 1) {
    const TiledCfg* cfgs = tiled_configs(&n);
    return pick_tiled(c, N, K) >= 0 && o.cfg >= 0 && o.cfg < n && N % (16 * cfgs[o.cfg].ntw * cfgs[o.cfg].wn) == 0;
  }
  const bool a32 = uint64_t(M) * uint64_t(K) * act_bytes_2k(c) / 2 < (uint64_t(1) << 32);
  if (o.kind == 2) {
    const PipeCfg* cfgs = pipe_configs(&n);
    return a32 && K % 128 == 0 && o.cfg >= 0 && o.cfg < n && N % (16 * cfgs[o.cfg].ntw * cfgs[o.cfg].wn) == 0 &&
           pipe_lds_bytes(c.fam, o.cfg) <= 160 * 1024;
  }
  if (o.kind == 3) {
    const PPCfg* cfgs = pp_configs(&n);
    return a32 && K % 128 == 0 && o.cfg >= 0 && o.cfg < n && N % (16 * cfgs[o.cfg].ntw * cfgs[o.cfg].wn) == 0 &&
           pp_lds_bytes(c.fam, o.cfg) <= 160 * 1024;
  }
  return false;
}

}  // namespace

int kernel_config_count(int kind) {
  int n = 0;
  if (kind == 0) skinny_configs(&n);
  else if (kind == 1) tiled_configs(&n);
  else if (kind == 2) pipe_configs(&n);
  else if (kind == 3) pp_configs(&n);
  return n;
}

// The batch-invariant configuration: one skinny configuration per (family, N) for every M, no
// K split across workgroups (a row's sum order is then its own units in order per wave and the
// waves in order, whatever the other rows), two 16-row blocks per workgroup.
int invariant_skinny_cfg(const Combo& c, int64_t N) {
  int n_cfg = 0;
  const SkinnyCfg* cfgs = skinny_configs(&n_cfg);
  for (int i : {29, 15, 8})
    if ((N / 16) % cfgs[i].ntw == 0 && skinny_lds_bytes(c.fam, i) <= 160 * 1024) return i;
  return 8;
}

Plan plan_dense(const Combo& c, int64_t M, int64_t N, int64_t K) {
  Plan pl{};
  if (c.invariant) {
    pl.kind = 0;
    pl.cfg = invariant_skinny_cfg(c, N);
    pl.split = 1;
    pl.ws_bytes = 0;
    return pl;
  }
  TuneOverride tov = tune_override();
  if (tov.kind < 0) {
    // the run-time tuning table, when it has an entry for this shape that fits
    TuneOverride t;
    if (tuning_lookup(c, M, N, K, &t.kind, &t.cfg, &t.split) && override_fits(c, t, M, N, K)) tov = t;
  }
  RangeEntry pick = pick_range(c, M, N, K);
  // Sweep overrides (HQ_TUNE): an override that does not fit the shape (tile, LDS, K) is
  // refused (kind -1, the call fails) rather than silently replaced.
  if (tov.kind >= 0 && !override_fits(c, tov, M, N, K)) {
    pl.kind = -1;
    return pl;
  }
  if (tov.kind == 0) pick = {0, 0, 0};
  if (tov.kind == 1 && pick_tiled(c, N, K) >= 0) {
    int n_t = 0;
    const TiledCfg* tc = tiled_configs(&n_t);
    const int cfg = (tov.cfg >= 0 && tov.cfg < n_t && N % (16 * tc[tov.cfg].ntw * tc[tov.cfg].wn) == 0)
                        ? tov.cfg : pick_tiled(c, N, K);
    pick = {kInf, 1, cfg};
  }
  if (tov.kind == 2 && K % 128 == 0) {
    int n_p = 0;
    const PipeCfg* pc = pipe_configs(&n_p);
    if (tov.cfg >= 0 && tov.cfg < n_p && N % (16 * pc[tov.cfg].ntw * pc[tov.cfg].wn) == 0 &&
        pipe_lds_bytes(c.fam, tov.cfg) <= 160 * 1024)
      pick = {kInf, 2, tov.cfg};
  }
  if (tov.kind == 3 && K % 128 == 0) {
    int n_p = 0;
    const PPCfg* pc = pp_configs(&n_p);
    if (tov.cfg >= 0 && tov.cfg < n_p && N % (16 * pc[tov.cfg].ntw * pc[tov.cfg].wn) == 0 &&
        pp_lds_bytes(c.fam, tov.cfg) <= 160 * 1024)
      pick = {kInf, 3, tov.cfg};
  }
  // The direct-to-LDS kernels address activations with 32-bit offsets.
  if ((pick.kind == 2 || pick.kind == 3) &&
      uint64_t(M) * uint64_t(K) * act_bytes_2k(c) / 2 >= (uint64_t(1) << 32)) {
    const int tc = pp_only(c) ? -1 : pick_tiled(c, N, K);
    pick = tc >= 0 ? RangeEntry{kInf, 1, tc} : RangeEntry{0, 0, 0};
  }
  if (pick.kind != 0) {
    pl.kind = pick.kind;
    pl.cfg = pick.cfg;
    pl.split = 1;
    // WNA16: the activation group sums of the offset term
    pl.ws_bytes = family_int_groups(c.fam) ? group_sums_split_bytes(M, K) : 0;
    return pl;
  }
  pl.kind = 0;
  pl.cfg = pick_skinny(c, M, N);
  int n_cfg = 0;
  const SkinnyCfg* cfgs = skinny_configs(&n_cfg);
  if (tov.kind == 0 && tov.cfg >= 0 && tov.cfg < n_cfg && (N / 16) % cfgs[tov.cfg].ntw == 0 &&
      skinny_lds_bytes(c.fam, tov.cfg) <= 160 * 1024 && (!cfgs[tov.cfg].few || M <= kFewRows))
    pl.cfg = tov.cfg;
  const SkinnyCfg& sc = cfgs[pl.cfg];
  const int64_t units = K / k_unit(c);
  const int64_t wgs = (N / 16 / sc.ntw) * ((M + 16 * sc.mb - 1) / (16 * sc.mb));
  int split = 1;
  // Far too few workgroups to cover the chip: split K across workgroups (partials + a reduction
  // launch) as long as every wave keeps at least two units. Measured: with a few hundred
  // workgroups the extra launch costs more than the idle CUs.
  while (wgs * split < kCUs / 2 && units / (int64_t(split) * 2 * sc.nw) >= 2) split *= 2;
  if (tov.kind == 0 && tov.split >= 1 && tov.split <= units) split = tov.split;
  pl.split = split;
  pl.ws_bytes = split > 1 ? size_t(split) * M * N * acc_elem_bytes() : 0;
  // Stream-K: one row block, a configuration with a Stream-K form, fewer tile groups than the
  // workgroups the chip runs at once (one per CU; two for workgroups of at most eight waves), so
  // that a plain launch would leave CUs idle; at least one K unit per wave
  const long long res_wgs = (long long)kCUs * (sc.nw <= 8 ? 2 : 1);
  if (c.stream_k && tov.kind < 0 && M <= 16 * sc.mb && skinny_stream_k_cfg(pl.cfg) &&
      N / 16 / sc.ntw < res_wgs && N / 16 / sc.ntw <= kSkMaxGroups) {
    const long long items = (long long)(N / 16 / sc.ntw) * units;
    const long long wgs = std::min<long long>(res_wgs, items / sc.nw);
    if (wgs >= 1) {
      const long long per = items / wgs;                 // every workgroup gets per or per + 1
      const int slots = int((units + per - 1) / per) + 1;  // pieces a tile group can be cut into
      pl.kind = 4;
      pl.split = int(wgs);
      pl.sk_items = items;
      pl.sk_slots = slots;
      pl.ws_bytes = size_t(N / 16 / sc.ntw) * slots * size_t(sc.mb * sc.ntw * 4 * 64) * acc_elem_bytes();
    }
  }
  return pl;
}

Plan plan_moe(const Combo& c, int64_t T, int32_t, int32_t, int64_t N, int64_t K, int32_t block_m) {
  Plan pl{};
  pl.split = 1;
  pl.ws_bytes = 0;
  if (c.invariant) {   // the dense path's fixed configuration; its 32-row blocks are block_m
    pl.kind = 0;
    pl.cfg = invariant_skinny_cfg(c, N);
    return pl;
  }
  // Sweep overrides (HQ_TUNE="kind=3,cfg=<i>", "kind=2,cfg=<i>" or "kind=0,cfg=<i>"): a
  // ping-pong, pipelined (WNA16 and block-scaled FP8) or skinny configuration whose tile rows
  // equal block_m; one that does not fit is refused (kind -1).
  const TuneOverride tov = tune_override();
  if (tov.kind == 0) {
    int n_s = 0;
    const SkinnyCfg* sc = skinny_configs(&n_s);
    const bool fits = tov.cfg >= 0 && tov.cfg < n_s && 16 * sc[tov.cfg].mb == block_m && !sc[tov.cfg].few &&
                      (N / 16) % sc[tov.cfg].ntw == 0 && skinny_lds_bytes(c.fam, tov.cfg) <= 160 * 1024;
    pl.kind = fits ? 0 : -1;
    pl.cfg = tov.cfg;
    return pl;
  }
  if (tov.kind == 2) {
    int n_p = 0;
    const PipeCfg* pc = pipe_configs(&n_p);
    const bool fits = has_pipe_moe(c) && tov.cfg >= 0 && tov.cfg < n_p &&
                      16 * pc[tov.cfg].mw * pc[tov.cfg].wm == block_m && K % 128 == 0 &&
                      N % (16 * pc[tov.cfg].ntw * pc[tov.cfg].wn) == 0 &&
                      pipe_lds_bytes(c.fam, tov.cfg) <= 160 * 1024 &&
                      uint64_t(T) * uint64_t(K) * act_bytes_2k(c) / 2 < (uint64_t(1) << 32);
    pl.kind = fits ? 2 : -1;
    pl.cfg = tov.cfg;
    pl.ws_bytes = family_int_groups(c.fam) ? group_sums_split_bytes(T, K) : 0;
    return pl;
  }
  if (tov.kind == 3) {
    int n_p = 0;
    const PPCfg* pc = pp_configs(&n_p);
    const bool fits = tov.cfg >= 0 && tov.cfg < n_p && 16 * pc[tov.cfg].mw * pc[tov.cfg].wm == block_m &&
                      K % 128 == 0 && N % (16 * pc[tov.cfg].ntw * pc[tov.cfg].wn) == 0 &&
                      pp_lds_bytes(c.fam, tov.cfg) <= 160 * 1024 && uint64_t(T) * uint64_t(K) * 2u < (uint64_t(1) << 32);
    pl.kind = fits ? 3 : -1;
    pl.cfg = tov.cfg;
    pl.ws_bytes = family_int_groups(c.fam) ? group_sums_split_bytes(T, K) : 0;
    return pl;
  }
  // Blocks of 32 and 64 rows: the ping-pong kernel with one expert block per tile row, its
  // widest tile that divides N (measured on MI355X at the DeepSeek-V3 gate_up and Down shapes,
  // T = 32..4096: 32 x 256 and 64 x 512 beat the LDS-tiled and skinny kernels from two routed
  // rows per expert up); otherwise the LDS-tiled 64 x 128 tile, then the skinny kernel.
  const bool a32 = uint64_t(T) * uint64_t(K) * act_bytes_2k(c) / 2 < (uint64_t(1) << 32);   // 32-bit row offsets
  if (K % 128 == 0 && a32 && (block_m == 32 || block_m == 64 || block_m == 128)) {
    // (the 8-bit-activation formats' 32-row tiles do not split into whole-wave copies: skinny)
    static const int pp32[1] = {7}, pp64[2] = {5, 4}, pp128[2] = {0, 3};
    const int* cands = block_m == 32 ? pp32 : block_m == 64 ? pp64 : pp128;
    const int n_c = block_m == 32 ? 1 : 2;
    int n_p = 0;
    const PPCfg* pc = pp_configs(&n_p);
    for (int j = 0; j < n_c; ++j) {
      const PPCfg& t = pc[cands[j]];
      if (N % (16 * t.ntw * t.wn) == 0 && pp_lds_bytes(c.fam, cands[j]) <= 160 * 1024 &&
          16 * t.mw * t.wm == block_m) {
        pl.kind = 3;
        pl.cfg = cands[j];
        pl.ws_bytes = family_int_groups(c.fam) ? group_sums_split_bytes(T, K) : 0;  // WNA16 offset term
        return pl;
      }
    }
  }
  if (block_m == 128) {   // only the ping-pong kernel has 128-row tiles
    pl.kind = -1;
    return pl;
  }
  if (c.fam == FAM_WNA16 && block_m == 64 && N % 128 == 0 && K % 128 == 0) {
    pl.kind = 1;       // LDS-tiled, 64 x 128 tiles: one expert block per tile row
    pl.cfg = 3;
    pl.ws_bytes = group_sums_split_bytes(T, K);  // per-token activation group sums
    return pl;
  }
  // MoE row blocks: many small workgroups share the GPU, so keep the per-workgroup LDS small
  pl.kind = 0;
  const int64_t nt = N / 16;
  int n_cfg = 0;
  const SkinnyCfg* cfgs = skinny_configs(&n_cfg);
  // the kernel's row block (16 * mb rows) is the alignment's block of block_m rows; the last
  // candidate of each list has one channel tile per workgroup and always fits
  // (16-row blocks: the double-buffered 8-wave configuration, measured on the DeepSeek-V3 gate_up
  // shape at T = 1 / 32: 23.9 / 126.9 us against 29.7 / 158.6 us for single-buffered INT4)
  static const int c16[3] = {13, 1, 2}, c32[3] = {3, 7, 8}, c64[3] = {4, 5, 6};
  const int* cands = block_m <= 16 ? c16 : block_m <= 32 ? c32 : c64;
  pl.cfg = cands[2];
  for (int j = 0; j < 3; ++j)
    if (nt % cfgs[cands[j]].ntw == 0) {
      pl.cfg = cands[j];
      break;
    }
  return pl;
}

bool moe_block_m_supported(int32_t block_m) {
  return block_m == 16 || block_m == 32 || block_m == 64 || block_m == 128;
}

// Measured on MI355X (gate_up 4096 x 7168 and Down 7168 x 2048, 256 experts, top-8, skewed
// routing): 16-row blocks below 2 routed rows per expert, 32-row blocks from 2, 64-row blocks
// (ping-pong 64 x 512 / 64 x 256) from 8 -- at 8 and 16 rows per expert (T = 256 / 512) they beat
// 32-row blocks in every format measured (INT4 gate_up 375 / 566 us against 399 / 636; MXFP4 315 /
// 478 against 325 / 515; block-scaled FP8 463 / 620 against 569 / 928; the INT4 and W4A8 layers at
// T = 512 942 / 612 us against 1026 / 894). 128-row blocks (ping-pong 128 x 256): for bf16
// activations with 4-bit weights from 64 rows per expert (INT4 gate_up T = 2048 / 4096: 1423 / 2504
// us against 1528 / 2713; MXFP4 1201 / 2079 against 1277 / 2295; the INT4 layer 2254 / 4021 against
// 2330 / 4235; a tie at 32 rows), for block-scaled FP8 from 8 (T = 256 / 1024 / 4096: 454 / 816 /
// 2064 us against 463 / 939 / 2591). The other 8-bit-activation formats keep 64-row blocks (the
// W4A8 layer at T = 4096: 2707 us with 128 against 2509).
int32_t moe_block_m(const Combo& c, int64_t T, int32_t topk, int32_t E, int64_t N, int64_t K) {
  if (c.invariant) return 32;
  const double rows_per_expert = double(T) * topk / std::max(1, E);
  if (rows_per_expert < 2) return 16;
  if (rows_per_expert < 8) return 32;
  const bool fits128 = K % 128 == 0 && N % 128 == 0 &&
                       uint64_t(T) * uint64_t(K) * act_bytes_2k(c) / 2 < (uint64_t(1) << 32);
  // 128-row blocks: INT4 / MXFP4 experts with bf16 activations from 24 routed rows per expert
  // (gate_up 4096 x 7168, skewed top-8 of 256, T = 512 / 768 / 1024 / 1536: INT4 558 / 680 / 830 /
  // 1081 us against 554 / 693 / 860 / 1135 with 64-row blocks), block-scaled FP8 from 8
  const bool wide = (c.fam == FAM_WNA16 || c.fam == FAM_MXW4A16) ? rows_per_expert >= 24 : c.fam == FAM_FP8B;
  return wide && fits128 ? 128 : 64;
}

// Stream-K arrival counters: library-owned, zero from load time, and left at zero by every call
// (the workgroup that sums a tile group resets its counter). Each stream that runs a Stream-K
// call gets its own set, so calls ordered on one stream reuse it safely and calls on different
// streams never share one. The kernels get the device address of the current device's copy
// (taken once per device), never the array's name.
static __device__ uint32_t sk_counter_sets[kSkStreams * kSkMaxGroups];

static hipError_t stream_k_counters(hipStream_t stream, uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* base[kMaxDevices] = {};
  static hipStream_t owner[kMaxDevices][kSkStreams] = {};
  static int used[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(sk_counter_sets));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    base[dev] = static_cast<uint32_t*>(p);
  }
  *out = nullptr;
  for (int i = 0; i < used[dev]; ++i)
    if (owner[dev][i] == stream) {
      *out = base[dev] + size_t(i) * kSkMaxGroups;
      return hipSuccess;
    }
  if (used[dev] < kSkStreams) {
    owner[dev][used[dev]] = stream;
    *out = base[dev] + size_t(used[dev]) * kSkMaxGroups;
    ++used[dev];
  }
  return hipSuccess;
}

hipError_t launch_gemm(const GemmCall& call, const Plan& plan) {
  const Combo& c = call.c;
  const PackedLayout L = make_layout(c.fam, c.asym, call.N, call.K);
  KParams p{};
  p.a = static_cast<const uint8_t*>(call.a);
  p.a_scale = call.a_scale;
  p.w = call.w;
  p.y = call.y;
  p.ws = call.ws;
  p.N = int(call.N);
  p.K = int(call.K);
  p.k_units = int(L.k_units);
  p.asym = c.asym ? 1 : 0;
  p.out_i32 = c.out_i32 ? 1 : 0;
  p.expert_stride = L.expert_stride;
  p.scales_off = L.scales_off;
  p.zeros_off = L.zeros_off;
  const bool moe = call.sorted_ids != nullptr;
  if (plan.kind == 3 && !moe) {
    int n_cfg = 0;
    const PPCfg& pc = pp_configs(&n_cfg)[plan.cfg];
    const int bm = 16 * pc.mw * pc.wm, bn = 16 * pc.ntw * pc.wn;
    p.split = 1;
    p.units_per_split = p.k_units;
    p.M = int(call.M);
    if (family_int_groups(c.fam)) {
      hipError_t e = launch_group_sums_split(p.a, p.M, p.K, call.ws, call.stream);
      if (e != hipSuccess) return e;
    }
    const int tiles_n = int(call.N / bn);
    const int tiles_m = int((call.M + bm - 1) / bm);
    return launch_pingpong(p, c.fam, false, plan.cfg, dim3(unsigned(tiles_m * tiles_n)), tiles_m, tiles_n,
                           call.stream);
  }
  if (plan.kind == 3) {   // MoE: one workgroup row of tiles per block of the token sort
    int n_cfg = 0;
    const PPCfg& pc = pp_configs(&n_cfg)[plan.cfg];
    const int bm = 16 * pc.mw * pc.wm, bn = 16 * pc.ntw * pc.wn;
    if (bm != call.block_m) return hipErrorInvalidValue;
    p.split = 1;
    p.units_per_split = p.k_units;
    p.M = int(call.T * call.topk);
    p.sorted_ids = call.sorted_ids;
    p.block_expert = call.block_expert;
    p.num_padded = call.num_padded;
    p.topk_weights = call.topk_weights;
    p.topk = call.topk;
    p.E = call.E;
    if (family_int_groups(c.fam)) {
      hipError_t e = launch_group_sums_split(p.a, int(call.T), p.K, call.ws, call.stream);
      if (e != hipSuccess) return e;
    }
    const int tiles_n = int(call.N / bn);
    const int tiles_m = int(call.max_blocks);
    return launch_pingpong(p, c.fam, true, plan.cfg, dim3(unsigned(tiles_m * tiles_n)), tiles_m, tiles_n,
                           call.stream);
  }
  if (plan.kind == 1 || plan.kind == 2) {
    int n_cfg = 0;
    int bm, bn;
    if (plan.kind == 1) {
      const TiledCfg& tc = tiled_configs(&n_cfg)[plan.cfg];
      bm = 16 * tc.mw * tc.wm;
      bn = 16 * tc.ntw * tc.wn;
    } else {
      const PipeCfg& pc = pipe_configs(&n_cfg)[plan.cfg];
      bm = 16 * pc.mw * pc.wm;
      bn = 16 * pc.ntw * pc.wn;
    }
    auto launch = [&](dim3 grid, int tm, int tn) {
      return plan.kind == 1 ? launch_tiled(p, c.fam, moe, plan.cfg, grid, tm, tn, call.stream)
                            : launch_pipe(p, c.fam, moe, plan.cfg, grid, tm, tn, call.stream);
    };
    p.split = 1;
    p.units_per_split = p.k_units;
    const int tiles_n = int(call.N / bn);
    if (family_int_groups(c.fam)) {
      hipError_t e = launch_group_sums_split(p.a, int(moe ? call.T : call.M), p.K, call.ws, call.stream);
      if (e != hipSuccess) return e;
    }
    if (moe) {
      if (bm != call.block_m) return hipErrorInvalidValue;   // one workgroup row = one block
      p.M = int(call.T * call.topk);
      p.sorted_ids = call.sorted_ids;
      p.block_expert = call.block_expert;
      p.num_padded = call.num_padded;
      p.topk_weights = call.topk_weights;
      p.topk = call.topk;
      p.E = call.E;
      return launch(dim3(unsigned(tiles_n), unsigned(call.max_blocks)), int(call.max_blocks), tiles_n);
    }
    p.M = int(call.M);
    const int tiles_m = int((call.M + bm - 1) / bm);
    return launch(dim3(unsigned(tiles_m * tiles_n)), tiles_m, tiles_n);
  }
  int n_cfg = 0;
  const SkinnyCfg& sc = skinny_configs(&n_cfg)[plan.cfg];
  const int rows_per_block = 16 * sc.mb;
  if (plan.kind == 4 && !moe) {
    uint32_t* counters = nullptr;
    hipError_t e = stream_k_counters(call.stream, &counters);
    if (e != hipSuccess) return e;
    if (counters) {
      p.M = int(call.M);
      p.split = 1;
      p.units_per_split = p.k_units;
      p.sk_items = plan.sk_items;
      p.sk_slots = plan.sk_slots;
      p.sk_counters = counters;
      return launch_skinny_stream_k(p, c.fam, plan.cfg, plan.split, call.stream);
    }
    // every counter set is held by other streams: the plain small-M launch (no K split)
  }
  if (moe) {
    if (rows_per_block != call.block_m) return hipErrorInvalidValue;   // one row block = one block
    p.M = int(call.T * call.topk);
    p.sorted_ids = call.sorted_ids;
    p.block_expert = call.block_expert;
    p.num_padded = call.num_padded;
    p.topk_weights = call.topk_weights;
    p.topk = call.topk;
    p.E = call.E;
    p.split = 1;
    p.units_per_split = p.k_units;
    dim3 grid(unsigned(call.N / 16 / sc.ntw), unsigned(call.max_blocks), 1);
    return launch_skinny(p, c.fam, true, plan.cfg, grid, call.stream);
  }
  p.M = int(call.M);
  p.split = plan.kind == 4 ? 1 : plan.split;
  const int sk_units = int(call.K / k_unit(c));   // skinny units (128-k steps for block-scaled FP8)
  p.units_per_split = (sk_units + p.split - 1) / p.split;
  dim3 grid(unsigned(call.N / 16 / sc.ntw), unsigned((call.M + rows_per_block - 1) / rows_per_block),
            unsigned(p.split));
  hipError_t e = launch_skinny(p, c.fam, false, plan.cfg, grid, call.stream);
  if (e != hipSuccess || p.split == 1) return e;
  return launch_splitk_reduce(p, c.fam, call.stream);
}

// ---- library-owned scratch for hq_gemm_noalloc --------------------------------------------------
// One array per GPU (each device holds its own copy of a __device__ variable), alive until the
// process ends. Host code never passes `scratch` itself to a kernel or a copy: on the host that
// name is only a stand-in symbol, not a device address. The device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and is what the kernels
// receive, exactly as they receive a caller's workspace in hq_gemm.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace hq
