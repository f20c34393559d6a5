/*
 * hq.h -- C ABI of the MI355X (gfx950) fused-dequantization quantized GEMM library (libhq.so).
 *
 * Computes Y = X . dequant(Wq, scales, zero-points)^T for dense layers and for the MoE grouped
 * GEMM, with three weight/activation pairs:
 *   WNA16  : group-wise INT4 weights (symmetric, or unsigned with a zero-point) x bf16 activations
 *   W8A8   : per-channel INT8 weights x per-token INT8 activations
 *   W4A8   : MXFP4 weights (e2m1 + e8m0 block scales) x per-token FP8 e4m3 activations
 *
 * Source of the method: "Humming: vLLM and Ant Group Open-Source a General-Purpose Kernel
 * Library for Quantized Inference" (English announcement page). Its section "A unified
 * quantization representation" describes one standard quantization description in which
 * weight format, scale granularity, scale dtype and zero-points are separate parameters and
 * activations have their own format; `hq_quant_desc` is that description. Section "Tuning and
 * JIT compilation per workload" describes preprocessing that validates parameters and repacks
 * tensors into the target kernel's layout (`hq_prepack_weights`), and inference that combines
 * the preprocessed weights with runtime activations (`hq_gemm`, `hq_moe_grouped_gemm`). The
 * MoE token sort (`hq_moe_align`) is not described by the page; it is the step that feeds the
 * "Indexed" MoE path of section "Results: kernel microbenchmarks" (rows gathered through a
 * sorted index).
 *
 * General conventions
 *   - Ownership: the caller allocates every buffer. Host buffers for the prepack; device
 *     buffers (e.g. from PyTorch) for everything else. The library keeps no pointer after a
 *     call returns and allocates no device memory (hq_gemm_noalloc's scratch is a static device
 *     array of the library, not an allocation).
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream). Device calls only enqueue
 *     work and never synchronize. `hq_moe_grouped_gemm` reads the padded row count on the
 *     device, so no host round trip is needed between the two MoE calls.
 *   - Errors: every argument is checked on the host before any launch. A non-HQ_OK status
 *     leaves outputs untouched and sets a thread-local message (`hq_last_error`). A failed
 *     launch returns HQ_ERR_HIP.
 *   - Device pointers must be 16-byte aligned. Shapes: N % 16 == 0 and K a multiple of the
 *     format's K unit (128 for WNA16 and W4A8, 64 for W8A8); other shapes are rejected with
 *     HQ_ERR_UNSUPPORTED (the caller pads).
 */
#ifndef HQ_H_
#define HQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* hq_stream_t; /* a hipStream_t */

typedef enum {
  HQ_OK = 0,
  HQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, misaligned pointer      */
  HQ_ERR_UNSUPPORTED = 2,      /* valid description, but a combination/shape not provided  */
  HQ_ERR_WORKSPACE = 3,        /* workspace or output buffer smaller than required          */
  HQ_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed                */
} hq_status;

typedef enum {
  HQ_W_INT4_SYM = 0,   /* two's-complement INT4 in [-8, 7], packed 2 per byte, low nibble = even k */
  HQ_W_UINT4_ASYM = 1, /* unsigned INT4 in [0, 15] with a uint4 zero-point per (n, group)          */
  HQ_W_INT8_SYM = 2,   /* two's-complement INT8 (codes in [-127, 127]), fp32 scale per channel      */
  HQ_W_FP4_E2M1 = 3,   /* OCP MX e2m1, packed 2 per byte, low nibble = even k                      */
  HQ_W_FP8_E4M3 = 4,   /* OCP e4m3 [N, K]: one fp32 scale per 128 x 128 block (group_size 128) or,
                          with bf16 activations, per output channel (group_size 0)              */
  HQ_W_UINT2_ASYM = 5, /* unsigned INT2 in [0, 3], packed 4 per byte (code k in bits 2 (k % 4)),
                          with a uint2 zero-point per (n, group)                                  */
  HQ_W_UINT3_ASYM = 6  /* unsigned INT3 in [0, 7], each row a little-endian bit string (code k in
                          bits 3k .. 3k + 2), with a uint3 zero-point per (n, group)              */
} hq_weight_fmt;

typedef enum {
  HQ_SCALE_BF16 = 0, /* one bf16 scale per (n, group)                         */
  HQ_SCALE_FP32 = 1, /* one fp32 scale per output channel n (group = whole K) */
  HQ_SCALE_E8M0 = 2  /* one e8m0 byte per (n, 32-element block): 2^(b - 127)  */
} hq_scale_dtype;

typedef enum {
  HQ_ACT_BF16 = 0,             /* bf16 [M, K] row-major, no activation scale          */
  HQ_ACT_INT8_PER_TOKEN = 1,   /* int8 [M, K] row-major + fp32 scale per row [M]      */
  HQ_ACT_FP8E4M3_PER_TOKEN = 2, /* OCP e4m3 [M, K] row-major + fp32 scale per row [M] */
  HQ_ACT_MXFP4 = 3,             /* OCP MX e2m1 [M, K/2] (low nibble = even k) + e8m0 byte per
                                   (row, 32-element block) [M, K/32]                        */
  HQ_ACT_MXFP8 = 4,             /* OCP MX e4m3 [M, K] + e8m0 byte per (row, 32-element block)
                                   [M, K/32]                                                 */
  HQ_ACT_FP8E4M3_BLOCK128 = 5   /* OCP e4m3 [M, K] + fp32 scale per (row, 128-k block) [M, K/128] */
} hq_act_fmt;

typedef enum {
  HQ_OUT_BF16 = 0,     /* bf16 [M, N] row-major                                           */
  HQ_OUT_INT32_ACC = 1 /* W8A8 only: the raw int32 accumulator sum_k xq*wq, [M, N] (test) */
} hq_out_fmt;

/* The standard quantization description (one per layer). Fields are int32 for a stable ABI. */
typedef struct {
  uint32_t struct_size;   /* = sizeof(hq_quant_desc)                                         */
  int32_t weight_fmt;     /* hq_weight_fmt                                                   */
  int32_t group_size;     /* along K: 128 (INT4), 32 (FP4/MX), 0 = per channel (INT8)        */
  int32_t scale_dtype;    /* hq_scale_dtype                                                  */
  int32_t has_zero_point; /* 1 for HQ_W_UINT4_ASYM, else 0                                   */
  int32_t act_fmt;        /* hq_act_fmt                                                      */
  int32_t out_fmt;        /* hq_out_fmt                                                      */
  int32_t compute_flags;  /* HQ_COMPUTE_* bits, 0 = none                                     */
} hq_quant_desc;

/* Batch invariance (a compute option of the announcement's section "Tuning and JIT compilation
 * per workload"): every output row is a function of its own activation row (and the weights)
 * alone, bit for bit, whatever M (dense) or T (MoE) and whatever the other rows. The library
 * then runs one fixed kernel configuration per (format, N) for all M -- the skinny kernel, two
 * 16-row blocks per workgroup, no K split across workgroups -- and ignores tuning tables and
 * overrides; MoE calls need block_m = 32 (what hq_moe_block_m returns with the flag). The cost
 * is the tuned kernels' speed at large M (measured about 2x slower for W4A16 at M = 8192). */
#define HQ_COMPUTE_BATCH_INVARIANT 1

/* Stream-K (the announcement's section "Device-specific performance tuning" names Stream-K
 * scheduling among its tuning controls): for a dense call whose rows fit one row block of the
 * small-M kernel (M <= 16 for most formats), the (16-channel tile group, K unit) work items are cut
 * into one equal contiguous range per workgroup, about one workgroup per CU, instead of one
 * workgroup per tile group -- so no CU idles when the tile groups do not divide evenly over the
 * CUs. A tile group split between workgroups is summed by the last of them to finish (a per-group
 * arrival counter in library-owned device memory, reset by that workgroup), in a fixed order: the
 * result is deterministic, but not bit-identical to a call without the flag. The workspace holds
 * the partial tiles (hq_gemm_workspace_bytes with the flag). The counters are kept per stream (up
 * to 16 streams per GPU; calls on further streams run without Stream-K), so calls on one stream
 * never share them with calls on another. Two things must not run at the same time: two replays
 * of one captured HIP graph holding such a call, or such a replay and other work of the stream it
 * was captured on. Other calls, other shapes and MoE ignore the flag. Ignored with
 * HQ_COMPUTE_BATCH_INVARIANT. Measured on MI355X it is slower at the dense W4A16 decode shape
 * (N=14336, K=4096, M=1: 17.1 us against 9.6 us without it): a workgroup then works through its
 * two pieces one after the other, and decode time is set by load latency and total bytes, not by
 * the per-CU share -- so it is off unless asked for. */
#define HQ_COMPUTE_STREAM_K 2

/*
 * Supported combinations (others return HQ_ERR_UNSUPPORTED):
 *   INT4_SYM   + BF16 scale, group 128, no zero-point + ACT_BF16              -> OUT_BF16
 *   UINT4_ASYM + BF16 scale, group 128, zero-point    + ACT_BF16              -> OUT_BF16
 *   INT8_SYM   + FP32 scale, group 0                  + ACT_INT8_PER_TOKEN    -> OUT_BF16 | OUT_INT32_ACC
 *   FP4_E2M1   + E8M0 scale, group 32                 + ACT_FP8E4M3_PER_TOKEN -> OUT_BF16
 *   FP4_E2M1   + E8M0 scale, group 32                 + ACT_MXFP8             -> OUT_BF16
 *   FP4_E2M1   + E8M0 scale, group 32                 + ACT_MXFP4  (W4A4)     -> OUT_BF16
 *   FP4_E2M1   + E8M0 scale, group 32                 + ACT_BF16   (W4A16)    -> OUT_BF16
 *   FP8_E4M3   + FP32 scale, 128 x 128 blocks         + ACT_FP8E4M3_BLOCK128  -> OUT_BF16
 *              (N % 128 == 0, K % 128 == 0)
 *   INT8_SYM   + FP32 scale, group 0                  + ACT_BF16   (W8A16)    -> OUT_BF16
 *   FP8_E4M3   + FP32 scale, group 0                  + ACT_BF16   (W8A16)    -> OUT_BF16
 *              (the 8-bit WnA16 widths; K % 128 == 0)
 *   UINT2_ASYM + BF16 scale, group 128, zero-point    + ACT_BF16   (W2A16)    -> OUT_BF16
 *   UINT3_ASYM + BF16 scale, group 128, zero-point    + ACT_BF16   (W3A16)    -> OUT_BF16
 *              (the 2- and 3-bit WnA16 widths; 3-bit weights on the small-M kernel at every M)
 * MoE grouped GEMM and grouped GEMM: every combination above with OUT_BF16 -- ACT_BF16 (INT4 sym /
 * asym, FP4, INT8, FP8 weights), per-token activations (INT8 W8A8, FP4 + ACT_FP8E4M3_PER_TOKEN
 * W4A8), block-scaled FP8 (a_scale = fp32 [T, K/128]) and MX activations (ACT_MXFP4, ACT_MXFP8:
 * a_scale = the e8m0 bytes [T, K/32]); activation scales are one row per token.
 * Every combination also takes compute_flags = HQ_COMPUTE_BATCH_INVARIANT.
 */

/* ---------------------------------------------------------------------------------------------
 * Per-token dynamic activation quantization (device), the step before the W8A8 and W4A8 GEMMs.
 * The announcement's section "Tuning and JIT compilation per workload" lists per-token input
 * scales among the compute options, and its section "End-to-end performance" credits tokenwise
 * FP8 activations; the rule implemented is symmetric absmax scaling per row:
 *   s_tok[m] = fp32(max_k |x[m,k]| / Q), Q = 127 (INT8) or 448 (e4m3); 1 for an all-zero row
 *   v        = fp32(x[m,k] / s_tok[m])            (IEEE binary32 division)
 *   INT8     : xq = clamp(round_half_even(v), -127, 127)
 *   e4m3     : xq = nearest OCP e4m3 code to clamp(v, -448, 448), ties to the even code
 *              (negative values that round to zero give -0, 0x80)
 * act_fmt  HQ_ACT_INT8_PER_TOKEN or HQ_ACT_FP8E4M3_PER_TOKEN (the desc act_fmt of the GEMM), or
 *          HQ_ACT_FP8E4M3_BLOCK128: the e4m3 rule above on every 128-k block of a row (s_tok then
 *            receives fp32 [M, K/128], xq e4m3 [M, K]; K % 128 == 0). Or
 *          HQ_ACT_MXFP8: the same rule with e4m3 elements -- e = floor(log2 max|x|) - 8, code =
 *            e4m3 of clamp(x * 2^-e, -448, 448) as above; xq is e4m3 [M, K], s_tok receives
 *            the e8m0 bytes [M, K/32] (cast); K % 32 == 0. Or
 *          HQ_ACT_MXFP4 (W4A4), which follows the OCP Microscaling rule per row and block of 32 k:
 *            e = floor(log2 max|x|) - 2 clamped to [-127, 127] (-127 for a zero block),
 *            scale byte e + 127, code = nearest e2m1 to x * 2^-e (ties to even, saturating at 6;
 *            a value that rounds to zero gives +0). xq then holds packed e2m1 [M, K/2] (low
 *            nibble = even k) and s_tok receives the e8m0 bytes [M, K/32] through its pointer
 *            (cast); K % 32 == 0.
 * x        bf16 [M, K] row-major (device, 16-byte aligned); K % 8 == 0
 * xq       int8 / e4m3 bytes [M, K] row-major (device, 16-byte aligned), the GEMM's `a`
 * s_tok    fp32 [M] (device), the GEMM's `a_scale`
 * Inputs with NaN or infinity give unspecified codes. M == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
hq_status hq_quantize_activations(int32_t act_fmt, int64_t M, int64_t K, const void* x, void* xq,
                                  float* s_tok, hq_stream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Weight prepack (host).  Standard-format inputs, all host memory, row-major:
 *   wq      INT4/FP4: uint8 [E, N, K/2] (two codes per byte, low nibble = even k)
 *           UINT2   : uint8 [E, N, K/4] (four codes per byte, code k in bits 2 (k % 4) .. +1)
 *           UINT3   : uint8 [E, N, 3K/8] (each row a little-endian bit string, code k in bits
 *                     3k .. 3k + 2)
 *           INT8    : int8  [E, N, K];  FP8: e4m3 bytes [E, N, K]
 *   scales  BF16: uint16 bf16 bits [E, N, K/group];  FP32: float [E, N] (per channel: INT8,
 *           and FP8 with group_size 0) or float [E, N/128, K/128] (FP8 block scales);
 *           E8M0: uint8 [E, N, K/32]
 *   zeros   UINT4_ASYM / UINT3_ASYM / UINT2_ASYM only: uint8 [E, N, K/group], values 0..15 / 0..7 /
 *           0..3; NULL otherwise
 * E = 1 for a dense layer, E = number of experts for MoE (experts stacked).
 * Output: `out` (host, `hq_prepacked_bytes` bytes) receives the weights rearranged into the
 * MFMA operand order of the kernels. The layout is private to this library version; the caller
 * only copies it to the device unchanged. A bijective rearrangement: no value is rounded.
 * Returns HQ_ERR_WORKSPACE if out_bytes is too small. Codes outside a format's range are not
 * checked (INT8 -128 is accepted and used as is).
 * ------------------------------------------------------------------------------------------- */
size_t hq_prepacked_bytes(const hq_quant_desc* desc, int64_t E, int64_t N, int64_t K);
hq_status hq_prepack_weights(const hq_quant_desc* desc, int64_t E, int64_t N, int64_t K,
                             const void* wq, const void* scales, const void* zeros,
                             void* out, size_t out_bytes);

/* ---------------------------------------------------------------------------------------------
 * Dense GEMM (device):  y[m, n] = epilogue( sum_k a[m, k] * w[n, k] ),  0 <= m < M, 0 <= n < N
 *   a        activations, format desc->act_fmt, [M, K] row-major (device)
 *   a_scale  fp32 [M] per-token scales for INT8/FP8 activations (device); NULL for BF16.
 *            MXFP4 / MXFP8 activations: the e8m0 block-scale bytes, uint8 [M, K/32] row-major,
 *            passed through this pointer (cast) -- the activations' own scale tensor
 *   w_packed the prepacked weights of ONE layer (E = 1) (device)
 *   y        [M, N] row-major, bf16 or int32 per desc->out_fmt (device)
 *   ws       scratch of at least hq_gemm_workspace_bytes(desc, M, N, K) bytes (device); may be
 *            NULL when that size is 0. Contents on entry do not matter.
 * Epilogues:  WNA16: bf16( sum_g s[n,g] * sum_{k in g} a*(q - z) )  (fp32 accumulation; the
 *                    same for the 2-bit UINT2 codes)
 *             W8A8 : bf16( float(acc) * a_scale[m] * s_ch[n] ),  acc exact int32
 *             W4A8 : bf16( a_scale[m] * sum_k e4m3(a) * e2m1(q) * 2^(e - 127) ) (fp32 accumulation)
 *             W4A4 : bf16( sum_k e2m1(a) 2^(ea - 127) * e2m1(q) 2^(e - 127) ) (fp32 accumulation;
 *                    weights as W4A8, desc act_fmt HQ_ACT_MXFP4)
 *             MXFP4 weights with bf16 activations (desc act_fmt HQ_ACT_BF16), "W4A16-MXFP4":
 *                    bf16( sum_k a * e2m1(q) 2^(e - 127) ) (each weight dequantized exactly to
 *                    bf16, fp32 accumulation); also for hq_moe_grouped_gemm / hq_grouped_gemm
 *             FP8 W8A8 with block scales (HQ_W_FP8_E4M3 + HQ_ACT_FP8E4M3_BLOCK128; a_scale =
 *                    fp32 [M, K/128]): bf16( sum_g a_scale[m, g] * s_w[n/128, g] *
 *                    sum_{k in g} e4m3(a) * e4m3(q) ) (fp32 accumulation)
 *             INT8 or FP8 e4m3 weights with bf16 activations ("W8A16"; the page's WnA16 at an
 *                    8-bit weight width, section "Results: kernel microbenchmarks"):
 *                    bf16( s_ch[n] * sum_k a * q ), q the INT8 integer or the e4m3 value (each
 *                    exact in bf16), fp32 accumulation
 *             W4A8 with MXFP8 activations (desc act_fmt HQ_ACT_MXFP8):
 *                    bf16( sum_k e4m3(a) 2^(ea - 127) * e2m1(q) 2^(e - 127) ) (fp32 accumulation)
 * All bf16 results use round-to-nearest-even. M = 0 is a no-op returning HQ_OK.
 * ------------------------------------------------------------------------------------------- */
size_t hq_gemm_workspace_bytes(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K);
hq_status hq_gemm(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K,
                  const void* a, const float* a_scale, const void* w_packed,
                  void* y, void* ws, size_t ws_bytes, hq_stream_t stream);

/* ---------------------------------------------------------------------------------------------
 * hq_gemm without a workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (minus ws / ws_bytes), kernels, results and errors as hq_gemm, bit for bit. The
 * split-K partials and activation group sums that hq_gemm keeps in the caller's workspace live in
 * a library-owned device array of HQ_NOALLOC_SCRATCH_BYTES per GPU instead, held until the
 * process ends. Nothing is allocated by the call.
 *   - A call whose workspace (hq_gemm_workspace_bytes) exceeds HQ_NOALLOC_SCRATCH_BYTES fails
 *     with HQ_ERR_WORKSPACE before any launch.
 *   - The array keeps the last call's contents; no call depends on them (every byte a launch
 *     reads from it was written by the same call).
 *   - Calls on one GPU share its array: calls that overlap in time on one GPU (different
 *     streams or threads) race and give unspecified results. Serialize them.
 * ------------------------------------------------------------------------------------------- */
#define HQ_NOALLOC_SCRATCH_BYTES (16u << 20)
hq_status hq_gemm_noalloc(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K,
                          const void* a, const float* a_scale, const void* w_packed,
                          void* y, hq_stream_t stream);

/* ---------------------------------------------------------------------------------------------
 * MoE token sort / expert offsets (device).
 *   topk_ids       int32 [T, topk] expert of each (token, slot); ids outside [0, E) are routed
 *                  nowhere (no row is produced for them)
 *   block_m        rows per GEMM block, a multiple of 16 in [16, 256]
 * Outputs (device, caller-allocated):
 *   sorted_ids     int32 [hq_moe_align_capacity(T, topk, E, block_m)]: for each expert e in
 *                  order, the flat indices f = t*topk + j routed to e in ascending order, then
 *                  sentinel T*topk up to the next multiple of block_m. Entries past num_padded
 *                  are unspecified.
 *   block_expert   int32 [capacity / block_m]: expert of each block of block_m sorted rows;
 *                  blocks past num_padded / block_m hold -1 (no expert; the grouped GEMM
 *                  skips them)
 *   expert_offsets int32 [E + 1]: exclusive prefix sum of the padded per-expert counts
 *   num_padded     int32 [1]: total padded rows (= expert_offsets[E])
 *   ws             scratch of hq_moe_align_workspace_bytes(...) bytes (contents irrelevant)
 * The result is deterministic (stable order), independent of thread scheduling.
 * ------------------------------------------------------------------------------------------- */
size_t hq_moe_align_capacity(int64_t T, int32_t topk, int32_t E, int32_t block_m);
size_t hq_moe_align_workspace_bytes(int64_t T, int32_t topk, int32_t E, int32_t block_m);
hq_status hq_moe_align(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                       int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* expert_offsets, int32_t* num_padded,
                       void* ws, size_t ws_bytes, hq_stream_t stream);

/* Recommended block_m for a grouped GEMM over T tokens (the tuning table's choice). */
int32_t hq_moe_block_m(const hq_quant_desc* desc, int64_t T, int32_t topk, int32_t E,
                       int64_t N, int64_t K);

/* ---------------------------------------------------------------------------------------------
 * MoE grouped GEMM (device): bf16 activations with INT4 group weights (WNA16), MXFP4 weights or
 * per-channel INT8 / FP8 weights (W8A16), per-token 8-bit activations with INT8 (W8A8) or MXFP4
 * (W4A8) weights, block-scaled FP8 activations and weights (the page's FP8 W8A8 with blockwise
 * scaling, whose MoE form it compares in section "W8A8 / W4A8 / W4A4"), or MXFP4 / MXFP8
 * activations with MXFP4 weights (W4A4, W4A8-MXFP8; same section):
 *   y[f, :] = (topk_weights ? topk_weights[f] : 1) * a[f / topk, :] . dequant(W_{e(f)})^T
 * for every flat index f = t*topk + j that hq_moe_align routed to a valid expert e(f), with the
 * dense path's epilogue per format (W8A8: bf16(float(acc) * a_scale[t] * s_ch_e[n] * weight),
 * W4A8: bf16(acc * a_scale[t] * weight); block-scaled FP8: the block scales of token t and the
 * expert per 128-k step, then * weight). Rows of y for unrouted f are not written.
 *   a             [T, K] row-major (device): bf16, or int8 / e4m3 codes
 *   a_scale       fp32 [T] per-token scales for INT8 / FP8 activations, fp32 [T, K/128] for
 *                 block-scaled FP8, e8m0 bytes [T, K/32] for MXFP4 / MXFP8 activations
 *                 (required); NULL for bf16
 *   w_packed      prepacked weights of all E experts (hq_prepack_weights with E experts)
 *   sorted_ids, block_expert, num_padded: outputs of hq_moe_align with the same T, topk, E,
 *                 block_m (device)
 *   block_m       16, 32, 64 or 128 (HQ_ERR_UNSUPPORTED otherwise); 128 needs K % 128 == 0 and
 *                 N % 128 == 0 (HQ_ERR_UNSUPPORTED otherwise)
 *   topk_weights  fp32 [T*topk] or NULL (device)
 *   y             bf16 [T*topk, N] row-major (device)
 *   ws            hq_moe_gemm_workspace_bytes(...) bytes (may be 0 / NULL)
 * ------------------------------------------------------------------------------------------- */
size_t hq_moe_gemm_workspace_bytes(const hq_quant_desc* desc, int64_t T, int32_t topk,
                                   int32_t E, int64_t N, int64_t K, int32_t block_m);
hq_status hq_moe_grouped_gemm(const hq_quant_desc* desc, int64_t T, int32_t topk, int32_t E,
                              int64_t N, int64_t K, const void* a, const float* a_scale,
                              const void* w_packed, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              int32_t block_m, const float* topk_weights, void* y,
                              void* ws, size_t ws_bytes, hq_stream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped GEMM (device), the formats of hq_moe_grouped_gemm: the "Grouped" MoE path of the announcement's section
 * "Results: kernel microbenchmarks", for activations that arrive already grouped by expert.
 *   y[r, :] = a[r, :] . dequant(W_e)^T   for r in [expert_offsets[e], expert_offsets[e+1])
 *             (times a_scale[r], and W8A8's channel scale, for 8-bit activations)
 *   a               [R, K] row-major (device), bf16 or int8 / e4m3 codes
 *   a_scale         fp32 [R] per-row scales for INT8 / FP8 activations (required), NULL for bf16
 *   w_packed        prepacked weights of all E experts (hq_prepack_weights with E experts)
 *   expert_offsets  int32 [E + 1] (device): non-decreasing, 0 <= offsets[0], offsets[E] <= R.
 *                   Each range is clipped to [0, R); rows in no range are not written. Offsets
 *                   that overlap break the contract: the rows concerned get unspecified values,
 *                   and no access leaves the buffers.
 *   y               bf16 [R, N] row-major (device), same row order as a
 *   ws              hq_grouped_gemm_workspace_bytes(...) bytes, 256-byte aligned (required)
 * The row block size comes from the tuning table (rows per expert = R / E); the call runs a
 * small index kernel (the padded row index of each expert, into ws) and the grouped GEMM kernels
 * of hq_moe_grouped_gemm with every row as its own token. Asynchronous on `stream`.
 * ------------------------------------------------------------------------------------------- */
size_t hq_grouped_gemm_workspace_bytes(const hq_quant_desc* desc, int64_t R, int32_t E, int64_t N, int64_t K);
hq_status hq_grouped_gemm(const hq_quant_desc* desc, int64_t R, int32_t E, int64_t N, int64_t K,
                          const void* a, const float* a_scale, const void* w_packed,
                          const int32_t* expert_offsets, void* y, void* ws, size_t ws_bytes,
                          hq_stream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Tuning (host). The built-in table picks a kernel per range of M (the announcement's section
 * "Tuning and JIT compilation per workload"); a tuning table measured on the device by
 * `python -m quantized_gemm_prepacked_amd.autotune` (the roadmap's autotune, run offline) takes
 * precedence for the shapes it lists. Text, one entry per line ('#' comments):
 *     <family> <asym 0|1> <N> <K> <max_m> <kind> <cfg> <split>
 * family wna16 | wna2 | wna3 | w8a8 | w4a8 | w4a4 | w4a8mx | mxw4a16 | fp8b | w8a16 | f8a16; kind 0
 * skinny, 1 LDS-tiled, 2 async-pipelined, 3 ping-pong; cfg indexes that kind's configurations
 * (hq_kernel_config_count); split = K splits of the skinny kernel, -1 = the heuristic's. A dense
 * call uses the first entry of its family, asym, N and K whose max_m >= M, if that configuration
 * fits the shape (the skinny kernel's few-row configurations fit only M <= 4); otherwise the
 * built-in choice. The table is process-wide:
 *   hq_load_tuning_table(path)  replaces it (NULL clears it); a malformed line fails with
 *                               HQ_ERR_INVALID_ARGUMENT and leaves the table unchanged.
 *   Without a call, the file named by the environment variable HQ_TUNING_FILE (if any) is read
 *   at the first dense plan. Loading while other threads launch GEMMs is safe (locked).
 * hq_gemm_plan reports the (kind, cfg, split) a dense call of that shape would run; with
 * HQ_COMPUTE_STREAM_K it may report kind 4 (the small-M kernel's configuration cfg in Stream-K
 * form) with split = the number of workgroups.
 * ------------------------------------------------------------------------------------------- */
hq_status hq_load_tuning_table(const char* path);
hq_status hq_gemm_plan(const hq_quant_desc* desc, int64_t M, int64_t N, int64_t K, int32_t* kind,
                       int32_t* cfg, int32_t* split);
int32_t hq_kernel_config_count(int32_t kind);

/* Thread-local message describing the last non-HQ_OK status of this thread ("" if none). */
const char* hq_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t hq_version(void);

/* ---------------------------------------------------------------------------------------------
 * MoE layer stages around the two grouped GEMMs (device). The announcement's section "Results:
 * kernel microbenchmarks" times MoE as gate_up plus Down; a full layer for T tokens is
 *   hq_moe_align(topk_ids, T, topk, E, block_m, ...)
 *   hq_moe_grouped_gemm(desc, T, topk, E, 2I, H, x [T, H], ...)           -> gate_up [T*topk, 2I]
 *   hq_moe_silu_mul(T*topk, I, gate_up, act)                              -> act     [T*topk, I]
 *   hq_moe_grouped_gemm(desc, T*topk, 1, E, H, I, act, ..., same sorted_ids / block_expert /
 *                       num_padded / block_m, topk_weights [T*topk])      -> down    [T*topk, H]
 *   hq_moe_combine(T, topk, E, H, topk_ids, down, out)                    -> out     [T, H]
 * The Down call treats every routed row as its own token (topk = 1): the alignment's flat ids
 * t*topk + k then index `act` rows directly, and the router weight of each row is applied in the
 * Down GEMM's epilogue.
 *
 * hq_moe_silu_mul: act[r, i] = bf16(silu(g) * u), g = gate_up[r, i], u = gate_up[r, I + i],
 *   silu(g) = g / (1 + exp(-g)) = g * e / (1 + e) with e = exp(g) for g < 0, fp32 arithmetic. gate_up bf16 [R, 2I], act bf16 [R, I], both
 *   16-byte aligned; I % 8 == 0. Rows that no GEMM wrote (ids outside [0, E)) give unspecified
 *   values that the later stages never read.
 * hq_moe_combine: out[t, n] = bf16(sum_k y[t*topk + k, n]) over the k with topk_ids[t, k] in
 *   [0, E), summed in fp32 in k order; a token with no valid k gets zeros. y bf16 [T*topk, N],
 *   out bf16 [T, N], 16-byte aligned; N % 8 == 0; topk_ids int32 [T, topk] (device).
 * hq_moe_silu_mul_quantize: the gated activation quantized per row for a Down GEMM with 8-bit
 *   activations (the page's tokenwise FP8 activations, section "End-to-end inference
 *   performance"), in one launch: bit for bit hq_moe_silu_mul(R, I, gate_up, act) followed by
 *   hq_quantize_activations(act_fmt, R, I, act, act_q, act_scale), without the bf16 act tensor.
 *   act_fmt HQ_ACT_FP8E4M3_PER_TOKEN or HQ_ACT_INT8_PER_TOKEN; gate_up bf16 [R, 2I] (16-byte
 *   aligned), act_q e4m3 / int8 [R, I] (16-byte aligned), act_scale fp32 [R]; I % 8 == 0.
 * ------------------------------------------------------------------------------------------- */
hq_status hq_moe_silu_mul(int64_t R, int64_t I, const void* gate_up, void* act, hq_stream_t stream);
hq_status hq_moe_silu_mul_quantize(int32_t act_fmt, int64_t R, int64_t I, const void* gate_up, void* act_q,
                                   float* act_scale, hq_stream_t stream);
hq_status hq_moe_combine(int64_t T, int32_t topk, int32_t E, int64_t N, const int32_t* topk_ids,
                         const void* y, void* out, hq_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HQ_H_ */
