/*
 * mxg.h -- C ABI of the MI355X (gfx950) block-scaled grouped-GEMM / MoE library.
 *
 * Conventions shared by every entry point
 *  - Pointers named as device pointers must point into HBM of the current HIP
 *    device; host pointers are marked "host".  The caller owns every buffer;
 *    the library allocates nothing inside a call.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns before the GPU work ends.  Inputs must stay alive and
 *    unmodified, and outputs unread, until the stream has reached that point.
 *  - Errors are return codes (mxg_status); nothing aborts or throws.  Argument
 *    checks run on the host before any HIP call, so a rejected call touches no
 *    GPU state.  mxg_last_error() gives a thread-local message for the last
 *    failure on the calling thread.
 *  - NVFP4 tensors: e2m1 codes, two per byte, element 2i in the low nibble,
 *    row-major [rows, K/2]; one e4m3fn scale byte per 16 consecutive K
 *    elements, row-major [rows, K/16]; one fp32 global dequantization scale
 *    per tensor.  A value decodes as e2m1 * e4m3(scale) * global.
 *  - All device pointers must be 16-byte aligned.
 *  - Calls on one stream are ordered; calls on different streams that share
 *    an output race.
 */
#ifndef MXG_H
#define MXG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXG_OK = 0,
  MXG_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad combination */
  MXG_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle  */
  MXG_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  MXG_ERR_HIP = 4          /* a HIP launch or runtime call failed             */
} mxg_status;

/* MXG_E4M3_POW2 (sf_dtype only): e4m3 scale bytes that the caller declares to be positive
 * powers of two, 2^-9 .. 2^8 (codes (u + 7) << 3 for u in [-6, 8], and 0x01, 0x02, 0x04);
 * see mx_grouped_gemm. */
typedef enum { MXG_E2M1 = 1, MXG_E4M3 = 2, MXG_BF16 = 3, MXG_F32 = 4, MXG_E4M3_POW2 = 5 } mxg_dtype;

/* Static text for a status code ("unknown status" for anything else). */
const char* mxg_status_string(int status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* mxg_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int mxg_version(void);

/*
 * Masked grouped NT GEMM over NVFP4 operands.
 * Source: "The CuteDSL Gamble: Chasing Kernel Efficiency on Blackwell GPUs",
 * section "The Message" -- grouped_gemm_nt_masked(lhs=(data, sf), rhs=(data,
 * sf), out, masked_m, ab_dtype, sf_dtype, c_dtype, sf_vec_size, sm_count), a
 * masked batched GEMM with scale factors and optional alpha at output.
 *
 *   out[g, m, n] = alpha[g] * sum_k dec(A)[g, m, k] * dec(B)[g, n, k]
 *   for g < G, m < min(max(masked_m[g], 0), max_m), n < N, accumulated in fp32.
 *
 *   a, a_sf    device, A codes [G, max_m, K/2], scales [G, max_m, K/16]
 *   b, b_sf    device, B codes [G, N, K/2],     scales [G, N, K/16]
 *   alpha      device fp32 [G] (product of the A and B global scales), or NULL = 1
 *   masked_m   device int32 [G], valid rows per group; clamped to [0, max_m]
 *   out        device [G, max_m, N] of c_dtype (bf16, round to nearest even, or
 *              fp32); rows at or beyond masked_m[g] are never written
 *   ab_dtype = MXG_E2M1, sf_dtype = MXG_E4M3 or MXG_E4M3_POW2 (same kernels here),
 *   sf_vec_size = 16; c_dtype = MXG_BF16 or MXG_F32.
 *   cu_limit   0 = use the whole GPU; > 0 caps the number of resident
 *              workgroups to about that many CUs (sm_count analog)
 * Requirements: G in [1, 65535], max_m >= 1, N >= 1, K % 64 == 0 (else
 * MXG_ERR_UNSUPPORTED).  Rows of A at or beyond masked_m are never read.
 */
int mx_grouped_gemm_masked(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                           const uint8_t* b_sf, const float* alpha, const int32_t* masked_m,
                           void* out, int G, int max_m, int N, int K, int ab_dtype,
                           int sf_dtype, int c_dtype, int sf_vec_size, int cu_limit,
                           void* stream);

/*
 * Grouped NVFP4 NT GEMM over the contiguous (expert-sorted) layout for prefill:
 * the rows of all groups sit in one A [M_total, K], group g's from row
 * group_start[g], with aligned padding between groups.
 * Source: "Helion Pretuned Kernels" README, kernel table row grouped_gemm_deepgemm
 * (DeepGEMM's packed contiguous A layout, heterogeneous per-group M, aligned
 * padding excluded from the result).
 *
 *   out[r, n] = alpha[g] * sum_k dec(A)[r, k] * dec(B)[g, n, k]
 *   for r in [group_start[g], group_start[g] + count[g]), n < N, fp32 sums
 *
 *   a, a_sf      device A codes [M_total, K/2], scales [M_total, K/16]
 *   b, b_sf      device B codes [G, N, K/2], scales [G, N, K/16]
 *   alpha        device fp32 [G], or NULL = 1
 *   group_start  device int32 [G + 1], non-decreasing, group_start[G] <= M_total
 *   count        device int32 [G], valid rows of each group
 *   out          device [M_total, N] of c_dtype; padding rows are never written
 * The kernel clamps group_start to [0, M_total] and to a running maximum, and
 * count[g] to [0, group_start[g + 1] - group_start[g]], so no access leaves the
 * M_total rows whatever those arrays hold.  Requirements: G <= 512, N % 128 == 0,
 * K % 128 == 0 (else MXG_ERR_UNSUPPORTED); dtypes as in mx_grouped_gemm_masked.
 */
int mx_grouped_gemm_contiguous(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                               const uint8_t* b_sf, const float* alpha, const int32_t* group_start,
                               const int32_t* count, void* out, int G, int M_total, int N, int K,
                               int ab_dtype, int sf_dtype, int c_dtype, int sf_vec_size, int cu_limit,
                               void* stream);

/*
 * One group of a heterogeneous grouped GEMM: its own (M, N, K), operand and
 * output pointers (device), alpha by value, and the output row stride ldc in
 * elements (0 = N).
 * Source: "Helion Pretuned Kernels" README, kernel table row grouped_gemm
 * (heterogeneous grouped NT cases with M/N tails) and the benchmark notes
 * (device pointer tables set up before graph capture); "llm-assisted-kernel-
 * dev" README, NVFP4 grouped GEMM table (group metadata moved from runtime GPU
 * reads into launch-time specialization).
 */
typedef struct {
  int M, N, K, ldc;
  float alpha;
  const uint8_t* a;    /* [M, K/2]  */
  const uint8_t* a_sf; /* [M, K/16] */
  const uint8_t* b;    /* [N, K/2]  */
  const uint8_t* b_sf; /* [N, K/16] */
  void* out;           /* [M, ldc] of c_dtype */
} mxg_group_desc;

#define MXG_MAX_GROUPS 32

/*
 * Heterogeneous grouped NVFP4 NT GEMM: out_g = alpha_g * A_g * B_g^T for every
 * group.  `groups` is a HOST array of G descriptors (copied into the kernel's
 * launch arguments, so nothing is read from device metadata); the pointers
 * inside are device pointers.  G in [1, MXG_MAX_GROUPS]; each group needs
 * M >= 0, N >= 1, K % 64 == 0.  Same dtype rules as mx_grouped_gemm_masked.
 * The descriptors travel by value in the launch arguments, which a captured graph
 * records with the launch: the table the pages set up on the device before graph
 * capture is, here, part of the captured kernel node, and the cap of 32 groups keeps
 * it inside the kernel-argument space.  Larger group counts with one shared N and K
 * are the masked (mx_grouped_gemm_masked) or contiguous layouts.
 * sf_dtype = MXG_E4M3_POW2 declares that every scale byte of every group is a positive
 * power of two.  When every group with rows has N and K multiples of 128 and 16-byte
 * aligned output rows (out and ldc), the call runs on the scaled fp4 MFMA: each
 * power-of-two scale is exactly an e8m0 MFMA scale, so the result is the same
 * exact-product fp32 sum as with general scales, at up to twice the rate of the fp16 MFMA
 * the general decode uses (two fp4 MFMAs per 128-K block, one per 16-element half of each
 * 32-element MFMA scale block, each at four times the fp16 rate).  Otherwise the general
 * kernels run.  Scale bytes outside the
 * declared set give wrong results (a zero scale counts as 2^-127, a mantissa is
 * dropped), never an out-of-bounds access.
 * Source for the power-of-two path: the per-16 e4m3 scales of NVFP4 do not map onto the
 * per-32 e8m0 scales of the MX MFMA in general; a K split around the scaled MFMA does
 * when the scales are powers of two.
 */
int mx_grouped_gemm(const mxg_group_desc* groups, int G, int ab_dtype, int sf_dtype,
                    int c_dtype, int sf_vec_size, int cu_limit, void* stream);

/*
 * NVFP4-weight x bf16-activation GEMV for decode batches (W4A16).
 * Source: "Helion Pretuned Kernels" README, kernel table row nvfp4_gemv (NVFP4
 * decode GEMV at M = 1, W4A4 and W4A16 variants, Llama-3 / Qwen (N, K) shapes);
 * single-stream decode in "The CuteDSL Gamble".
 *
 *   out[m, n] = g_w * sum_k x[m, k] * dec(W)[n, k]   for m < M, n < N, fp32 sums
 *
 *   x          device bf16 [M, K], row stride K
 *   w, w_sf    device NVFP4 weight codes [N, K/2], e4m3 scales [N, K/16]
 *   g_w        host fp32 global dequantization scale of W
 *   out        device [M, N] of c_dtype (MXG_BF16, round to nearest even, or MXG_F32)
 *   cu_limit   as in mx_grouped_gemm_masked
 * Requirements: 1 <= M <= 4, M * K <= 32768 and K % 1024 == 0 (else
 * MXG_ERR_UNSUPPORTED); N >= 1.  The activations are used as fp16 after
 * scaling each row by a power of two chosen from its largest magnitude, which
 * is exact for every element at least 2^-28 times that magnitude.
 */
int mx_gemv_nvfp4_w4a16(const void* x, int M, int K, const uint8_t* w, const uint8_t* w_sf, float g_w,
                        void* out, int N, int c_dtype, int cu_limit, void* stream);

/*
 * NVFP4 quantization of rows of x [rows, K] (x_dtype MXG_BF16 or MXG_F32,
 * device) with global dequantization scale g > 0 (host fp32).  Per 16-element
 * block, in fp32 with round-to-nearest at every step:
 *   S = e4m3_rne_sat(amax / (6 g));  d = value(S) * g;
 *   code_i = e2m1_rne_sat(x_i * (1 / d))   (all codes keep the sign of x_i;
 *   a block whose S rounds to 0 gets zero codes)
 * Source: NVFP4 as e2m1 values with block scale factors and a global scale
 * ("The CuteDSL Gamble", "Input Knowledge Required"); the per-step recipe is a
 * reading of that description.  codes [rows, K/2], sf [rows, K/16] (device).
 * K % 16 == 0 required.
 */
int mx_quantize_nvfp4(const void* x, int x_dtype, long rows, int K, float g, uint8_t* codes,
                      uint8_t* sf, void* stream);

/*
 * DeepSeek-V3 no-aux routing.  Source: "llm-assisted-kernel-dev" README,
 * mixture-of-experts table, moe_fibench_ref.py row (sigmoid(logits) + bias,
 * grouped top-k, routed_scaling_factor).  Per token t:
 *   s_e  = fp32 of the fp64 value 1 / (1 + exp(-logit_e))
 *   sb_e = s_e + bias_e (fp32)
 *   group score = fp32 sum of the two largest sb in each of n_group contiguous
 *   groups of E / n_group experts; keep the topk_group best groups; take the
 *   top_k best sb among their experts; ties go to the lower index; slot j
 *   holds the j-th best.  w_j = fp32(fp32(s_j / sum_slots s) * rsf), the sum
 *   taken in slot order.
 *   logits device fp32 [T, E]; bias device fp32 [E];
 *   topk_ids device int32 [T, top_k]; topk_w device fp32 [T, top_k].
 * Supported: E == 256, n_group in {1, 2, 4, 8}, 1 <= topk_group <= n_group,
 * 1 <= top_k <= 8, top_k <= topk_group * E / n_group.
 */
int moe_route_noaux(const float* logits, const float* bias, int T, int E, int n_group,
                    int topk_group, int top_k, float rsf, int32_t* topk_ids, float* topk_w,
                    void* stream);

/*
 * Token-to-expert permutation for the contiguous layout (stable counting sort in
 * token order, each expert's rows starting at a multiple of align).
 * Source: "Helion Pretuned Kernels" README, kernel table row grouped_gemm_deepgemm
 * (DeepGEMM's packed contiguous A layout with aligned padding per group); the
 * permutation is the one the masked layout's masked_m implies ("The CuteDSL
 * Gamble", "The Message"), with the groups packed one after another.
 *   count[e]        = number of tokens routed to e
 *   group_start[e]  = sum over e' < e of count[e'] rounded up to a multiple of align;
 *                     group_start[E] = the total rows (with padding)
 *   row[t, j]       = group_start[e] + number of tokens t' < t routed to e, e = topk_ids[t, j]
 * topk_ids device int32 [T, top_k] (distinct per token, in [0, E)); group_start
 * device int32 [E + 1]; count device int32 [E]; row device int32 [T, top_k].
 * 1 <= align <= 4096; T * top_k + E * align < 2^31.
 */
int moe_dispatch_contiguous(const int32_t* topk_ids, int T, int E, int top_k, int align,
                            int32_t* group_start, int32_t* count, int32_t* row, void* stream);

/*
 * Token-to-expert permutation for the masked layout (stable counting sort in
 * token order).  Source: the per-expert valid row count masked_m of
 * grouped_gemm_nt_masked ("The CuteDSL Gamble", "The Message").
 *   row[t, j]   = number of tokens t' < t routed to expert topk_ids[t, j]
 *   masked_m[e] = min(number of tokens routed to e, max_m)
 *   offsets[e]  = sum over e' < e of masked_m[e'] (exclusive scan; offsets[E] =
 *                 the number of slots kept), or nothing when offsets is NULL
 * A slot whose row is >= max_m does not fit the capacity and is dropped by the
 * later stages.  topk_ids device int32 [T, top_k] (distinct per token, in
 * [0, E)); masked_m device int32 [E]; row device int32 [T, top_k]; offsets
 * device int32 [E + 1] or NULL.
 */
int moe_dispatch(const int32_t* topk_ids, int T, int E, int top_k, int max_m, int32_t* masked_m,
                 int32_t* row, int32_t* offsets, void* stream);

/*
 * NVFP4-quantize the bf16 activations x [T, H] (global scale g_x, same recipe
 * as mx_quantize_nvfp4) and scatter each token's codes/scales to every expert
 * row it was dispatched to: a[e, row, :], a_sf[e, row, :] for each slot with
 * row < max_m.  a [E, max_m, H/2], a_sf [E, max_m, H/16] (device).
 * H % 64 == 0 required.
 * Source: activations "quantized on the fly" to NVFP4 ahead of the masked grouped
 * GEMM ("The CuteDSL Gamble", "Input Knowledge Required": NVFP4 as 4-bit values
 * with block scale factors; "The Message": the per-expert masked layout that
 * grouped_gemm_nt_masked reads).
 */
int moe_quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x,
                              const int32_t* topk_ids, const int32_t* row, int top_k, int E,
                              int max_m, uint8_t* a, uint8_t* a_sf, void* stream);

/* moe_dispatch (without offsets) followed by moe_quantize_gather_nvfp4, in one launch
 * when T * top_k <= 256 (the decode batches; larger batches run the two kernels).
 * Source: as those two calls ("The CuteDSL Gamble", "The Message" and "Input Knowledge
 * Required"); a single-stream decode step is where launch count matters ("Context: The
 * Performance Crisis").  Outputs, layouts
 * and requirements are those of the two calls (masked_m [E], row [T, top_k], a, a_sf),
 * bit for bit.  For callers of small decode steps, which save a launch and the wait
 * between the two. */
int moe_dispatch_quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x,
                                       const int32_t* topk_ids, int top_k, int E, int max_m,
                                       int32_t* masked_m, int32_t* row, uint8_t* a, uint8_t* a_sf,
                                       void* stream);

/* Precision of moe_expert_forward. */
typedef enum { MXG_MOE_FP8_BLOCK128 = 1, MXG_MOE_NVFP4 = 2, MXG_MOE_FP8_BLOCK128_F32H = 3 } mxg_moe_precision;

/* Row order of W13 (and of its scale rows).
 *   MXG_W13_STACKED: gate rows [0, I), then up rows [I, 2I).
 *   MXG_W13_INTERLEAVED16: gate and up rows interleaved in blocks of 16: rows
 *     [32 j, 32 j + 16) hold gate rows [16 j, 16 j + 16) and rows [32 j + 16, 32 j + 32)
 *     the matching up rows, so every 32-row slice holds the gate and up columns of
 *     the same 16 h columns.
 * Source: Helion "pretuned_kernels" README, interleaved_swiglu row (a projection
 * with interleaved gate/value columns feeding a compact SwiGLU epilogue).  The
 * block of 16 rows (one MFMA tile) is this library's reading of "interleaved". */
typedef enum { MXG_W13_STACKED = 0, MXG_W13_INTERLEAVED16 = 16 } mxg_w13_layout;

/* Reorders the rows of a stacked W13 array (codes [E, 2I, H/2] or scales
 * [E, 2I, H/16], row_bytes = H/2 or H/16) into the MXG_W13_INTERLEAVED16 order:
 * dst row r of expert e is src row (r mod 32 < 16 ? 16 (r / 32) + r mod 32 :
 * I + 16 (r / 32) + r mod 32 - 16).  src and dst are device arrays of E * 2I *
 * row_bytes bytes that must not overlap.  Requires I % 16 == 0, row_bytes % 4 == 0,
 * 4-byte aligned pointers (else MXG_ERR_INVALID_ARG / MXG_ERR_UNSUPPORTED).
 * Asynchronous on `stream`; a one-off weight preparation, not part of a layer step. */
int moe_interleave_w13(const uint8_t* src, uint8_t* dst, int E, int I, int row_bytes, void* stream);

/*
 * The routed expert computation of one MoE layer: gather -> GEMM1 (W13, gate
 * rows [0, I) and up rows [I, 2I)) -> SwiGLU h = silu(gate) * up -> GEMM2 (W2)
 * -> weighted combine y[t] = sum_j w[t, j] * o[topk_ids[t, j], row[t, j]].
 * Source: "llm-assisted-kernel-dev" README, mixture-of-experts table
 * (moe_fibench_ref.py: FP8 e4m3fn hidden states and both weight sets with
 * block scales; moe_fp8fpX_fused.py: GEMM1 -> SwiGLU -> GEMM2, BF16 default).
 *
 * MXG_MOE_FP8_BLOCK128:
 *   x        e4m3 codes [T, H], x_scale fp32 [T, H/128] (1x128 blocks)
 *   w13      e4m3 [E, 2I, H], w13_scale fp32 [E, 2I/128, H/128]
 *   w2       e4m3 [E, H, I],  w2_scale fp32 [E, H/128, I/128]
 *   h        = bf16 (round to nearest even) of silu(gate) * up
 * MXG_MOE_FP8_BLOCK128_F32H: as MXG_MOE_FP8_BLOCK128 with a full-precision
 *   intermediate: the fp32 h is kept as hi = bf16(h) and lo = bf16(h - hi)
 *   (about 16 significant bits) and GEMM2 runs over both planes, o = (hi + lo) W2,
 *   at about twice GEMM2's cost.  Source: "llm-assisted-kernel-dev" README,
 *   moe_fibench_ref.py (experts in full precision) and the fp32 expert variants of
 *   moe_fp8fpX_fused.py; the hi/lo split is this library's reading of it.
 * MXG_MOE_NVFP4:
 *   x        bf16 [T, H], quantized in the layer with global scale g_x
 *   w13      codes [E, 2I, H/2], w13_scale e4m3 [E, 2I, H/16], g_w13 fp32 [E]
 *   w2       codes [E, H, I/2],  w2_scale e4m3 [E, H, I/16],  g_w2 fp32 [E]
 *   h        fp32 silu(gate) * up, requantized to NVFP4 with global scale g_h
 * Both: GEMM outputs accumulate in fp32; GEMM2 results stay fp32 until the
 * combine, which sums in slot order in fp32 and rounds y once to bf16.
 *   topk_ids/topk_w/masked_m/row as produced by moe_route_noaux + moe_dispatch
 *   (device); y device bf16 [T, H].
 *   dbg_h    optional device fp32 [E, max_m, I]: NVFP4 only, receives the
 *            pre-quantization intermediate for the rows it computes (NULL in
 *            production; y is bit-identical either way).
 *   dbg_g1   optional device fp32 [E, max_m, 2I]: receives GEMM1's fp32 outputs (alpha
 *            applied) for the rows it computes, gate in columns [0, I) and up in [I, 2I)
 *            whatever the W13 layout (NULL in production; y is bit-identical either way)
 *   w13_layout  mxg_w13_layout of w13 and its scales; MXG_W13_INTERLEAVED16 is
 *            NVFP4 only (MXG_ERR_UNSUPPORTED for the FP8 precisions).  The layer's
 *            result does not depend on the layout: y is bit-identical for the same
 *            logical weights.
 * Requirements: H % 128 == 0, I % 128 == 0, 1 <= top_k <= 8, max_m >= 1; both FP8
 * precisions also E <= 1024 and T*H, 4*max_m*I and 2*I*H below 2^32 (the GEMMs
 * address token rows, an expert's rows and its weights with 32-bit byte offsets), else
 * MXG_ERR_UNSUPPORTED.
 * Workspace: ws of at least moe_expert_forward_workspace_size(desc) bytes,
 * 256-byte aligned, device; its regions hold the expert rows' activations (FP8:
 * their tokens, the rows being read from x), h and the GEMM2 output (offsets from
 * moe_expert_forward_workspace_layout).
 */
typedef struct {
  int precision;
  int T, H, I, E, top_k, max_m;
  const void* x;
  const float* x_scale;
  float g_x;
  const uint8_t* w13;
  const void* w13_scale;
  const float* g_w13;
  const uint8_t* w2;
  const void* w2_scale;
  const float* g_w2;
  float g_h;
  const int32_t* topk_ids;
  const float* topk_w;
  const int32_t* masked_m;
  const int32_t* row;
  uint16_t* y;
  float* dbg_h;
  int w13_layout;
  float* dbg_g1;
} mxg_moe_desc;

/* Bytes of workspace moe_expert_forward needs for this descriptor (0 on a bad
 * descriptor). */
size_t moe_expert_forward_workspace_size(const mxg_moe_desc* desc);

/* Byte offsets (host array of 6) of the workspace regions:
 *   [0] expert rows (FP8: int32 [E, max_m], the token of each row below masked_m, whose
 *       row of x GEMM1 reads; NVFP4: the gathered codes [E, max_m, H/2])
 *   [1] their scales (FP8: fp32 [E, H/128, max_m rounded up to a multiple of 4], i.e.
 *       transposed; NVFP4: e4m3 [E, max_m, H/16])
 *   [2] h (FP8: bf16 [E, max_m, I] followed by one scratch row; FP8 F32H: bf16 [E, max_m, 2I],
 *       hi in columns [0, I) and lo in [I, 2I), then one scratch row; NVFP4: codes [E, max_m, I/2])
 *   [3] h scales (FP8: unused; NVFP4: e4m3 [E, max_m, I/16])
 *   [4] GEMM2 output fp32 [E, max_m, H]
 *   [5] total size
 * Returns MXG_OK or MXG_ERR_INVALID_ARG. */
int moe_expert_forward_workspace_layout(const mxg_moe_desc* desc, size_t* offsets);

int moe_expert_forward(const mxg_moe_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes moe_expert_forward_noalloc can serve (192 MiB per GPU). */
#define MXG_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)

/*
 * moe_expert_forward with no workspace argument, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels run on the same workspace regions
 * (moe_expert_forward_workspace_layout), placed in a device array the library holds on
 * every GPU it runs on until the process ends (MXG_NOALLOC_SCRATCH_BYTES of workspace;
 * its address is looked up once per device, on the first call there).  Nothing is
 * allocated or freed in the call.  y and every output are those of moe_expert_forward,
 * bit for bit.
 *   A layer whose workspace exceeds MXG_NOALLOC_SCRATCH_BYTES returns MXG_ERR_WORKSPACE
 *   with nothing launched.  At E = 256, H = 7168, I = 2048 it serves max_m up to 16
 *   (132 MiB for NVFP4, 157 MiB for FP8): decode batches.  The fp32 GEMM2 output alone
 *   takes E * max_m * H * 4 bytes.
 *   All calls on one GPU share its array, which keeps the last call's contents; no
 *   region needs to start at zero (each call writes every row it later reads).  Calls
 *   that overlap on one GPU (other streams, or host threads without ordering) race on
 *   the array and corrupt each other's results: order them on one stream.
 */
int moe_expert_forward_noalloc(const mxg_moe_desc* desc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXG_H */
