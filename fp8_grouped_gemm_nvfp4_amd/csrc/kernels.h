// kernels.h -- host-visible launch interfaces of the library's HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mxg.h"

namespace mxg {

enum { EPI_BF16 = 0, EPI_F32 = 1, EPI_SWIGLU_NVFP4 = 2, EPI_SWIGLU_BF16 = 3 };
enum { MODE_MASKED = 0, MODE_HETERO = 1, MODE_CONTIG = 2 };

// Masked layout: A [G, max_m, K], B [G, N, K], C [G, max_m, N].  For the fused
// SwiGLU epilogue N = 2I (W13 rows: gate [0, I), up [I, 2I)) and the outputs
// are the NVFP4 codes/scales of h [G, max_m, I] (plus optional fp32 dbg_h).
struct MaskedGemmArgs {
  const uint8_t* a;
  const uint8_t* a_sf;
  const uint8_t* b;
  const uint8_t* b_sf;
  void* out;
  const int32_t* masked_m;
  const float* alpha;   // [G] or NULL
  float alpha_scale;    // multiplies alpha[g]
  int G, max_m, N, K;
  int tiles_m, tiles_n, total_tiles;
  uint8_t* h_codes;
  uint8_t* h_sf;
  float* dbg_h;
  float* dbg_g1;        // SwiGLU epilogue: optional fp32 GEMM1 outputs [G, max_m, N] (gate | up)
  float g_h;
  // contiguous layout (MODE_CONTIG): A [max_m, K] and C [max_m, N] hold every group's rows,
  // group g from row row_start[g] (row_start [G + 1]); masked_m[g] counts its valid rows
  const int32_t* row_start;
  // SwiGLU epilogue: B holds W13 with gate and up rows interleaved in 16-row blocks
  // (gate rows [16 j, 16 j + 16) at [32 j, 32 j + 16), the matching up rows after them)
  int w13_il16;
  // the caller expects most groups to hold at most 8 valid rows (a decode batch: T * top_k
  // at most 4 E): the decode kernel then uses 8-row M tiles up to max_m = 16, a group with
  // more rows taking two (its weights streamed twice)
  int sparse_rows;
};

struct HeteroGroup {
  const uint8_t* a;
  const uint8_t* a_sf;
  const uint8_t* b;
  const uint8_t* b_sf;
  void* out;
  int M, N, K, ldc;
  float alpha;
  int tiles_m, tiles_n, tile_base;
};

// An item schedule of heterogeneous groups over the workgroups (numbered XCD by XCD):
// npat > 0 patterns, where workgroups [pat_start[p], pat_start[p + 1]) take pat_cnt[p][g]
// items of group g each, as contiguous ranges of the group's items in workgroup order; or
// npat = 0, round robin over the items in group order (item t to workgroup t % grid).
constexpr int MX_MAX_PAT = 16;
struct HeteroSchedule {
  int npat;
  int pat_start[MX_MAX_PAT + 1];
  unsigned char pat_cnt[MX_MAX_PAT][MXG_MAX_GROUPS];
};
// Longest-first deal of every group's tiles_m * tiles_n items (all items of group g at
// cost[g], groups in the given order) to the least-loaded of W workgroups, ties to the
// lower index, folded into patterns; npat = 0 when they do not fit the table (more than
// MX_MAX_PAT distinct count vectors, a count above 255, W above 4096, or more than 65,536
// items).  The result depends only on its inputs and is cached per input set.
void hetero_lpt_schedule(const HeteroGroup* grp, const double* cost, int G, int W, HeteroSchedule& out);

struct HeteroGemmArgs {
  HeteroGroup grp[MXG_MAX_GROUPS];
  int G;
  int total_tiles;
  HeteroSchedule sched;  // used by the streaming kernel's heterogeneous mode
};

// Heterogeneous groups on the scaled fp4 MFMA (power-of-two e4m3 scales): the groups in
// schedule order (tiles_m, tiles_n and tile_base filled in) and their item schedule.
struct MxGemmArgs {
  HeteroGroup grp[MXG_MAX_GROUPS];
  int bm[MXG_MAX_GROUPS];  // M tile of each group (128 or 256 rows)
  int G;
  HeteroSchedule sched;
};
hipError_t gemm_nvfp4_mx_hetero(HeteroGemmArgs p, int epi, int cu_limit, hipStream_t s);

template <int MODE> struct ArgsOf;
template <> struct ArgsOf<MODE_MASKED> { typedef MaskedGemmArgs type; };
template <> struct ArgsOf<MODE_HETERO> { typedef HeteroGemmArgs type; };
template <> struct ArgsOf<MODE_CONTIG> { typedef MaskedGemmArgs type; };

hipError_t gemm_nvfp4_masked(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s);
hipError_t gemm_nvfp4_hetero(HeteroGemmArgs p, int epi, int cu_limit, hipStream_t s);
// Decode-shaped masked GEMM (8- or 16-row M tiles, weights streamed into LDS by DMA);
// returns hipErrorNotSupported without launching for shapes it does not take.
hipError_t gemm_nvfp4_skinny(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s);
constexpr int SKINNY_MAX_M = 32;  // row capacity up to which the skinny kernel is used
// Larger masked groups (prefill): persistent weight-streaming kernel, 256-row M tiles;
// returns hipErrorNotSupported without launching for shapes it does not take.
hipError_t gemm_nvfp4_stream(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s);
// The same kernel over the contiguous layout (bf16 / fp32 outputs, N and K multiples of
// 128, at most STREAM_CONTIG_MAX_G groups); hipErrorNotSupported otherwise.
constexpr int STREAM_CONTIG_MAX_G = 512;
hipError_t gemm_nvfp4_contiguous(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s);
// The same kernel over heterogeneous groups (bf16 / fp32 outputs); hipErrorNotSupported for
// groups it does not take (N or K not a multiple of 128, unaligned output rows).
hipError_t gemm_nvfp4_stream_hetero(HeteroGemmArgs p, int epi, int cu_limit, hipStream_t s);

// Workgroups of `kernel` (with `threads` threads) resident on the device at once, over
// at most cu_limit CUs when cu_limit > 0; 0 on a runtime error.
int resident_grid(const void* kernel, int threads, int cu_limit);

// FP8 block-scaled GEMMs of the DeepSeek-V3-style expert path (masked layout).
struct Fp8GemmArgs {
  const uint8_t* a;     // GEMM1: e4m3 token rows [T, K]; GEMM2: bf16 h [G, max_m, K]
  const int32_t* a_tok; // GEMM1: the token of each expert row [G, max_m] (rows below masked_m)
  int tokens;           // GEMM1: rows of a (T)
  const float* a_s;     // GEMM1: fp32 [G, K/128, a_s_stride] (row scales, transposed); GEMM2: unused
  const uint8_t* b;     // e4m3 [G, N, K]
  const float* b_s;     // fp32 [G, N/128, K/128]
  void* out;            // GEMM1: bf16 h [G * max_m + 1, N/2] (the last row takes the stores of
                        // masked rows); GEMM2: fp32 [G, max_m, N]
  const int32_t* masked_m;
  int G, max_m, N, K;
  int a_s_stride;       // GEMM1: max_m rounded up to a multiple of 4
  int tiles_m, tiles_n, total_tiles;
  // h kept as two bf16 planes (hi = bf16(h), lo = bf16(h - hi)) in rows of 2 * (N/2):
  // GEMM1 writes both, GEMM2 runs over K = 2I with W2's K index wrapping at b_k = I
  int h_split;
  int b_k;              // GEMM2: K extent of W2 when h_split (else K)
  float* dbg_g1;        // GEMM1: optional fp32 outputs [G, max_m, N] (gate | up), promoted sums
};
constexpr int fp8_scale_stride(int max_m) { return (max_m + 3) / 4 * 4; }
hipError_t gemm_fp8_swiglu(Fp8GemmArgs p, int cu_limit, hipStream_t s);
hipError_t gemm_bf16_fp8w(Fp8GemmArgs p, int cu_limit, hipStream_t s);

// NVFP4-weight x bf16-activation GEMV (W4A16) for decode batches: out[m, n] = g_w *
// sum_k x[m, k] * dec(W)[n, k].  hipErrorNotSupported (nothing launched) unless
// 1 <= M <= GEMV_MAX_M, M * K <= GEMV_MAX_MK and K % 1024 == 0.
constexpr int GEMV_MAX_M = 4;
constexpr int GEMV_MAX_MK = 32768;  // fp16 activation elements held in LDS
struct GemvArgs {
  const uint16_t* x;    // bf16 [M, K]
  const uint8_t* w;     // NVFP4 codes [N, K/2]
  const uint8_t* w_sf;  // e4m3 scales [N, K/16]
  void* out;            // [M, N] bf16 or fp32
  float g_w;
  int M, K, N;
};
hipError_t gemv_nvfp4_w4a16(GemvArgs p, int epi, int cu_limit, hipStream_t s);

// Quantization, routing, dispatch, gather and combine.
hipError_t quantize_nvfp4(const void* x, int x_dtype, long rows, int K, float g, uint8_t* codes,
                          uint8_t* sf, hipStream_t s);
hipError_t route_noaux(const float* logits, const float* bias, int T, int E, int n_group,
                       int topk_group, int top_k, float rsf, int32_t* ids, float* w,
                       hipStream_t s);
hipError_t dispatch(const int32_t* ids, int T, int E, int top_k, int max_m, int32_t* masked_m,
                    int32_t* row, int32_t* offsets, hipStream_t s);
// contiguous layout: count[e] tokens of expert e from row start[e] (start[E + 1], each
// start a multiple of align), row[t, j] the absolute row of slot (t, j)
hipError_t dispatch_contiguous(const int32_t* ids, int T, int E, int top_k, int align, int32_t* start,
                               int32_t* count, int32_t* row, hipStream_t s);
hipError_t dispatch_quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x, const int32_t* ids,
                                          int top_k, int E, int max_m, int32_t* masked_m, int32_t* row,
                                          uint8_t* a, uint8_t* a_sf, hipStream_t s);
hipError_t quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x, const int32_t* ids,
                                 const int32_t* row, int top_k, int max_m, uint8_t* a,
                                 uint8_t* a_sf, hipStream_t s);
// FP8 expert rows: a_tok [E, max_m] receives the token of every dispatched expert row,
// a_s the row scales transposed: [E, H/128, fp8_scale_stride(max_m)] (rows below
// masked_m; the rest are left as they were).
hipError_t fp8_expert_rows(const float* xs, int T, int H, const int32_t* ids, const int32_t* row, int top_k,
                           int E, int max_m, const int32_t* masked_m, int32_t* a_tok, float* a_s,
                           hipStream_t s);
hipError_t interleave_w13(const uint8_t* src, uint8_t* dst, int E, int I, int row_bytes, hipStream_t s);
hipError_t combine(const float* o, const int32_t* ids, const int32_t* row, const float* w, int T,
                   int H, int top_k, int max_m, uint16_t* y, hipStream_t s);

}  // namespace mxg
