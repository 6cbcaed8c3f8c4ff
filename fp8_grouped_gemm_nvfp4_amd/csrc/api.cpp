// api.cpp -- the C ABI (include/mxg.h): host-side argument validation, status
// reporting and kernel dispatch.  Every check runs before the first HIP call,
// so a rejected call leaves the GPU untouched.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kernels.h"

// Device scratch of moe_expert_forward_noalloc: one copy on every GPU the library runs
// on, held until the process ends.  Its name is a host-side stand-in in host code, never
// a device address: the address on each device comes from hipGetSymbolAddress, taken
// once per device with that device current.  The array holds MXG_NOALLOC_SCRATCH_BYTES
// of workspace plus a 64 KiB tail that no region reaches.
static __device__ __align__(256) uint8_t scratch[MXG_NOALLOC_SCRATCH_BYTES + (64u << 10)];

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MXG_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MXG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_nvfp4_types(int ab_dtype, int sf_dtype, int c_dtype, int sf_vec_size) {
  if (ab_dtype != MXG_E2M1 || (sf_dtype != MXG_E4M3 && sf_dtype != MXG_E4M3_POW2) || sf_vec_size != 16)
    return fail(MXG_ERR_UNSUPPORTED,
                "only ab_dtype=E2M1, sf_dtype=E4M3 or E4M3_POW2, sf_vec_size=16 is supported (got %d, %d, %d)",
                ab_dtype, sf_dtype, sf_vec_size);
  if (c_dtype != MXG_BF16 && c_dtype != MXG_F32)
    return fail(MXG_ERR_UNSUPPORTED, "c_dtype must be BF16 or F32 (got %d)", c_dtype);
  return MXG_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // address of `scratch` on each device, once looked up

// The scratch array's address on the current device (looked up on the first call there).
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_expert_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moe_expert_forward_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(MXG_ERR_HIP, "moe_expert_forward_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MXG_OK;
}

}  // namespace

extern "C" {

const char* mxg_status_string(int status) {
  switch (status) {
    case MXG_OK: return "MXG_OK";
    case MXG_ERR_INVALID_ARG: return "MXG_ERR_INVALID_ARG";
    case MXG_ERR_UNSUPPORTED: return "MXG_ERR_UNSUPPORTED";
    case MXG_ERR_WORKSPACE: return "MXG_ERR_WORKSPACE";
    case MXG_ERR_HIP: return "MXG_ERR_HIP";
    default: return "unknown status";
  }
}

const char* mxg_last_error(void) { return g_err; }

int mxg_version(void) { return 100; }

int mx_grouped_gemm_masked(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                           const uint8_t* b_sf, const float* alpha, const int32_t* masked_m,
                           void* out, int G, int max_m, int N, int K, int ab_dtype, int sf_dtype,
                           int c_dtype, int sf_vec_size, int cu_limit, void* stream) {
  if (!a || !a_sf || !b || !b_sf || !masked_m || !out)
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm_masked: null pointer");
  if (G < 1 || G > 65535 || max_m < 1 || N < 1 || K < 1 || cu_limit < 0)
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm_masked: bad sizes G=%d max_m=%d N=%d K=%d", G,
                max_m, N, K);
  int st = check_nvfp4_types(ab_dtype, sf_dtype, c_dtype, sf_vec_size);
  if (st) return st;
  if (K % 64 != 0) return fail(MXG_ERR_UNSUPPORTED, "mx_grouped_gemm_masked: K %% 64 != 0 (K=%d)", K);
  if (!aligned16(a) || !aligned16(b) || !aligned16(out) || !aligned16(a_sf) || !aligned16(b_sf))
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm_masked: misaligned pointer");
  if ((long long)G * max_m * N >= (1LL << 40))
    return fail(MXG_ERR_UNSUPPORTED, "mx_grouped_gemm_masked: problem too large");
  mxg::MaskedGemmArgs p{};
  p.a = a; p.a_sf = a_sf; p.b = b; p.b_sf = b_sf; p.out = out;
  p.masked_m = masked_m; p.alpha = alpha; p.alpha_scale = 1.0f;
  p.G = G; p.max_m = max_m; p.N = N; p.K = K;
  int epi = c_dtype == MXG_BF16 ? mxg::EPI_BF16 : mxg::EPI_F32;
  return hip_status(mxg::gemm_nvfp4_masked(p, epi, cu_limit, (hipStream_t)stream),
                    "mx_grouped_gemm_masked launch");
}

int mx_grouped_gemm_contiguous(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                               const float* alpha, const int32_t* group_start, const int32_t* count, void* out,
                               int G, int M_total, int N, int K, int ab_dtype, int sf_dtype, int c_dtype,
                               int sf_vec_size, int cu_limit, void* stream) {
  if (!a || !a_sf || !b || !b_sf || !group_start || !count || !out)
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm_contiguous: null pointer");
  if (G < 1 || M_total < 1 || N < 1 || K < 1 || cu_limit < 0)
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm_contiguous: bad sizes G=%d M_total=%d N=%d K=%d", G,
                M_total, N, K);
  int st = check_nvfp4_types(ab_dtype, sf_dtype, c_dtype, sf_vec_size);
  if (st) return st;
  if (G > mxg::STREAM_CONTIG_MAX_G || N % 128 != 0 || K % 128 != 0)
    return fail(MXG_ERR_UNSUPPORTED, "mx_grouped_gemm_contiguous: needs G <= %d, N %% 128 == 0, K %% 128 == 0",
                mxg::STREAM_CONTIG_MAX_G);
  if (!aligned16(a) || !aligned16(b) || !aligned16(out) || !aligned16(a_sf) || !aligned16(b_sf))
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm_contiguous: misaligned pointer");
  mxg::MaskedGemmArgs p{};
  p.a = a; p.a_sf = a_sf; p.b = b; p.b_sf = b_sf; p.out = out;
  p.masked_m = count; p.alpha = alpha; p.alpha_scale = 1.0f; p.row_start = group_start;
  p.G = G; p.max_m = M_total; p.N = N; p.K = K;
  int epi = c_dtype == MXG_BF16 ? mxg::EPI_BF16 : mxg::EPI_F32;
  return hip_status(mxg::gemm_nvfp4_contiguous(p, epi, cu_limit, (hipStream_t)stream),
                    "mx_grouped_gemm_contiguous launch");
}

int mx_grouped_gemm(const mxg_group_desc* groups, int G, int ab_dtype, int sf_dtype, int c_dtype,
                    int sf_vec_size, int cu_limit, void* stream) {
  if (!groups) return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: null descriptor array");
  if (G < 1 || G > MXG_MAX_GROUPS)
    return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: G=%d outside [1, %d]", G, MXG_MAX_GROUPS);
  if (cu_limit < 0) return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: cu_limit < 0");
  int st = check_nvfp4_types(ab_dtype, sf_dtype, c_dtype, sf_vec_size);
  if (st) return st;
  mxg::HeteroGemmArgs p{};
  p.G = G;
  for (int g = 0; g < G; g++) {
    const mxg_group_desc& d = groups[g];
    if (d.M < 0 || d.N < 1 || d.K < 1 || d.ldc < 0)
      return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: group %d has bad sizes", g);
    if (d.K % 64 != 0) return fail(MXG_ERR_UNSUPPORTED, "mx_grouped_gemm: group %d K %% 64 != 0", g);
    int ldc = d.ldc ? d.ldc : d.N;
    if (ldc < d.N) return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: group %d ldc < N", g);
    if (d.M > 0 && (!d.a || !d.a_sf || !d.b || !d.b_sf || !d.out))
      return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: group %d null pointer", g);
    if (d.M > 0 && (!aligned16(d.a) || !aligned16(d.b) || !aligned16(d.a_sf) || !aligned16(d.b_sf)))
      return fail(MXG_ERR_INVALID_ARG, "mx_grouped_gemm: group %d misaligned pointer", g);
    mxg::HeteroGroup& q = p.grp[g];
    q.a = d.a; q.a_sf = d.a_sf; q.b = d.b; q.b_sf = d.b_sf; q.out = d.out;
    q.M = d.M; q.N = d.N; q.K = d.K; q.ldc = ldc; q.alpha = d.alpha;
  }
  int epi = c_dtype == MXG_BF16 ? mxg::EPI_BF16 : mxg::EPI_F32;
  if (sf_dtype == MXG_E4M3_POW2) {
    const hipError_t e = mxg::gemm_nvfp4_mx_hetero(p, epi, cu_limit, (hipStream_t)stream);
    if (e != hipErrorNotSupported) return hip_status(e, "mx_grouped_gemm launch (power-of-two scales)");
  }
  return hip_status(mxg::gemm_nvfp4_hetero(p, epi, cu_limit, (hipStream_t)stream),
                    "mx_grouped_gemm launch");
}

int mx_gemv_nvfp4_w4a16(const void* x, int M, int K, const uint8_t* w, const uint8_t* w_sf, float g_w,
                        void* out, int N, int c_dtype, int cu_limit, void* stream) {
  if (!x || !w || !w_sf || !out) return fail(MXG_ERR_INVALID_ARG, "mx_gemv_nvfp4_w4a16: null pointer");
  if (M < 1 || K < 1 || N < 1 || cu_limit < 0)
    return fail(MXG_ERR_INVALID_ARG, "mx_gemv_nvfp4_w4a16: bad sizes M=%d K=%d N=%d", M, K, N);
  if (c_dtype != MXG_BF16 && c_dtype != MXG_F32)
    return fail(MXG_ERR_UNSUPPORTED, "mx_gemv_nvfp4_w4a16: c_dtype must be BF16 or F32 (got %d)", c_dtype);
  if (M > mxg::GEMV_MAX_M || (long long)M * K > mxg::GEMV_MAX_MK || K % 1024 != 0)
    return fail(MXG_ERR_UNSUPPORTED, "mx_gemv_nvfp4_w4a16: needs M <= %d, M * K <= %d, K %% 1024 == 0 (M=%d K=%d)",
                mxg::GEMV_MAX_M, mxg::GEMV_MAX_MK, M, K);
  if (!aligned16(x) || !aligned16(w) || !aligned16(w_sf) || !aligned16(out))
    return fail(MXG_ERR_INVALID_ARG, "mx_gemv_nvfp4_w4a16: misaligned pointer");
  mxg::GemvArgs p{};
  p.x = (const uint16_t*)x; p.w = w; p.w_sf = w_sf; p.out = out; p.g_w = g_w;
  p.M = M; p.K = K; p.N = N;
  int epi = c_dtype == MXG_BF16 ? mxg::EPI_BF16 : mxg::EPI_F32;
  return hip_status(mxg::gemv_nvfp4_w4a16(p, epi, cu_limit, (hipStream_t)stream), "mx_gemv_nvfp4_w4a16 launch");
}

int mx_quantize_nvfp4(const void* x, int x_dtype, long rows, int K, float g, uint8_t* codes,
                      uint8_t* sf, void* stream) {
  if (!x || !codes || !sf) return fail(MXG_ERR_INVALID_ARG, "mx_quantize_nvfp4: null pointer");
  if (rows < 0 || K < 16) return fail(MXG_ERR_INVALID_ARG, "mx_quantize_nvfp4: bad sizes");
  if (K % 16 != 0) return fail(MXG_ERR_UNSUPPORTED, "mx_quantize_nvfp4: K %% 16 != 0");
  if (x_dtype != MXG_BF16 && x_dtype != MXG_F32)
    return fail(MXG_ERR_UNSUPPORTED, "mx_quantize_nvfp4: x_dtype must be BF16 or F32");
  if (!(g > 0.0f) || g == __builtin_inff())
    return fail(MXG_ERR_INVALID_ARG, "mx_quantize_nvfp4: global scale must be finite and > 0");
  if (!aligned16(x) || ((uintptr_t)codes & 7u))
    return fail(MXG_ERR_INVALID_ARG, "mx_quantize_nvfp4: misaligned pointer");
  return hip_status(mxg::quantize_nvfp4(x, x_dtype, rows, K, g, codes, sf, (hipStream_t)stream),
                    "mx_quantize_nvfp4 launch");
}

int moe_route_noaux(const float* logits, const float* bias, int T, int E, int n_group,
                    int topk_group, int top_k, float rsf, int32_t* topk_ids, float* topk_w,
                    void* stream) {
  if (!logits || !bias || !topk_ids || !topk_w)
    return fail(MXG_ERR_INVALID_ARG, "moe_route_noaux: null pointer");
  if (T < 0 || E < 1 || n_group < 1 || topk_group < 1 || top_k < 1)
    return fail(MXG_ERR_INVALID_ARG, "moe_route_noaux: bad sizes");
  if (E != 256) return fail(MXG_ERR_UNSUPPORTED, "moe_route_noaux: E must be 256 (got %d)", E);
  if (n_group != 1 && n_group != 2 && n_group != 4 && n_group != 8)
    return fail(MXG_ERR_UNSUPPORTED, "moe_route_noaux: n_group must be 1, 2, 4 or 8");
  if (topk_group > n_group) return fail(MXG_ERR_INVALID_ARG, "moe_route_noaux: topk_group > n_group");
  if (top_k > 8) return fail(MXG_ERR_UNSUPPORTED, "moe_route_noaux: top_k > 8");
  if (top_k > topk_group * (E / n_group))
    return fail(MXG_ERR_INVALID_ARG, "moe_route_noaux: top_k exceeds the experts of the kept groups");
  if (!aligned16(logits) || !aligned16(bias))
    return fail(MXG_ERR_INVALID_ARG, "moe_route_noaux: misaligned pointer");
  return hip_status(mxg::route_noaux(logits, bias, T, E, n_group, topk_group, top_k, rsf, topk_ids,
                                     topk_w, (hipStream_t)stream),
                    "moe_route_noaux launch");
}

int moe_dispatch(const int32_t* topk_ids, int T, int E, int top_k, int max_m, int32_t* masked_m,
                 int32_t* row, int32_t* offsets, void* stream) {
  if (!topk_ids || !masked_m || !row) return fail(MXG_ERR_INVALID_ARG, "moe_dispatch: null pointer");
  if (T < 0 || E < 1 || top_k < 1 || max_m < 1 || E > 65535)
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch: bad sizes");
  if ((long long)T * top_k >= (1LL << 31)) return fail(MXG_ERR_UNSUPPORTED, "moe_dispatch: too many slots");
  return hip_status(mxg::dispatch(topk_ids, T, E, top_k, max_m, masked_m, row, offsets, (hipStream_t)stream),
                    "moe_dispatch launch");
}

int moe_dispatch_contiguous(const int32_t* topk_ids, int T, int E, int top_k, int align, int32_t* group_start,
                            int32_t* count, int32_t* row, void* stream) {
  if (!topk_ids || !group_start || !count || !row)
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch_contiguous: null pointer");
  if (T < 0 || E < 1 || top_k < 1 || E > 65535 || align < 1 || align > 4096)
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch_contiguous: bad sizes");
  if ((long long)T * top_k + (long long)E * align >= (1LL << 31))
    return fail(MXG_ERR_UNSUPPORTED, "moe_dispatch_contiguous: too many rows");
  return hip_status(mxg::dispatch_contiguous(topk_ids, T, E, top_k, align, group_start, count, row,
                                             (hipStream_t)stream),
                    "moe_dispatch_contiguous launch");
}

int moe_quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x, const int32_t* topk_ids,
                              const int32_t* row, int top_k, int E, int max_m, uint8_t* a,
                              uint8_t* a_sf, void* stream) {
  if (!x || !topk_ids || !row || !a || !a_sf)
    return fail(MXG_ERR_INVALID_ARG, "moe_quantize_gather_nvfp4: null pointer");
  if (T < 0 || H < 64 || top_k < 1 || E < 1 || max_m < 1)
    return fail(MXG_ERR_INVALID_ARG, "moe_quantize_gather_nvfp4: bad sizes");
  if (H % 64 != 0) return fail(MXG_ERR_UNSUPPORTED, "moe_quantize_gather_nvfp4: H %% 64 != 0");
  if (!(g_x > 0.0f) || g_x == __builtin_inff())
    return fail(MXG_ERR_INVALID_ARG, "moe_quantize_gather_nvfp4: g_x must be finite and > 0");
  if (!aligned16(x) || !aligned16(a))
    return fail(MXG_ERR_INVALID_ARG, "moe_quantize_gather_nvfp4: misaligned pointer");
  return hip_status(mxg::quantize_gather_nvfp4(x, T, H, g_x, topk_ids, row, top_k, max_m, a, a_sf,
                                               (hipStream_t)stream),
                    "moe_quantize_gather_nvfp4 launch");
}

int moe_interleave_w13(const uint8_t* src, uint8_t* dst, int E, int I, int row_bytes, void* stream) {
  if (!src || !dst) return fail(MXG_ERR_INVALID_ARG, "moe_interleave_w13: null pointer");
  if (E < 0 || I < 0 || row_bytes < 0) return fail(MXG_ERR_INVALID_ARG, "moe_interleave_w13: bad sizes");
  if (I % 16 != 0 || row_bytes % 4 != 0)
    return fail(MXG_ERR_UNSUPPORTED, "moe_interleave_w13: needs I %% 16 == 0 and row_bytes %% 4 == 0");
  if (((uintptr_t)src & 3u) || ((uintptr_t)dst & 3u))
    return fail(MXG_ERR_INVALID_ARG, "moe_interleave_w13: misaligned pointer");
  const size_t n = (size_t)E * 2 * I * row_bytes;
  if ((uintptr_t)src < (uintptr_t)dst + n && (uintptr_t)dst < (uintptr_t)src + n && n > 0)
    return fail(MXG_ERR_INVALID_ARG, "moe_interleave_w13: src and dst overlap");
  return hip_status(mxg::interleave_w13(src, dst, E, I, row_bytes, (hipStream_t)stream), "moe_interleave_w13 launch");
}

int moe_dispatch_quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x, const int32_t* topk_ids,
                                       int top_k, int E, int max_m, int32_t* masked_m, int32_t* row, uint8_t* a,
                                       uint8_t* a_sf, void* stream) {
  if (!x || !topk_ids || !masked_m || !row || !a || !a_sf)
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch_quantize_gather_nvfp4: null pointer");
  if (T < 0 || H < 64 || top_k < 1 || E < 1 || max_m < 1 || E > 65535)
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch_quantize_gather_nvfp4: bad sizes");
  if (H % 64 != 0) return fail(MXG_ERR_UNSUPPORTED, "moe_dispatch_quantize_gather_nvfp4: H %% 64 != 0");
  if ((long long)T * top_k >= (1LL << 31))
    return fail(MXG_ERR_UNSUPPORTED, "moe_dispatch_quantize_gather_nvfp4: too many slots");
  if (!(g_x > 0.0f) || g_x == __builtin_inff())
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch_quantize_gather_nvfp4: g_x must be finite and > 0");
  if (!aligned16(x) || !aligned16(a))
    return fail(MXG_ERR_INVALID_ARG, "moe_dispatch_quantize_gather_nvfp4: misaligned pointer");
  return hip_status(mxg::dispatch_quantize_gather_nvfp4(x, T, H, g_x, topk_ids, top_k, E, max_m, masked_m, row, a,
                                                        a_sf, (hipStream_t)stream),
                    "moe_dispatch_quantize_gather_nvfp4 launch");
}

// ----------------------------------------------------------------------------- MoE layer
static int check_moe(const mxg_moe_desc* d) {
  if (!d) return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: null descriptor");
  if (d->precision != MXG_MOE_FP8_BLOCK128 && d->precision != MXG_MOE_NVFP4 &&
      d->precision != MXG_MOE_FP8_BLOCK128_F32H)
    return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward: unknown precision %d", d->precision);
  const bool fp8 = d->precision != MXG_MOE_NVFP4;
  if (d->T < 0 || d->H < 128 || d->I < 128 || d->E < 1 || d->top_k < 1 || d->max_m < 1)
    return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: bad sizes");
  if (d->H % 128 || d->I % 128)
    return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward: H and I must be multiples of 128");
  if (d->top_k > 8) return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward: top_k > 8");
  if (fp8 && d->E > 1024)
    return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward: FP8 takes at most 1024 experts");
  // the FP8 GEMMs address token rows, an expert's rows and its weights with 32-bit byte offsets
  if (fp8 && ((unsigned long long)d->T * d->H >= (1ull << 32) ||
              (unsigned long long)d->max_m * d->I * 4 >= (1ull << 32) ||
              2ull * d->I * d->H >= (1ull << 32) ||
              4ull * d->E * (d->H / 128) * (d->I / 128) >= (1ull << 32)))
    return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward: FP8 needs T*H, 4*max_m*I, 2*I*H below 2^32");
  if (!d->x || !d->w13 || !d->w13_scale || !d->w2 || !d->w2_scale || !d->topk_ids || !d->topk_w ||
      !d->masked_m || !d->row || !d->y)
    return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: null pointer");
  if (fp8 && !d->x_scale)
    return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: FP8 needs x_scale");
  if (d->w13_layout != MXG_W13_STACKED && d->w13_layout != MXG_W13_INTERLEAVED16)
    return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: unknown w13_layout %d", d->w13_layout);
  if (fp8 && d->w13_layout != MXG_W13_STACKED)
    return fail(MXG_ERR_UNSUPPORTED, "moe_expert_forward: the interleaved W13 layout is NVFP4 only");
  if (d->precision == MXG_MOE_NVFP4) {
    if (!d->g_w13 || !d->g_w2) return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: NVFP4 needs g_w13/g_w2");
    if (!(d->g_x > 0.0f) || !(d->g_h > 0.0f) || d->g_x == __builtin_inff() || d->g_h == __builtin_inff())
      return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: g_x and g_h must be finite and > 0");
  }
  if (!aligned16(d->x) || !aligned16(d->w13) || !aligned16(d->w2) || !aligned16(d->y))
    return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: misaligned pointer");
  return MXG_OK;
}

int moe_expert_forward_workspace_layout(const mxg_moe_desc* d, size_t* off) {
  int st = check_moe(d);
  if (st) return st;
  if (!off) return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward_workspace_layout: null output");
  size_t rows = (size_t)d->E * d->max_m;
  size_t sz[5];
  if (d->precision != MXG_MOE_NVFP4) {
    const size_t planes = d->precision == MXG_MOE_FP8_BLOCK128_F32H ? 2 : 1;
    sz[0] = rows * 4;                        // the token of each expert row (int32)
    sz[1] = (size_t)d->E * (d->H / 128) * mxg::fp8_scale_stride(d->max_m) * 4;  // fp32 1x128 scales
    sz[2] = (rows + 1) * d->I * 2 * planes;  // bf16 h (hi, lo), plus one row that masked rows' stores land in
    sz[3] = 0;
  } else {
    sz[0] = rows * (d->H / 2);
    sz[1] = rows * (d->H / 16);
    sz[2] = rows * (d->I / 2);
    sz[3] = rows * (d->I / 16);
  }
  sz[4] = rows * d->H * 4;                   // fp32 GEMM2 output
  size_t o = 0;
  for (int i = 0; i < 5; i++) {
    off[i] = o;
    o += align256(sz[i]);
  }
  off[5] = o;
  return ok();
}

size_t moe_expert_forward_workspace_size(const mxg_moe_desc* d) {
  size_t off[6];
  if (moe_expert_forward_workspace_layout(d, off) != MXG_OK) return 0;
  return off[5];
}

int moe_expert_forward(const mxg_moe_desc* d, void* ws, size_t ws_bytes, void* stream) {
  size_t off[6];
  int st = moe_expert_forward_workspace_layout(d, off);
  if (st) return st;
  if (!ws || ws_bytes < off[5])
    return fail(MXG_ERR_WORKSPACE, "moe_expert_forward: workspace of %zu bytes needed, %zu given", off[5],
                ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & 255u) != 0) return fail(MXG_ERR_INVALID_ARG, "moe_expert_forward: workspace not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  const int E = d->E, H = d->H, I = d->I, T = d->T, k = d->top_k, mm = d->max_m;
  float* o = (float*)(w + off[4]);
  hipError_t e;
  if (d->precision != MXG_MOE_NVFP4) {
    const int split = d->precision == MXG_MOE_FP8_BLOCK128_F32H;
    int32_t* a_tok = (int32_t*)(w + off[0]);
    float* a_s = (float*)(w + off[1]);
    uint16_t* h = (uint16_t*)(w + off[2]);
    e = mxg::fp8_expert_rows(d->x_scale, T, H, d->topk_ids, d->row, k, E, mm, d->masked_m, a_tok, a_s, s);
    if (e != hipSuccess) return hip_status(e, "fp8_expert_rows");
    mxg::Fp8GemmArgs p1{};
    p1.a = (const uint8_t*)d->x; p1.a_tok = a_tok; p1.tokens = T;
    p1.a_s = a_s; p1.b = d->w13; p1.b_s = (const float*)d->w13_scale; p1.out = h;
    p1.masked_m = d->masked_m; p1.G = E; p1.max_m = mm; p1.N = 2 * I; p1.K = H;
    p1.a_s_stride = mxg::fp8_scale_stride(mm);
    p1.h_split = split;
    p1.dbg_g1 = d->dbg_g1;
    e = mxg::gemm_fp8_swiglu(p1, 0, s);
    if (e != hipSuccess) return hip_status(e, "gemm_fp8_swiglu");
    mxg::Fp8GemmArgs p2{};
    p2.a = (const uint8_t*)h; p2.b = d->w2; p2.b_s = (const float*)d->w2_scale; p2.out = o;
    p2.masked_m = d->masked_m; p2.G = E; p2.max_m = mm; p2.N = H; p2.K = split ? 2 * I : I;
    p2.b_k = I; p2.h_split = split;
    e = mxg::gemm_bf16_fp8w(p2, 0, s);
    if (e != hipSuccess) return hip_status(e, "gemm_bf16_fp8w");
  } else {
    uint8_t* a = w + off[0];
    uint8_t* a_sf = w + off[1];
    uint8_t* hc = w + off[2];
    uint8_t* hsf = w + off[3];
    e = mxg::quantize_gather_nvfp4((const uint16_t*)d->x, T, H, d->g_x, d->topk_ids, d->row, k, mm, a,
                                   a_sf, s);
    if (e != hipSuccess) return hip_status(e, "quantize_gather_nvfp4");
    mxg::MaskedGemmArgs p1{};
    p1.a = a; p1.a_sf = a_sf; p1.b = d->w13; p1.b_sf = (const uint8_t*)d->w13_scale;
    p1.out = nullptr; p1.masked_m = d->masked_m; p1.alpha = d->g_w13; p1.alpha_scale = d->g_x;
    p1.G = E; p1.max_m = mm; p1.N = 2 * I; p1.K = H;
    p1.h_codes = hc; p1.h_sf = hsf; p1.dbg_h = d->dbg_h; p1.dbg_g1 = d->dbg_g1; p1.g_h = d->g_h;
    p1.w13_il16 = d->w13_layout == MXG_W13_INTERLEAVED16;
    // a decode batch leaves most experts with a few rows: 8-row tiles stream less padding
    const int sparse = (long long)T * k <= 4LL * E;
    p1.sparse_rows = sparse;
    e = mxg::gemm_nvfp4_masked(p1, mxg::EPI_SWIGLU_NVFP4, 0, s);
    if (e != hipSuccess) return hip_status(e, "gemm1 nvfp4 swiglu");
    mxg::MaskedGemmArgs p2{};
    p2.a = hc; p2.a_sf = hsf; p2.b = d->w2; p2.b_sf = (const uint8_t*)d->w2_scale; p2.out = o;
    p2.masked_m = d->masked_m; p2.alpha = d->g_w2; p2.alpha_scale = d->g_h;
    p2.G = E; p2.max_m = mm; p2.N = H; p2.K = I;
    p2.sparse_rows = sparse;
    e = mxg::gemm_nvfp4_masked(p2, mxg::EPI_F32, 0, s);
    if (e != hipSuccess) return hip_status(e, "gemm2 nvfp4");
  }
  e = mxg::combine(o, d->topk_ids, d->row, d->topk_w, T, H, k, mm, d->y, s);
  return hip_status(e, "combine");
}

int moe_expert_forward_noalloc(const mxg_moe_desc* d, void* stream) {
  size_t off[6];
  int st = moe_expert_forward_workspace_layout(d, off);
  if (st) return st;
  if (off[5] > MXG_NOALLOC_SCRATCH_BYTES)
    return fail(MXG_ERR_WORKSPACE,
                "moe_expert_forward_noalloc: the layer needs %zu bytes of workspace; the device scratch holds %zu",
                off[5], (size_t)MXG_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st) return st;
  return moe_expert_forward(d, ws, off[5], stream);
}

}  // extern "C"
