// quant.hip -- NVFP4 quantization of activations, the gather of quantized
// token rows into the per-expert masked layout, and the FP8 row gather.
//
// NVFP4 recipe (e2m1 values with per-16 e4m3 block scales and an fp32 global
// scale; "The CuteDSL Gamble", "Input Knowledge Required"), per block, fp32,
// round to nearest at every step: S = e4m3(amax / (6 g)), d = S * g,
// code = e2m1(x * (1 / d)).  One thread owns one 16-element block, so loads of
// consecutive threads are contiguous.
#include "device_common.h"
#include "kernels.h"

namespace mxg {

template <bool BF16>
__device__ __forceinline__ void load_block16(const void* x, size_t elem0, float v[16]) {
  if constexpr (BF16) {
    const u32x4_t* p = (const u32x4_t*)((const uint16_t*)x + elem0);
    u32x4_t w0 = p[0], w1 = p[1];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w0[i] << 16);
      v[2 * i + 1] = __uint_as_float(w0[i] & 0xFFFF0000u);
      v[8 + 2 * i] = __uint_as_float(w1[i] << 16);
      v[8 + 2 * i + 1] = __uint_as_float(w1[i] & 0xFFFF0000u);
    }
  } else {
    const float4_t* p = (const float4_t*)((const float*)x + elem0);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float4_t w = p[i];
      v[4 * i] = w[0]; v[4 * i + 1] = w[1]; v[4 * i + 2] = w[2]; v[4 * i + 3] = w[3];
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_quantize_nvfp4(const void* x, long nblocks, int K, float g,
                                                        uint8_t* codes, uint8_t* sf) {
  long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  float v[16];
  load_block16<BF16>(x, (size_t)b * 16, v);
  uint32_t w[2];
  uint32_t s = quantize_block16(v, g, 6.0f * g, w);
  *(u32x2_t*)(codes + (size_t)b * 8) = u32x2_t{w[0], w[1]};
  sf[b] = (uint8_t)s;
  (void)K;
}

hipError_t quantize_nvfp4(const void* x, int x_dtype, long rows, int K, float g, uint8_t* codes,
                          uint8_t* sf, hipStream_t s) {
  long nblocks = rows * (long)(K / 16);
  if (nblocks == 0) return hipSuccess;
  dim3 grid((unsigned)((nblocks + 255) / 256));
  if (x_dtype == MXG_BF16)
    hipLaunchKernelGGL(k_quantize_nvfp4<true>, grid, dim3(256), 0, s, x, nblocks, K, g, codes, sf);
  else
    hipLaunchKernelGGL(k_quantize_nvfp4<false>, grid, dim3(256), 0, s, x, nblocks, K, g, codes, sf);
  return hipGetLastError();
}

// Quantize token t's block once and write it to each expert row it was
// dispatched to (slots with row >= max_m are dropped).
__global__ __launch_bounds__(256) void k_quantize_gather(const uint16_t* x, int T, int H, float g,
                                                         const int32_t* ids, const int32_t* row,
                                                         int top_k, int max_m, uint8_t* a,
                                                         uint8_t* a_sf) {
  const int nb = H / 16;
  long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= (long)T * nb) return;
  int t = (int)(b / nb), blk = (int)(b % nb);
  float v[16];
  load_block16<true>(x, (size_t)t * H + (size_t)blk * 16, v);
  uint32_t w[2];
  uint32_t s = quantize_block16(v, g, 6.0f * g, w);
  for (int j = 0; j < top_k; j++) {
    int e = ids[(size_t)t * top_k + j];
    int r = row[(size_t)t * top_k + j];
    if (r >= max_m) continue;
    size_t dst = (size_t)e * max_m + r;
    *(u32x2_t*)(a + dst * (H / 2) + (size_t)blk * 8) = u32x2_t{w[0], w[1]};
    a_sf[dst * nb + blk] = (uint8_t)s;
  }
}

// The same with one wave per 64 blocks of a token (H % 1024 == 0) and top_k fixed at
// compile time: the token's experts and rows are wave-uniform and come in through scalar
// loads once per wave, ahead of the row read, instead of as vector loads inside the loop.
template <int K>
__global__ __launch_bounds__(256) void k_quantize_gather_wave(const uint16_t* __restrict__ x, int T, int H,
                                                              float g, const int32_t* __restrict__ ids,
                                                              const int32_t* __restrict__ row, int max_m,
                                                              uint8_t* __restrict__ a, uint8_t* __restrict__ a_sf) {
  const int nb = H / 16, per_t = nb / 64;
  const long wv = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= (long)T * per_t) return;
  const int t = (int)(wv / per_t);
  const int blk = (int)(wv - (long)t * per_t) * 64 + (threadIdx.x & 63);
  int ej[K], rj[K];
#pragma unroll
  for (int j = 0; j < K; j++) {
    ej[j] = ids[(size_t)t * K + j];
    rj[j] = row[(size_t)t * K + j];
  }
  float v[16];
  load_block16<true>(x, (size_t)t * H + (size_t)blk * 16, v);
  uint32_t w[2];
  const uint32_t sc = quantize_block16(v, g, 6.0f * g, w);
#pragma unroll
  for (int j = 0; j < K; j++) {
    if (rj[j] >= max_m) continue;
    const size_t dst = (size_t)ej[j] * max_m + rj[j];
    *(u32x2_t*)(a + dst * (H / 2) + (size_t)blk * 8) = u32x2_t{w[0], w[1]};
    a_sf[dst * nb + blk] = (uint8_t)sc;
  }
}

hipError_t quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x, const int32_t* ids,
                                 const int32_t* row, int top_k, int max_m, uint8_t* a,
                                 uint8_t* a_sf, hipStream_t s) {
  long n = (long)T * (H / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (H % 1024 == 0 && (top_k == 8 || top_k == 6 || top_k == 4 || top_k == 2)) {
    if (top_k == 8)
      hipLaunchKernelGGL(k_quantize_gather_wave<8>, grid, dim3(256), 0, s, x, T, H, g_x, ids, row, max_m, a, a_sf);
    else if (top_k == 6)
      hipLaunchKernelGGL(k_quantize_gather_wave<6>, grid, dim3(256), 0, s, x, T, H, g_x, ids, row, max_m, a, a_sf);
    else if (top_k == 4)
      hipLaunchKernelGGL(k_quantize_gather_wave<4>, grid, dim3(256), 0, s, x, T, H, g_x, ids, row, max_m, a, a_sf);
    else
      hipLaunchKernelGGL(k_quantize_gather_wave<2>, grid, dim3(256), 0, s, x, T, H, g_x, ids, row, max_m, a, a_sf);
  } else {
    hipLaunchKernelGGL(k_quantize_gather, grid, dim3(256), 0, s, x, T, H, g_x, ids, row, top_k, max_m, a, a_sf);
  }
  return hipGetLastError();
}

// Dispatch and quantize-gather in one launch for small batches (T * top_k <= 256): every
// workgroup reads all ids into LDS and gives each slot its row, the number of earlier
// tokens routed to the same expert (a token's ids are distinct), exactly as k_dispatch;
// then it quantizes its (token, 16-block) items as k_quantize_gather.  Workgroup 0 also
// writes row[] and masked_m[] (one thread per expert counts its slots).
constexpr int DQ_MAX_SLOTS = 256;
__global__ __launch_bounds__(256) void k_dispatch_quantize_gather(const uint16_t* x, int T, int H, float g,
                                                                  const int32_t* ids, int top_k, int E,
                                                                  int max_m, int32_t* masked_m, int32_t* row,
                                                                  uint8_t* a, uint8_t* a_sf) {
  __shared__ int id_s[DQ_MAX_SLOTS];
  __shared__ int row_s[DQ_MAX_SLOTS];
  const int n = T * top_k, tid = threadIdx.x;
  if (tid < n) id_s[tid] = ids[tid];
  __syncthreads();
  if (tid < n) {
    const int e = id_s[tid], t = tid / top_k;
    int r = 0;
    for (int f = 0; f < t * top_k; f++) r += id_s[f] == e;
    row_s[tid] = r;
    if (blockIdx.x == 0) row[tid] = r;
  }
  if (blockIdx.x == 0)
    for (int e = tid; e < E; e += 256) {
      int c = 0;
      for (int f = 0; f < n; f++) c += id_s[f] == e;
      masked_m[e] = c < max_m ? c : max_m;
    }
  __syncthreads();
  const int nb = H / 16;
  const long b = (long)blockIdx.x * 256 + tid;
  if (b >= (long)T * nb) return;
  const int t = (int)(b / nb), blk = (int)(b % nb);
  float v[16];
  load_block16<true>(x, (size_t)t * H + (size_t)blk * 16, v);
  uint32_t w[2];
  const uint32_t sc = quantize_block16(v, g, 6.0f * g, w);
  for (int j = 0; j < top_k; j++) {
    const int e = id_s[t * top_k + j], r = row_s[t * top_k + j];
    if (r >= max_m) continue;
    const size_t dst = (size_t)e * max_m + r;
    *(u32x2_t*)(a + dst * (H / 2) + (size_t)blk * 8) = u32x2_t{w[0], w[1]};
    a_sf[dst * nb + blk] = (uint8_t)sc;
  }
}

hipError_t dispatch_quantize_gather_nvfp4(const uint16_t* x, int T, int H, float g_x, const int32_t* ids,
                                          int top_k, int E, int max_m, int32_t* masked_m, int32_t* row,
                                          uint8_t* a, uint8_t* a_sf, hipStream_t s) {
  if ((long)T * top_k > DQ_MAX_SLOTS) {
    const hipError_t e = dispatch(ids, T, E, top_k, max_m, masked_m, row, nullptr, s);
    if (e != hipSuccess) return e;
    return quantize_gather_nvfp4(x, T, H, g_x, ids, row, top_k, max_m, a, a_sf, s);
  }
  const long items = (long)T * (H / 16);
  const long blocks = items > 0 ? (items + 255) / 256 : 1;  // at least one, for masked_m
  hipLaunchKernelGGL(k_dispatch_quantize_gather, dim3((unsigned)blocks), dim3(256), 0, s, x, T, H, g_x, ids, top_k,
                     E, max_m, masked_m, row, a, a_sf);
  return hipGetLastError();
}

// FP8 expert rows.  GEMM1 reads each expert row's activations straight from its
// token's row of x, so the rows are not copied: a_tok[e * max_m + r] is the token of
// expert e's row r (one thread per dispatched slot), and the 1x128 scales are stored
// transposed, one contiguous column of rows per (expert, 128-block), as the GEMM streams
// them (one thread per (expert, block, row), reading the token through a_tok).
__global__ __launch_bounds__(256) void k_fp8_row_tokens(const int32_t* ids, const int32_t* row, int n_slots,
                                                        int top_k, int E, int max_m, int32_t* a_tok) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_slots) return;
  const int e = ids[i], r = row[i];
  if ((unsigned)r < (unsigned)max_m && (unsigned)e < (unsigned)E) a_tok[(size_t)e * max_m + r] = i / top_k;
}

__global__ __launch_bounds__(256) void k_fp8_row_scales(const float* xs, int T, int KB, const int32_t* masked_m,
                                                        int max_m, const int32_t* a_tok, float* a_s) {
  const int e = blockIdx.z, kb = blockIdx.y, r = blockIdx.x * 256 + threadIdx.x;
  int mm = masked_m[e];
  mm = mm < 0 ? 0 : (mm > max_m ? max_m : mm);
  if (r >= mm) return;
  int t = a_tok[(size_t)e * max_m + r];
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);  // any table entry reads a row of xs
  a_s[((size_t)e * KB + kb) * fp8_scale_stride(max_m) + r] = xs[(size_t)t * KB + kb];
}

hipError_t fp8_expert_rows(const float* xs, int T, int H, const int32_t* ids, const int32_t* row, int top_k,
                           int E, int max_m, const int32_t* masked_m, int32_t* a_tok, float* a_s,
                           hipStream_t s) {
  const int n = T * top_k, KB = H / 128;
  if (n == 0 || E == 0 || KB == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fp8_row_tokens, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, row, n, top_k,
                     E, max_m, a_tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fp8_row_scales, dim3((unsigned)((max_m + 255) / 256), (unsigned)KB, (unsigned)E),
                     dim3(256), 0, s, xs, T, KB, masked_m, max_m, a_tok, a_s);
  return hipGetLastError();
}

// Weighted combine: y[t, :] = bf16(sum_j w[t, j] * o[ids[t, j], row[t, j], :]),
// fp32 sum in slot order; each thread owns 4 consecutive columns.  All of a thread's slot
// loads are issued before the sum (top_k <= 8), so it keeps up to eight 16-byte reads of
// o in flight; o is read once, with nontemporal loads.
__global__ __launch_bounds__(256) void k_combine(const float* o, const int32_t* ids, const int32_t* row,
                                                 const float* w, int T, int H, int top_k, int max_m,
                                                 uint16_t* y) {
  constexpr int MAXK = 8;
  const int nq = H / 4;
  long c = (long)blockIdx.x * 256 + threadIdx.x;
  if (c >= (long)T * nq) return;
  int t = (int)(c / nq), q = (int)(c % nq);
  int rj[MAXK];
  float wj[MAXK];
  float4_t v[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; j++) {
    rj[j] = max_m;
    wj[j] = 0.f;
    if (j < top_k) {
      rj[j] = row[(size_t)t * top_k + j];
      wj[j] = w[(size_t)t * top_k + j];
    }
  }
#pragma unroll
  for (int j = 0; j < MAXK; j++) {
    v[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (rj[j] < max_m) {
      const int e = ids[(size_t)t * top_k + j];
      v[j] = __builtin_nontemporal_load((const float4_t*)(o + ((size_t)e * max_m + rj[j]) * H + (size_t)q * 4));
    }
  }
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < MAXK; j++) {
    if (rj[j] >= max_m) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = __builtin_fmaf(wj[j], v[j][i], acc[i]);
  }
  uint32_t lo = bf16x2_rne(acc[0], acc[1]);
  uint32_t hi = bf16x2_rne(acc[2], acc[3]);
  *(u32x2_t*)(y + (size_t)t * H + (size_t)q * 4) = u32x2_t{lo, hi};
}

// The same sum with one wave per 256 columns of a token (H % 256 == 0) and top_k fixed at
// compile time: a token's slot rows, experts and weights are then wave-uniform and come in
// through a few wide scalar loads, once per wave, so the vector memory instructions are the
// eight 16-byte row reads and the store.
template <int K>
__global__ __launch_bounds__(256) void k_combine_wave(const float* __restrict__ o,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ row,
                                                      const float* __restrict__ w, int T, int H,
                                                      int max_m, uint16_t* __restrict__ y) {
  const int per_t = H / 256;
  const long wv = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= (long)T * per_t) return;
  const int t = (int)(wv / per_t);
  const int q = (int)(wv - (long)t * per_t) * 64 + (threadIdx.x & 63);
  int rj[K], ej[K];
  float wj[K];
#pragma unroll
  for (int j = 0; j < K; j++) {
    rj[j] = row[(size_t)t * K + j];
    ej[j] = ids[(size_t)t * K + j];
    wj[j] = w[(size_t)t * K + j];
  }
  float4_t v[K];
#pragma unroll
  for (int j = 0; j < K; j++) {
    v[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (rj[j] < max_m)
      v[j] = __builtin_nontemporal_load((const float4_t*)(o + ((size_t)ej[j] * max_m + rj[j]) * H + (size_t)q * 4));
  }
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K; j++) {
    if (rj[j] >= max_m) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = __builtin_fmaf(wj[j], v[j][i], acc[i]);
  }
  uint32_t lo = bf16x2_rne(acc[0], acc[1]);
  uint32_t hi = bf16x2_rne(acc[2], acc[3]);
  *(u32x2_t*)(y + (size_t)t * H + (size_t)q * 4) = u32x2_t{lo, hi};
}

// Stacked -> interleaved W13 rows, one dword per thread (grid-stride).
__global__ __launch_bounds__(256) void k_interleave_w13(const uint32_t* src, uint32_t* dst, int E, int I,
                                                        int row_dw) {
  const long total = (long)E * 2 * I * row_dw;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long prow = i / row_dw;
    const int c = (int)(i - prow * row_dw);
    const int e = (int)(prow / (2 * I)), r = (int)(prow - (long)e * 2 * I);
    const int j = 16 * (r >> 5) + (r & 15);  // gate / up index of physical row r
    const int lrow = (r & 16) ? I + j : j;
    dst[i] = src[((long)e * 2 * I + lrow) * row_dw + c];
  }
}

hipError_t interleave_w13(const uint8_t* src, uint8_t* dst, int E, int I, int row_bytes, hipStream_t s) {
  const long dw = (long)E * 2 * I * (row_bytes / 4);
  if (dw == 0) return hipSuccess;
  const long blocks = (dw + 255) / 256;
  hipLaunchKernelGGL(k_interleave_w13, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     (const uint32_t*)src, (uint32_t*)dst, E, I, row_bytes / 4);
  return hipGetLastError();
}

hipError_t combine(const float* o, const int32_t* ids, const int32_t* row, const float* w, int T,
                   int H, int top_k, int max_m, uint16_t* y, hipStream_t s) {
  long n = (long)T * (H / 4);
  if (n == 0) return hipSuccess;
  if (top_k < 1 || top_k > 8 || H % 4 != 0) return hipErrorNotSupported;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (H % 256 == 0 && top_k == 8)
    hipLaunchKernelGGL(k_combine_wave<8>, grid, dim3(256), 0, s, o, ids, row, w, T, H, max_m, y);
  else
    hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, o, ids, row, w, T, H, top_k, max_m, y);
  return hipGetLastError();
}

}  // namespace mxg
