// route.hip -- DeepSeek-V3 no-aux routing and the token -> expert permutation.
//
// Routing ("llm-assisted-kernel-dev" README, mixture-of-experts table:
// sigmoid(logits) + bias, grouped top-k, routed_scaling_factor).  One
// wavefront per token; with E = 256 each lane owns 4 consecutive experts, so
// a group of E / n_group experts is a run of 64 / n_group lanes.  Group top-2
// sums are xor-shuffle reductions and each top-k round a DPP row reduction plus
// readlanes; ties resolve to the lower index at every comparison.  All value
// arithmetic is fp32 with
// round to nearest; the sigmoid is evaluated in fp64 and rounded once.
//
// Dispatch (per-expert valid row count masked_m of the masked grouped GEMM,
// "The CuteDSL Gamble", "The Message"): one workgroup per expert scans the
// flattened [T * top_k] id list in order; wavefront ballots and a prefix count
// give each matching slot its stable rank.
#include "device_common.h"
#include "kernels.h"

namespace mxg {

__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

constexpr int NONE = 0x7FFFFFFF;  // no candidate

// Combine this lane's candidate with the one DPP control CTRL brings in from its row
// (a rotation: every source lane is valid).
template <int CTRL>
__device__ __forceinline__ void row_best(float& bv, int& bi, float& bsv) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xF, 0xF, false);
  const float os = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bsv), CTRL, 0xF, 0xF, false));
  if (oi != NONE && (bi == NONE || better(ov, oi, bv, bi))) { bv = ov; bi = oi; bsv = os; }
}

__global__ __launch_bounds__(256) void k_route_noaux(const float* logits, const float* bias, int T,
                                                     int n_group, int topk_group, int top_k, float rsf,
                                                     int32_t* ids, float* wout) {
  constexpr int E = 256;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together

  float s[4], sb[4];
  const float4_t lg = *(const float4_t*)(logits + (size_t)t * E + lane * 4);
  const float4_t bs = *(const float4_t*)(bias + lane * 4);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    s[i] = (float)(1.0 / (1.0 + exp(-(double)lg[i])));
    sb[i] = s[i] + bs[i];
  }
  // group score: sum of the two largest sb in the group (values only)
  float m1 = sb[0], m2 = -INFINITY;
#pragma unroll
  for (int i = 1; i < 4; i++) {
    float v = sb[i];
    if (v > m1) { m2 = m1; m1 = v; } else if (v > m2) { m2 = v; }
  }
  const int glanes = 64 / n_group;
  for (int off = 1; off < glanes; off <<= 1) {
    float o1 = __shfl_xor(m1, off), o2 = __shfl_xor(m2, off);
    float n1 = fmaxf(m1, o1);
    float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
    m1 = n1; m2 = n2;
  }
  const float gscore = m1 + m2;
  const int mygroup = lane / glanes;
  // rank of my group among all groups (score desc, index asc)
  int rank = 0;
  for (int q = 0; q < n_group; q++) {
    float gq = __shfl(gscore, q * glanes);
    if (better(gq, q, gscore, mygroup)) rank++;
  }
  const bool keep = rank < topk_group;

  float den = 0.0f;  // fp32 sum of the selected s in slot order
  uint32_t taken = 0;  // bit i: this lane's expert 4 lane + i already selected (a mask, not an array: no scratch)
  int my_id = -1;
  float my_s = 0.0f;
  for (int j = 0; j < top_k; j++) {
    float bv = -INFINITY;
    int bi = NONE;
    float bsv = 0.0f;
    if (keep) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int e = lane * 4 + i;
        if (!((taken >> i) & 1u) && (bi == NONE || better(sb[i], e, bv, bi))) { bv = sb[i]; bi = e; bsv = s[i]; }
      }
    }
    // the wave's best candidate: rotations inside each 16-lane row (DPP, VALU latency), then
    // the four row winners read into uniform registers; the order is total over the
    // distinct expert indices, so any reduction order picks the same expert
    row_best<0x128>(bv, bi, bsv);  // row_ror:8
    row_best<0x124>(bv, bi, bsv);  // row_ror:4
    row_best<0x122>(bv, bi, bsv);  // row_ror:2
    row_best<0x121>(bv, bi, bsv);  // row_ror:1
    float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    int wi = __builtin_amdgcn_readlane(bi, 0);
    float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bsv), 0));
#pragma unroll
    for (int r = 1; r < 4; r++) {
      const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
      const int oi = __builtin_amdgcn_readlane(bi, 16 * r);
      const float os = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bsv), 16 * r));
      if (oi != NONE && (wi == NONE || better(ov, oi, wv, wi))) { wv = ov; wi = oi; ws = os; }
    }
    bi = wi;
    bsv = ws;
    if ((bi >> 2) == lane) taken |= 1u << (bi & 3);
    if (lane == j) { my_id = bi; my_s = bsv; }
    den = den + bsv;
  }
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    float q = my_s / den;
    wout[(size_t)t * top_k + lane] = q * rsf;
  }
}

hipError_t route_noaux(const float* logits, const float* bias, int T, int E, int n_group,
                       int topk_group, int top_k, float rsf, int32_t* ids, float* w,
                       hipStream_t s) {
  (void)E;
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_route_noaux, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, bias, T,
                     n_group, topk_group, top_k, rsf, ids, w);
  return hipGetLastError();
}

// One workgroup per expert e.  Each pass covers 4096 flattened slots (16 per
// thread, in order); the rank of a matching slot is the number of matches at
// smaller flat index, which equals the number of earlier tokens routed to e
// because a token's ids are distinct.
__global__ __launch_bounds__(256) void k_dispatch(const int32_t* ids, int n, int max_m,
                                                  int32_t* masked_m, int32_t* row) {
  constexpr int PT = 16, PASS = 256 * PT;  // slots per thread and per pass
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int wave_tot[4];
  // the next pass's ids are loaded while the current pass is scanned (the passes would
  // otherwise each wait a full memory latency)
  const bool vec = ((uintptr_t)ids & 15u) == 0;
  auto load = [&](int f, int (&v)[PT]) {
#pragma unroll
    for (int c = 0; c < PT; c += 4) {
      if (vec && f + c + 3 < n) {
        const int4 q = *(const int4*)(ids + f + c);
        v[c] = q.x; v[c + 1] = q.y; v[c + 2] = q.z; v[c + 3] = q.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) v[c + i] = f + c + i < n ? ids[f + c + i] : -1;
      }
    }
  };
  int cur[PT], nxt[PT];
#pragma unroll
  for (int i = 0; i < PT; i++) nxt[i] = -1;
  load(tid * PT, cur);
  int base = 0;
  for (int f0 = 0; f0 < n; f0 += PASS) {
    const int f = f0 + tid * PT;
    if (f0 + PASS < n) load(f + PASS, nxt);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PT; i++) cnt += (f + i < n) && cur[i] == e;
    // inclusive wave scan of cnt
    int inc = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      int v = __shfl_up(inc, off);
      if (lane >= off) inc += v;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < 4; w++) {
      int tw = wave_tot[w];
      if (w < wave) before += tw;
      total += tw;
    }
    int r = base + before + inc - cnt;
#pragma unroll
    for (int i = 0; i < PT; i++)
      if ((f + i < n) && cur[i] == e) row[f + i] = r++;
    base += total;
#pragma unroll
    for (int i = 0; i < PT; i++) cur[i] = nxt[i];
    __syncthreads();
  }
  if (tid == 0) masked_m[e] = base < max_m ? base : max_m;
}

// Contiguous layout: start[e + 1] = start[e] + count[e] rounded up to a multiple of
// align (one wave, shuffle scans over 64 experts at a time), start[0] = 0.
__global__ __launch_bounds__(64) void k_contig_starts(const int32_t* count, int E, int align, int32_t* start) {
  const int lane = threadIdx.x;
  int run = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int c = e < E ? (count[e] + align - 1) / align * align : 0;
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (e < E) start[e + 1] = run + x;
    run += __shfl(x, 63);
  }
  if (lane == 0) start[0] = 0;
}

// row[f] (rank of slot f among its expert's slots) becomes its absolute row.
__global__ __launch_bounds__(256) void k_contig_rows(const int32_t* ids, int n, const int32_t* start, int32_t* row) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f < n) row[f] += start[ids[f]];
}

hipError_t dispatch_contiguous(const int32_t* ids, int T, int E, int top_k, int align, int32_t* start,
                               int32_t* count, int32_t* row, hipStream_t s) {
  const int n = T * top_k;
  hipLaunchKernelGGL(k_dispatch, dim3((unsigned)E), dim3(256), 0, s, ids, n, 0x7FFFFFFF, count, row);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_contig_starts, dim3(1), dim3(64), 0, s, count, E, align, start);
  e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  hipLaunchKernelGGL(k_contig_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, n, start, row);
  return hipGetLastError();
}

hipError_t dispatch(const int32_t* ids, int T, int E, int top_k, int max_m, int32_t* masked_m,
                    int32_t* row, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(k_dispatch, dim3((unsigned)E), dim3(256), 0, s, ids, T * top_k, max_m, masked_m,
                     row);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !offsets) return e;
  // offsets = exclusive scan of masked_m (the scan of the contiguous layout with align 1)
  hipLaunchKernelGGL(k_contig_starts, dim3(1), dim3(64), 0, s, masked_m, E, 1, offsets);
  return hipGetLastError();
}

}  // namespace mxg
