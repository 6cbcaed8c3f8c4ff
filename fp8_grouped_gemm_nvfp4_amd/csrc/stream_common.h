// stream_common.h -- work distribution shared by the persistent weight-streaming GEMMs
// (gemm_fp8.hip, gemm_nvfp4_stream.hip).
//
// A work item is (group g, 256-row M tile, one N tile).  Only M tiles that hold valid
// rows exist: their count per group comes from masked_m, and a prefix over the groups
// (in LDS) turns a linear unit index back into (g, M tile) by binary search.  Items are
// dealt out bx + i * grid, where bx numbers the workgroups XCD by XCD (workgroup b runs
// on XCD b % 8), so the workgroups of one XCD run neighbouring N tiles of one group
// together and share its activation rows in their L2.
#pragma once

#include "device_common.h"

namespace mxg {

constexpr int STREAM_BM = 256;      // rows of one M tile
constexpr int STREAM_MAX_G = 1024;  // groups whose prefix fits in LDS

struct StreamItem {
  int g, m0, mm, n0;  // group, first row of the tile, valid rows of the group, first column
};

// tprefix[g] = sum over g' < g of ceil(clamped masked_m[g'] / STREAM_BM); tprefix[G] = the
// number of units; mm_s[g] = masked_m[g] clamped to [0, max_m], or with `seg` (group row
// starts in LDS, seg[G] = the end) to [0, seg[g + 1] - seg[g]].  Wave 0 builds both with
// shuffle scans.  They live in LDS because a global load inside a main loop would make the
// compiler drain the DMA queue (vmcnt(0)) to wait for it.
__device__ __forceinline__ void stream_tile_prefix(const int32_t* masked_m, int G, int max_m, int* tprefix,
                                                   int* mm_s, int tid, const int* seg = nullptr) {
  if (tid < 64) {
    const int lane = tid;
    int run = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      int c = 0;
      if (g < G) {
        int mm = masked_m[g];
        const int lim = seg ? seg[g + 1] - seg[g] : max_m;
        mm = mm < 0 ? 0 : (mm > lim ? lim : mm);
        c = (mm + STREAM_BM - 1) / STREAM_BM;
        mm_s[g] = mm;
      }
      int x = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      if (g < G) tprefix[g] = run + x - c;
      run += __shfl(x, 63);
    }
    if (lane == 0) tprefix[G] = run;
  }
  __syncthreads();
}

__device__ __forceinline__ int stream_bx() {
  const int grid = gridDim.x;
  return (grid & 7) == 0 ? (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
}

// Item w: unit u = w / tiles_n (largest g with tprefix[g] <= u; that group has tiles),
// N tile w % tiles_n of `ncols` columns.  Every value is wave-uniform (scalar registers).
__device__ __forceinline__ StreamItem stream_item(int w, int tiles_n, int G, const int* tprefix, const int* mm_s,
                                                  int ncols) {
  StreamItem it;
  const int u = w / tiles_n, nt = w - u * tiles_n;
  int lo = 0, hi = G;  // tprefix[lo] <= u < tprefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(tprefix[mid]) <= u) lo = mid;
    else hi = mid;
  }
  it.g = lo;
  it.m0 = (u - __builtin_amdgcn_readfirstlane(tprefix[lo])) * STREAM_BM;
  it.mm = __builtin_amdgcn_readfirstlane(mm_s[lo]);
  it.n0 = nt * ncols;
  return it;
}

}  // namespace mxg
