// stream_common.h -- work distribution shared by the persistent weight-streaming GEMMs
// (gemm_fp8.hip, gemm_nvfp4_stream.hip).
//
// A work item is (group g, M tile of at most 256 rows, one N tile).  A group's tiles have
// one height (stream_tile_rows; 256 rows, or balanced for the SwiGLU GEMMs and long K).  Only M tiles
// that hold valid rows exist: their count per group comes from masked_m, and a prefix over
// the groups
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
  int g, m0, mm, n0;  // group, first row of the tile, end of the tile's valid rows, first column
};

// Height of a group's M tiles: STREAM_BM, or (balanced) the fewest tiles of at most
// STREAM_BM rows, all of one height (a multiple of 16), so that a group just above a
// multiple of STREAM_BM rows does not end in a small tile whose weight steps cost as much
// as a full tile's.  Balanced tiles took GEMM1 of the T=8192 NVFP4 layer (K = 7168) from
// 4.20 to 4.04 ms and the contiguous-layout GEMM1 from 3.69 to 3.51 ms, but GEMM2 (K = 2048)
// from 1.93 to 1.96 ms, so the SwiGLU GEMMs and those with K >= 4096 use them.
__device__ __forceinline__ int stream_tile_rows(int mm, bool balanced) {
  const int nt = (mm + STREAM_BM - 1) / STREAM_BM;
  return !balanced || nt <= 1 ? STREAM_BM : ((mm + nt - 1) / nt + 15) & ~15;
}

// tprefix[g] = sum over g' < g of the tile count of group g' (ceil(mm / stream_tile_rows(mm))
// for the clamped masked_m); tprefix[G] = the
// number of units; mm_s[g] = masked_m[g] clamped to [0, max_m], or with `seg` (group row
// starts in LDS, seg[G] = the end) to [0, seg[g + 1] - seg[g]].  Wave 0 builds both with
// shuffle scans.  They live in LDS because a global load inside a main loop would make the
// compiler drain the DMA queue (vmcnt(0)) to wait for it.
__device__ __forceinline__ void stream_tile_prefix(const int32_t* masked_m, int G, int max_m, int* tprefix,
                                                   int* mm_s, int tid, bool balanced, const int* seg = nullptr) {
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
        const int h = stream_tile_rows(mm, balanced);
        c = (mm + h - 1) / h;
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
// N tile w % tiles_n of `ncols` columns; the unit's rows are [m0, mm).  Every value is
// wave-uniform (scalar registers).
__device__ __forceinline__ StreamItem stream_item(int w, int tiles_n, int G, const int* tprefix, const int* mm_s,
                                                  int ncols, bool balanced) {
  StreamItem it;
  const int u = w / tiles_n, nt = w - u * tiles_n;
  int lo = 0, hi = G;  // tprefix[lo] <= u < tprefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(tprefix[mid]) <= u) lo = mid;
    else hi = mid;
  }
  it.g = lo;
  const int mm = __builtin_amdgcn_readfirstlane(mm_s[lo]);
  const int h = stream_tile_rows(mm, balanced);
  it.m0 = (u - __builtin_amdgcn_readfirstlane(tprefix[lo])) * h;
  it.mm = it.m0 + h < mm ? it.m0 + h : mm;
  it.n0 = nt * ncols;
  return it;
}

}  // namespace mxg
