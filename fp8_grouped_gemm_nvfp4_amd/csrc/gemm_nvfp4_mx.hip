// gemm_nvfp4_mx.hip -- heterogeneous grouped NVFP4 NT GEMM on the scaled fp4 MFMA, for
// operands whose e4m3 block scales are all positive powers of two (a property the caller
// declares with sf_dtype = MXG_E4M3_POW2; nothing is inferred from the data).
//
// Operation (Helion "pretuned_kernels" README, grouped_gemm row; "The CuteDSL Gamble",
// "The Message"): C_g = alpha_g * dec(A_g) dec(B_g)^T, dec = e2m1(code) * e4m3(scale of the
// 16-element block), fp32 sums.
//
// Exactness.  A power-of-two e4m3 scale 2^u is exactly the e8m0 scale 127 + u, and the
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4 with e2m1 operands) applies e8m0 scales
// to e2m1 codes without rounding.  The MFMA takes one scale per 32 K-elements of a row,
// NVFP4 one per 16, so each 128-K block runs through two MFMAs: the first with the second
// 16 of every lane's 32 weight elements zeroed and the scales of the first 16-blocks, the
// second the other way round.  The fp4 MFMA runs at twice the fp8 rate, so the pair runs at
// the fp8 rate, twice the fp16 MFMA that the exact decode of general e4m3 scales needs.
// The operands go from LDS to the MFMA as stored: no per-element decode.
//
// Tiles.  An item is (group, M tile of 256 or 128 rows, 256 output columns); a step is
// 128 K: per row 64 code bytes and 8 scale bytes, for 256 activation and 256 weight rows
// (36 KB), streamed by LDS DMA through a ring of four stages (three steps in flight).
// Eight waves as 2 (M) x 4 (N), each 128 (or 64) rows x 64 columns: per step 8 (4)
// activation and 4 weight fragments, 32 (16) MFMA tiles, 64 (32) MFMAs; the two waves of a
// SIMD cover each other's LDS reads.  The MFMA computes D = B A^T, so each lane ends with
// four consecutive output columns of one row; bf16 outputs pair lanes to store 8.  A wave
// whose rows or columns all lie past M or N skips its MFMAs and stores; activation rows
// past M inside a tile re-read row M - 1, and their outputs (equal to row M - 1's bit for
// bit) are stored to row M - 1, so every active wave issues a fixed number of stores per
// item, which the DMA waits count.  Groups of at most 128 rows or of 40 steps and more
// take 128-row tiles, so that no item is longer than a balanced share of the work.
//
// Schedule.  The host orders the groups by decreasing cost per item and deals the items
// longest-first to the least-loaded workgroup; workgroups with the same count of items per
// group form a pattern, and a workgroup takes its items of group g as a contiguous range
// derived from its pattern (at most MX_MAX_PAT patterns, else a round-robin deal).
#include <string.h>

#include <type_traits>
#include <vector>

#include "device_common.h"
#include "kernels.h"

namespace mxg {

namespace mx {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int RG = 8, NB = 4;                              // per wave: 16-row groups (BM rows), 16-column groups
constexpr int A_CODE = BM * 64, A_STAGE = A_CODE + BM * 8;  // codes [256][64], scales [256][8]
constexpr int B_CODE = BN * 64, B_STAGE = B_CODE + BN * 8;  // codes [256][64], scales [256][8]
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int NST = 4;                                     // ring stages; three steps in flight
constexpr int NDMA = 6;                                    // DMA instructions per wave and step
}  // namespace mx

// 16-byte chunk c of code row r sits at slot c ^ mx_swz(r) (conflict-free fragment reads)
__device__ __forceinline__ int mx_swz(int r) { return (r >> 2) & 2; }

// e8m0 exponents of the two e4m3 scale bytes in the low 16 bits of w (positive powers of
// two; subnormal e4m3 powers of two included): the fp32 exponent field of each value.
__device__ __forceinline__ uint32_t mx_e8m0_pair(uint32_t w) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  return ((__float_as_uint(f[0]) >> 23) & 0xFFu) | (((__float_as_uint(f[1]) >> 23) & 0xFFu) << 8);
}

struct MxJob {
  const uint8_t *a, *a_sf, *b, *b_sf;
  void* out;
  int m0, M, n0, N, K, ldc, bm;
  float alpha;
};

// Wait until the DMAs of the current step have landed: at most `later` vector memory
// operations (the DMAs of the two later steps and the stores of the item ends since) may
// still be outstanding.  `later` is 12 plus up to three store counts of 0, 8, 16 or 32,
// capped at the counter's 63; the wait takes the largest listed count not above it
// (waiting for fewer is always safe).
__device__ __forceinline__ void mx_wait(int later) {
  if (later >= 63) wait_vmcnt<63>();
  else if (later >= 60) wait_vmcnt<60>();
  else if (later >= 52) wait_vmcnt<52>();
  else if (later >= 44) wait_vmcnt<44>();
  else if (later >= 36) wait_vmcnt<36>();
  else if (later >= 28) wait_vmcnt<28>();
  else if (later >= 20) wait_vmcnt<20>();
  else wait_vmcnt<12>();
}

template <int EPI>
__global__ __launch_bounds__(mx::THREADS) void k_gemm_nvfp4_mx(const MxGemmArgs p) {
  using namespace mx;
  static_assert(EPI == EPI_BF16 || EPI == EPI_F32, "outputs");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NST * STAGE];
  __shared__ int my_cnt[MXG_MAX_GROUPS], my_base[MXG_MAX_GROUPS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int G = p.G, grid = gridDim.x;
  const int bx = (grid & 7) == 0 ? (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;

  // this workgroup's items: per group a count and the first local item index
  if (tid < MXG_MAX_GROUPS) {
    const int g = tid;
    int cnt = 0, base = 0;
    if (g < G) {
      const HeteroSchedule& sc = p.sched;
      if (sc.npat > 0) {
        int pp = 0;
        while (pp + 1 < sc.npat && sc.pat_start[pp + 1] <= bx) pp++;
        for (int t = 0; t < pp; t++) base += (sc.pat_start[t + 1] - sc.pat_start[t]) * sc.pat_cnt[t][g];
        cnt = bx < sc.pat_start[sc.npat] ? sc.pat_cnt[pp][g] : 0;
        base += (bx - sc.pat_start[pp]) * cnt;
      } else {
        // round robin over the items in group order: item t goes to workgroup t % grid
        const int t0 = p.grp[g].tile_base, n = p.grp[g].tiles_m * p.grp[g].tiles_n;
        const int first = ((bx - t0) % grid + grid) % grid;  // first local index with (t0 + i) % grid == bx
        cnt = first < n ? (n - 1 - first) / grid + 1 : 0;
        base = first;
      }
    }
    my_cnt[g] = cnt;
    my_base[g] = base;
  }
  __syncthreads();
  const int stride = p.sched.npat > 0 ? 1 : grid;  // local index step between a workgroup's items of a group
  int n_items = 0, nsteps = 0;
  for (int g = 0; g < G; g++) {
    const int c = __builtin_amdgcn_readfirstlane(my_cnt[g]);
    n_items += c;
    nsteps += c * (p.grp[g].K / BK);
  }
  if (n_items == 0) return;

  auto job_at = [&](int k) {
    int g = 0;
    for (; g < G; g++) {
      const int c = __builtin_amdgcn_readfirstlane(my_cnt[g]);
      if (k < c) break;
      k -= c;
    }
    if (g == G) g = G - 1, k = 0;  // past the last item (not reached)
    const HeteroGroup& q = p.grp[g];
    const int local = __builtin_amdgcn_readfirstlane(my_base[g]) + k * stride;
    const int mt = local / q.tiles_n;
    MxJob j;
    j.a = q.a; j.a_sf = q.a_sf; j.b = q.b; j.b_sf = q.b_sf; j.out = q.out;
    j.bm = p.bm[g];
    j.m0 = mt * j.bm; j.M = q.M; j.n0 = (local - mt * q.tiles_n) * BN; j.N = q.N; j.K = q.K; j.ldc = q.ldc;
    j.alpha = q.alpha;
    return j;
  };

  // ---- DMA: per step and wave, 2 activation and 2 weight code DMAs (rows 32 w ..) and 1
  // activation and 1 weight scale DMA (rows 32 w ..).  Activation rows past M re-read row
  // M - 1; with 128-row tiles rows 128 .. 255 of the stage re-read rows 0 .. 127; weight
  // rows past N re-read row N - 1.  Per-lane byte offsets from the item's operand bases
  // (uniform, in SGPRs).
  uint32_t aoff[2], aoff_s, boff[2], boff_s;
  const uint8_t *abase = nullptr, *abase_s = nullptr, *bbase = nullptr, *bbase_s = nullptr;
  auto dma_setup = [&](const MxJob& j) {
    const int K = j.K;
    auto arow = [&](int r) {
      const int rt = r < j.bm ? r : r - j.bm;
      return j.m0 + rt < j.M ? j.m0 + rt : j.M - 1;
    };
    auto brow = [&](int r) { return j.n0 + r < j.N ? j.n0 + r : j.N - 1; };
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int r = 32 * wave + 16 * h + (lane >> 2);
      const int sw = (((lane & 3) ^ mx_swz(r)) << 4);
      aoff[h] = (uint32_t)arow(r) * (uint32_t)(K / 2) + sw;
      boff[h] = (uint32_t)brow(r) * (uint32_t)(K / 2) + sw;
    }
    const int r = 32 * wave + (lane >> 1);
    aoff_s = (uint32_t)arow(r) * (uint32_t)(K / 16) + (lane & 1) * 4;
    boff_s = (uint32_t)brow(r) * (uint32_t)(K / 16) + (lane & 1) * 4;
    abase = j.a; abase_s = j.a_sf; bbase = j.b; bbase_s = j.b_sf;
  };
  int d_k = 0, d_kt = 0, d_KT = 0, d_step = 0, d_st = 0;
  // the DMAs of one step in three parts (interleaved with the MFMAs of the current step):
  // activation codes, weight codes, both scale rows; the last part advances the cursor
  auto dma_part = [&](int part) {
    uint8_t* st = ring + d_st * STAGE;
    if (part == 0) {
      const uint8_t* ab = abase + d_kt * (BK / 2);
#pragma unroll
      for (int h = 0; h < 2; h++) dma16_s(ab, aoff[h], st + (32 * wave + 16 * h) * 64);
    } else if (part == 1) {
      const uint8_t* bb = bbase + d_kt * (BK / 2);
#pragma unroll
      for (int h = 0; h < 2; h++) dma16_s(bb, boff[h], st + A_STAGE + (32 * wave + 16 * h) * 64);
    } else {
      dma4_s(abase_s + d_kt * (BK / 16), aoff_s, st + A_CODE + 32 * wave * 8);
      dma4_s(bbase_s + d_kt * (BK / 16), boff_s, st + A_STAGE + B_CODE + 32 * wave * 8);
      d_st = d_st + 1 == NST ? 0 : d_st + 1;
      // past the last step the cursor stays on it: the extra DMAs re-read it into stages
      // that are not read again
      if (d_step + 1 < nsteps) {
        d_step++;
        if (++d_kt == d_KT) {
          d_kt = 0;
          const MxJob j = job_at(++d_k);
          d_KT = j.K / BK;
          dma_setup(j);
        }
      }
    }
  };
  auto dma_issue = [&]() {
    dma_part(0);
    dma_part(1);
    dma_part(2);
  };
  {
    const MxJob j = job_at(0);
    d_KT = j.K / BK;
    dma_setup(j);
  }
#pragma unroll
  for (int i = 0; i < NST - 1; i++) dma_issue();

  // ---- compute state
  const int q = lane >> 4, rr = lane & 15;
  int st_h[3] = {0, 0, 0};  // stores issued at the ends of the last three steps
  int s = 0;                // global step

  // Fragments of a step, read at its start: activation row group i (16 rows), weight
  // column group n (16 columns); codes as stored and the two scale bytes of this lane's
  // 32-element slice.
  u32x4_t fa[RG], fb[NB];
  uint32_t fas[RG], fbs[NB];
  auto load_frags = [&](int rga, int bm, int stage) {
    const uint8_t* As = ring + stage * STAGE;
    const uint8_t* Bs = As + A_STAGE;
#pragma unroll
    for (int n = 0; n < NB; n++) {
      const int r = 64 * wn + 16 * n + rr;
      fb[n] = *(const u32x4_t*)(Bs + r * 64 + ((q ^ mx_swz(r)) << 4));
      fbs[n] = *(const uint32_t*)(Bs + B_CODE + r * 8 + 4 * (q >> 1));
    }
#pragma unroll
    for (int i = 0; i < RG; i++) {
      if (i < rga) {
        const int r = (bm / 2) * wm + 16 * i + rr;
        fa[i] = *(const u32x4_t*)(As + r * 64 + ((q ^ mx_swz(r)) << 4));
        fas[i] = *(const uint32_t*)(As + A_CODE + r * 8 + 4 * (q >> 1));
      }
    }
  };

  // One item over its KT steps with RGA 16-row groups per wave (0: the item has no rows or
  // columns for this wave, which only keeps the DMA pipeline going), then its stores.
  auto run_item = [&](auto rga_c, const MxJob& it) {
    constexpr int RGA = decltype(rga_c)::value;
    const int KT = it.K / BK, bmh = it.bm / 2;
    float4_t acc[RGA > 0 ? RGA : 1][NB];
#pragma unroll
    for (int i = 0; i < RGA; i++)
#pragma unroll
      for (int n = 0; n < NB; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < KT; kt++) {
      // step s's DMAs have landed for every wave, and every wave is past its reads of step
      // s - 1's stage, which the next DMA overwrites
      mx_wait(2 * NDMA + st_h[0] + st_h[1] + st_h[2]);
      __syncthreads();
      st_h[2] = st_h[1];
      st_h[1] = st_h[0];
      st_h[0] = 0;
      if constexpr (RGA > 0) {
        load_frags(RGA, it.bm, s % NST);
        uint32_t sa[RGA], sb[NB];
#pragma unroll
        for (int i = 0; i < RGA; i++) sa[i] = mx_e8m0_pair(fas[i] >> (16 * (q & 1)));
#pragma unroll
        for (int n = 0; n < NB; n++) sb[n] = mx_e8m0_pair(fbs[n] >> (16 * (q & 1)));
        // per pair of 16-row groups: the first 16-blocks of every lane's 32 elements for
        // their tiles, then the second ones (each hi MFMA 2 NB MFMAs after its lo MFMA);
        // a part of the next step's DMAs after each of the first three pairs, so that
        // their issue overlaps the MFMAs already queued
#pragma unroll
        for (int i0 = 0; i0 < RGA; i0 += 2) {
          if (i0 > 0 && i0 / 2 <= 3) {
            __builtin_amdgcn_sched_barrier(0);
            dma_part(i0 / 2 - 1);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = i0; i < i0 + 2; i++) {
            const int8v_t alo = __builtin_shufflevector((int4v_t)fa[i], int4v_t{0, 0, 0, 0}, 0, 1, 4, 5, -1, -1, -1, -1);
#pragma unroll
            for (int n = 0; n < NB; n++) {
              const int8v_t bv = __builtin_shufflevector((int4v_t)fb[n], (int4v_t)fb[n], 0, 1, 2, 3, -1, -1, -1, -1);
              acc[i][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, alo, acc[i][n], 4, 4, 0, sb[n], 0, sa[i]);
            }
          }
#pragma unroll
          for (int i = i0; i < i0 + 2; i++) {
            const int8v_t ahi = __builtin_shufflevector((int4v_t)fa[i], int4v_t{0, 0, 0, 0}, 4, 5, 2, 3, -1, -1, -1, -1);
#pragma unroll
            for (int n = 0; n < NB; n++) {
              const int8v_t bv = __builtin_shufflevector((int4v_t)fb[n], (int4v_t)fb[n], 0, 1, 2, 3, -1, -1, -1, -1);
              acc[i][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, ahi, acc[i][n], 4, 4, 1, sb[n], 1, sa[i]);
            }
          }
        }
        // with fewer than 8 row groups, the DMA parts not issued yet
#pragma unroll
        for (int part = RGA / 2 - 1; part < 3; part++) dma_part(part);
      } else {
        dma_issue();
      }
      s++;
    }
    if constexpr (RGA > 0) {
      // lane (rr, q): row (bm / 2) wm + 16 i + rr of the tile, columns 4 q .. 4 q + 3 of
      // each 16-column group n; rows past M hold row M - 1's values and go there
#pragma unroll
      for (int i = 0; i < RGA; i++) {
        int m = it.m0 + bmh * wm + 16 * i + rr;
        m = m < it.M ? m : it.M - 1;
        if constexpr (EPI == EPI_BF16) {
          // lanes q and q ^ 1 trade halves so that each holds 8 consecutive columns:
          // even q columns 8 (q / 2) .. + 7 of group n, odd q those of group n + 1
          const bool odd = q & 1;
#pragma unroll
          for (int n = 0; n < NB; n += 2) {
            const float4_t v0 = acc[i][n] * it.alpha, v1 = acc[i][n + 1] * it.alpha;
            const uint32_t a0 = bf16x2_rne(v0[0], v0[1]);
            const uint32_t a1 = bf16x2_rne(v0[2], v0[3]);
            const uint32_t b0 = bf16x2_rne(v1[0], v1[1]);
            const uint32_t b1 = bf16x2_rne(v1[2], v1[3]);
            const uint32_t s0 = __shfl_xor(odd ? a0 : b0, 16), s1 = __shfl_xor(odd ? a1 : b1, 16);
            const u32x4_t w = odd ? u32x4_t{s0, s1, b0, b1} : u32x4_t{a0, a1, s0, s1};
            const int c = it.n0 + 64 * wn + 16 * (n + (odd ? 1 : 0)) + 8 * (q >> 1);
            *(u32x4_t*)((uint16_t*)it.out + (size_t)m * it.ldc + c) = w;
          }
        } else {
#pragma unroll
          for (int n = 0; n < NB; n++) {
            const int c = it.n0 + 64 * wn + 16 * n + 4 * q;
            *(float4_t*)((float*)it.out + (size_t)m * it.ldc + c) = acc[i][n] * it.alpha;
          }
        }
      }
      st_h[0] = RGA * (EPI == EPI_BF16 ? NB / 2 : NB);  // stores issued at this step's end
    }
  };

  for (int k = 0; k < n_items; k++) {
    const MxJob it = job_at(k);
    const bool active = it.m0 + (it.bm / 2) * wm < it.M && it.n0 + 64 * wn < it.N;
    if (!active) run_item(std::integral_constant<int, 0>{}, it);
    else if (it.bm == BM) run_item(std::integral_constant<int, RG>{}, it);
    else run_item(std::integral_constant<int, RG / 2>{}, it);
  }
  wait_vmcnt<0>();  // the trailing DMAs land before the workgroup ends
}

// ---------------------------------------------------------------------------- host side
namespace {

// M tile of a group: 128 rows for groups of at most 128 rows (the other half of a 256-row
// tile would idle two of the four SIMDs) and for deep groups (K >= 40 steps), whose
// 256 x 256 items would be longer than a balanced share of the work; 256 otherwise.
int mx_bm(const HeteroGroup& q) { return (q.M <= 128 || q.K / mx::BK >= 40) ? 128 : 256; }

// Cost of one item of group q in the units of the schedule: steps times the share of a
// full 256 x 256 tile the waves compute, plus a per-step share for the barrier, the
// fragment reads and the DMA issue (measured: about 0.6 of a full step's MFMA time).
double mx_item_cost(const HeteroGroup& q) { return (q.K / mx::BK) * (mx_bm(q) / 256.0 + 0.6); }

}  // namespace

// Groups with rows need N % 128 == 0, K % 128 == 0 and 16-byte aligned output rows;
// returns hipErrorNotSupported (nothing launched) otherwise.  The groups are reordered by
// decreasing item cost and the items dealt longest-first (see the file comment).
hipError_t gemm_nvfp4_mx_hetero(HeteroGemmArgs in, int epi, int cu_limit, hipStream_t s) {
  using namespace mx;
  if (epi != EPI_BF16 && epi != EPI_F32) return hipErrorNotSupported;
  const int ldc_mult = epi == EPI_BF16 ? 8 : 4;  // 16-byte row starts
  MxGemmArgs p{};
  int order[MXG_MAX_GROUPS], n = 0;
  for (int g = 0; g < in.G; g++) {
    const HeteroGroup& q = in.grp[g];
    if (q.M == 0) continue;
    if (q.N % 128 != 0 || q.K % BK != 0 || q.K <= 0 || q.ldc % ldc_mult != 0 || ((uintptr_t)q.out & 15u) != 0)
      return hipErrorNotSupported;
    // the DMAs address operand rows by 32-bit byte offsets from the group's bases
    if ((long long)q.M * (q.K / 2) >= (1LL << 32) || (long long)q.N * (q.K / 2) >= (1LL << 32))
      return hipErrorNotSupported;
    order[n++] = g;
  }
  if (n == 0) return hipSuccess;
  // stable selection by decreasing item cost
  for (int i = 0; i < n; i++) {
    int best = i;
    for (int j = i + 1; j < n; j++)
      if (mx_item_cost(in.grp[order[j]]) > mx_item_cost(in.grp[order[best]])) best = j;
    const int t = order[best];
    for (int j = best; j > i; j--) order[j] = order[j - 1];
    order[i] = t;
  }
  long long items = 0;
  for (int i = 0; i < n; i++) {
    HeteroGroup q = in.grp[order[i]];
    p.bm[i] = mx_bm(q);
    q.tiles_m = (q.M + p.bm[i] - 1) / p.bm[i];
    q.tiles_n = (q.N + BN - 1) / BN;
    q.tile_base = (int)items;
    items += (long long)q.tiles_m * q.tiles_n;
    p.grp[i] = q;
  }
  if (items > 0x7FFFFFFFLL) return hipErrorNotSupported;
  p.G = n;
  const void* k = epi == EPI_BF16 ? (const void*)k_gemm_nvfp4_mx<EPI_BF16> : (const void*)k_gemm_nvfp4_mx<EPI_F32>;
  const int grid = resident_grid(k, THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;

  double cost[MXG_MAX_GROUPS];
  for (int g = 0; g < n; g++) cost[g] = mx_item_cost(p.grp[g]);
  hetero_lpt_schedule(p.grp, cost, n, grid, p.sched);
  if (epi == EPI_BF16) hipLaunchKernelGGL((k_gemm_nvfp4_mx<EPI_BF16>), dim3(grid), dim3(THREADS), 0, s, p);
  else hipLaunchKernelGGL((k_gemm_nvfp4_mx<EPI_F32>), dim3(grid), dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

void hetero_lpt_schedule(const HeteroGroup* grp, const double* cost, int G, int W, HeteroSchedule& out) {
  // the schedule depends only on its inputs: computed once per input set and thread
  struct Cache {
    int W = -1, G = -1;
    long long key[MXG_MAX_GROUPS][3];
    HeteroSchedule sched;
  };
  static thread_local Cache cache[2];  // the two callers use different costs
  static thread_local int next = 0;
  for (Cache& c : cache) {
    bool hit = c.W == W && c.G == G;
    for (int g = 0; g < G && hit; g++) {
      long long cb;
      memcpy(&cb, &cost[g], sizeof cb);
      hit = c.key[g][0] == grp[g].tiles_m && c.key[g][1] == grp[g].tiles_n && c.key[g][2] == cb;
    }
    if (hit) {
      out = c.sched;
      return;
    }
  }
  HeteroSchedule s{};
  s.npat = 0;
  long long items = 0;
  for (int g = 0; g < G; g++) items += (long long)grp[g].tiles_m * grp[g].tiles_n;
  bool ok = W > 0 && W <= 4096 && items <= 65536;
  std::vector<double> load(ok ? W : 0, 0.0);
  std::vector<unsigned char> cnt(ok ? (size_t)W * MXG_MAX_GROUPS : 0, 0);
  // a min-heap of (load, workgroup) would do the same; the linear scan is cheap at these
  // sizes and the result is cached
  for (int g = 0; g < G && ok; g++) {
    const long long ng = (long long)grp[g].tiles_m * grp[g].tiles_n;
    for (long long t = 0; t < ng && ok; t++) {
      int best = 0;
      for (int w = 1; w < W; w++)
        if (load[w] < load[best]) best = w;
      load[best] += cost[g];
      unsigned char& k = cnt[(size_t)best * MXG_MAX_GROUPS + g];
      if (k == 255) ok = false;
      else k++;
    }
  }
  if (ok) {
    int npat = 0, members[MX_MAX_PAT] = {};
    for (int w = 0; w < W && ok; w++) {
      const unsigned char* cw = &cnt[(size_t)w * MXG_MAX_GROUPS];
      int pp = 0;
      for (; pp < npat; pp++)
        if (memcmp(s.pat_cnt[pp], cw, MXG_MAX_GROUPS) == 0) break;
      if (pp == npat) {
        if (npat == MX_MAX_PAT) {
          ok = false;
          break;
        }
        memcpy(s.pat_cnt[pp], cw, MXG_MAX_GROUPS);
        npat++;
      }
      members[pp]++;
    }
    if (ok) {
      s.pat_start[0] = 0;
      for (int pp = 0; pp < npat; pp++) s.pat_start[pp + 1] = s.pat_start[pp] + members[pp];
      s.npat = npat;
    }
  }
  if (!ok) s = HeteroSchedule{};
  Cache& c = cache[next];
  next ^= 1;
  c.W = W;
  c.G = G;
  for (int g = 0; g < G; g++) {
    c.key[g][0] = grp[g].tiles_m;
    c.key[g][1] = grp[g].tiles_n;
    memcpy(&c.key[g][2], &cost[g], sizeof(long long));
  }
  c.sched = s;
  out = s;
}

}  // namespace mxg
