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
// Tiles.  An item is (group, 256-row M tile, 128 output columns); a step is 128 K: per
// row 64 code bytes and 8 scale bytes, for 256 activation and 128 weight rows (27 KB),
// streamed by LDS DMA through a ring of five stages (three steps in flight).  Eight waves
// as 2 (M) x 4 (N), each 128 rows x 32 columns: per step 8 activation and 2 weight
// fragments, 16 MFMA tiles, 32 MFMAs.  The fragments of step s + 1 are read from LDS while
// the MFMAs of step s run.  The MFMA computes D = B A^T, so each lane ends with four
// consecutive output columns of one row.  A wave whose 128 rows all lie past M skips its
// MFMAs and stores; activation rows past M inside a tile re-read row M - 1, and their
// outputs (equal to row M - 1's bit for bit) are stored to row M - 1, so every active wave
// issues the same number of stores per item.
//
// Schedule.  The host orders the groups by decreasing cost per item and deals the items
// longest-first to the least-loaded workgroup; workgroups with the same count of items per
// group form a pattern, and a workgroup takes its items of group g as a contiguous range
// derived from its pattern (at most MX_MAX_PAT patterns, else a round-robin deal).
#include <string.h>

#include <vector>

#include "device_common.h"
#include "kernels.h"

namespace mxg {

namespace mx {
constexpr int BM = 256, BN = 128, BK = 128;
constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int RG = 8, NB = 2;                              // per wave: 16-row groups, 16-column groups
constexpr int A_CODE = BM * 64, A_STAGE = A_CODE + BM * 8;  // codes [256][64], scales [256][8]
constexpr int B_CODE = BN * 64, B_STAGE = B_CODE + BN * 8;  // codes [128][64], scales [128][8]
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int NST = 5;                                     // ring stages; steps in flight NST - 2
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
  int m0, M, n0, K, ldc;
  float alpha;
};

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
      if (p.npat > 0) {
        int pp = 0;
        while (pp + 1 < p.npat && p.pat_start[pp + 1] <= bx) pp++;
        for (int q = 0; q < pp; q++) base += (p.pat_start[q + 1] - p.pat_start[q]) * p.pat_cnt[q][g];
        cnt = p.pat_cnt[pp][g];
        base += (bx - p.pat_start[pp]) * cnt;
        if (bx >= p.pat_start[p.npat]) cnt = 0;
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
  const int stride = p.npat > 0 ? 1 : grid;  // local index step between a workgroup's items of a group
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
    if (g == G) g = G - 1, k = 0;  // past the last item: the last group's first (never computed)
    const HeteroGroup& q = p.grp[g];
    const int local = __builtin_amdgcn_readfirstlane(my_base[g]) + k * stride;
    const int mt = local / q.tiles_n;
    MxJob j;
    j.a = q.a; j.a_sf = q.a_sf; j.b = q.b; j.b_sf = q.b_sf; j.out = q.out;
    j.m0 = mt * BM; j.M = q.M; j.n0 = (local - mt * q.tiles_n) * BN; j.K = q.K; j.ldc = q.ldc;
    j.alpha = q.alpha;
    return j;
  };

  // ---- DMA: per step and wave, 2 activation code DMAs (rows 32 w ..), 1 weight code DMA
  // (rows 16 w ..), 1 activation scale DMA (rows 32 w ..) and, for waves 0-3, 1 weight
  // scale DMA (rows 32 w ..).  Rows past M re-read row M - 1.
  const int n_dma = wave < 4 ? 5 : 4;
  const uint8_t* asrc[2];
  const uint8_t* asrc_s;
  const uint8_t* bsrc;
  const uint8_t* bsrc_s;
  auto dma_setup = [&](const MxJob& j) {
    const int K = j.K;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int r = 32 * wave + 16 * h + (lane >> 2);
      const int row = j.m0 + r < j.M ? j.m0 + r : j.M - 1;
      asrc[h] = j.a + (size_t)row * (K / 2) + (((lane & 3) ^ mx_swz(r)) << 4);
    }
    {
      const int r = 32 * wave + (lane >> 1);
      const int row = j.m0 + r < j.M ? j.m0 + r : j.M - 1;
      asrc_s = j.a_sf + (size_t)row * (K / 16) + (lane & 1) * 4;
    }
    {
      const int r = 16 * wave + (lane >> 2);
      bsrc = j.b + (size_t)(j.n0 + r) * (K / 2) + (((lane & 3) ^ mx_swz(r)) << 4);
    }
    {
      const int r = 32 * (wave & 3) + (lane >> 1);
      bsrc_s = j.b_sf + (size_t)(j.n0 + r) * (K / 16) + (lane & 1) * 4;
    }
  };
  int d_k = 0, d_kt = 0, d_KT = 0, d_step = 0, d_st = 0;
  auto dma_issue = [&]() {
    uint8_t* st = ring + d_st * STAGE;
    const int ko = d_kt;
#pragma unroll
    for (int h = 0; h < 2; h++) dma16(asrc[h] + ko * (BK / 2), st + (32 * wave + 16 * h) * 64);
    dma4(asrc_s + ko * (BK / 16), st + A_CODE + 32 * wave * 8);
    dma16(bsrc + ko * (BK / 2), st + A_STAGE + 16 * wave * 64);
    if (wave < 4) dma4(bsrc_s + ko * (BK / 16), st + A_STAGE + B_CODE + 32 * wave * 8);
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
  float4_t acc[RG][NB];
#pragma unroll
  for (int i = 0; i < RG; i++)
#pragma unroll
    for (int n = 0; n < NB; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
  struct Frag {
    u32x4_t a[RG];
    u32x4_t b[NB];
    u32x2_t as[RG];
    u32x2_t bs[NB];
  };
  Frag F[2];
  auto load_frags = [&](Frag& f, int stage) {
    const uint8_t* As = ring + stage * STAGE;
    const uint8_t* Bs = As + A_STAGE;
#pragma unroll
    for (int i = 0; i < RG; i++) {
      const int r = 128 * wm + 16 * i + rr;
      f.a[i] = *(const u32x4_t*)(As + r * 64 + ((q ^ mx_swz(r)) << 4));
      f.as[i] = *(const u32x2_t*)(As + A_CODE + r * 8);
    }
#pragma unroll
    for (int n = 0; n < NB; n++) {
      const int r = 32 * wn + 16 * n + rr;
      f.b[n] = *(const u32x4_t*)(Bs + r * 64 + ((q ^ mx_swz(r)) << 4));
      f.bs[n] = *(const u32x2_t*)(Bs + B_CODE + r * 8);
    }
  };

  // stores issued at the last three item ends (0 or RG * NB each), for the DMA waits
  int st_hist = 0;  // bit k: an item ended k + 1 iterations ago
  auto wait_next = [&]() {
    // the DMAs of step s + 1 have landed once at most the later ones are outstanding:
    // two steps of DMAs and the stores of the item ends since then
    const int ends = __builtin_popcount(st_hist & 7);
    if (n_dma == 5) {
      switch (ends) {
        case 0: wait_vmcnt<10>(); break;
        case 1: wait_vmcnt<10 + RG * NB>(); break;
        case 2: wait_vmcnt<10 + 2 * RG * NB>(); break;
        default: wait_vmcnt<10 + 3 * RG * NB>(); break;
      }
    } else {
      switch (ends) {
        case 0: wait_vmcnt<8>(); break;
        case 1: wait_vmcnt<8 + RG * NB>(); break;
        case 2: wait_vmcnt<8 + 2 * RG * NB>(); break;
        default: wait_vmcnt<8 + 3 * RG * NB>(); break;
      }
    }
  };

  // step 0's DMAs: the three later steps may be outstanding
  if (n_dma == 5) wait_vmcnt<15>();
  else wait_vmcnt<12>();
  __syncthreads();
  load_frags(F[0], 0);

  MxJob cit = job_at(0);
  int c_k = 0, c_kt = 0;
  const int zero = 0;

  auto step = [&](int s, Frag& cur, Frag& nxt) {
    wait_next();
    // every wave's DMAs of step s + 1 have landed and every wave is past its reads of
    // step s - 1's stage, which the next DMA overwrites
    __syncthreads();
    dma_issue();
    load_frags(nxt, (s + 1) % NST);
    st_hist <<= 1;

    const bool active = cit.m0 + 128 * wm < cit.M;
    if (active) {
      uint32_t sa[RG], sb[NB];
#pragma unroll
      for (int i = 0; i < RG; i++) sa[i] = mx_e8m0_pair(cur.as[i][q >> 1] >> (16 * (q & 1)));
#pragma unroll
      for (int n = 0; n < NB; n++) sb[n] = mx_e8m0_pair(cur.bs[n][q >> 1] >> (16 * (q & 1)));
      // first 16-blocks of every lane's 32 elements, then the second ones
#pragma unroll
      for (int n = 0; n < NB; n++) {
        const int8v_t blo = {(int)cur.b[n][0], (int)cur.b[n][1], zero, zero, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < RG; i++) {
          const int8v_t av = {(int)cur.a[i][0], (int)cur.a[i][1], (int)cur.a[i][2], (int)cur.a[i][3], 0, 0, 0, 0};
          acc[i][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(blo, av, acc[i][n], 4, 4, 0, sb[n], 0, sa[i]);
        }
      }
#pragma unroll
      for (int n = 0; n < NB; n++) {
        const int8v_t bhi = {zero, zero, (int)cur.b[n][2], (int)cur.b[n][3], 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < RG; i++) {
          const int8v_t av = {(int)cur.a[i][0], (int)cur.a[i][1], (int)cur.a[i][2], (int)cur.a[i][3], 0, 0, 0, 0};
          acc[i][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bhi, av, acc[i][n], 4, 4, 1, sb[n], 1, sa[i]);
        }
      }
    }

    if (++c_kt == cit.K / BK) {
      if (active) {
        // lane (rr, q): row 128 wm + 16 i + rr of the tile, columns 4 q .. 4 q + 3 of the
        // wave's 16-column group n; rows past M hold row M - 1's values and go there
#pragma unroll
        for (int i = 0; i < RG; i++) {
          int m = cit.m0 + 128 * wm + 16 * i + rr;
          m = m < cit.M ? m : cit.M - 1;
#pragma unroll
          for (int n = 0; n < NB; n++) {
            const int c = cit.n0 + 32 * wn + 16 * n + 4 * q;
            const float4_t v = acc[i][n] * cit.alpha;
            if constexpr (EPI == EPI_BF16) {
              const uint32_t lo = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
              const uint32_t hi = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
              *(u32x2_t*)((uint16_t*)cit.out + (size_t)m * cit.ldc + c) = u32x2_t{lo, hi};
            } else {
              *(float4_t*)((float*)cit.out + (size_t)m * cit.ldc + c) = v;
            }
          }
        }
        st_hist |= 1;
      }
#pragma unroll
      for (int i = 0; i < RG; i++)
#pragma unroll
        for (int n = 0; n < NB; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
      c_kt = 0;
      if (++c_k < n_items) cit = job_at(c_k);
    }
  };

  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, F[0], F[1]);
    step(s + 1, F[1], F[0]);
  }
  if (s < nsteps) step(s, F[0], F[1]);
  wait_vmcnt<0>();  // the trailing DMAs land before the workgroup ends
}

// ---------------------------------------------------------------------------- host side
namespace {

// Cost of one item of group q in the units of the schedule: steps times the waves per
// SIMD that compute (one when the tile's rows fit the first 128, else two), plus a fixed
// per-step share for the DMA issue and the barrier.
double mx_item_cost(const HeteroGroup& q) {
  const int rows = q.M < mx::BM ? q.M : mx::BM;  // the fullest tile of the group
  return (q.K / mx::BK) * ((rows > 128 ? 2.0 : 1.0) + 0.5);
}

// Longest-first deal of the items (groups in schedule order, every item of a group at the
// group's cost) to the least-loaded of W workgroups, ties to the lower index; the count
// vectors are folded into patterns.  npat = 0 when they do not fit the pattern table.
void mx_schedule(MxGemmArgs& p, int W) {
  p.npat = 0;
  if (W > 4096) return;
  std::vector<double> load(W, 0.0);
  std::vector<unsigned char> cnt((size_t)W * MXG_MAX_GROUPS, 0);
  // a min-heap of (load, workgroup) would do the same; the linear scan is cheap at these
  // sizes and the result is cached per shape
  for (int g = 0; g < p.G; g++) {
    const double c = mx_item_cost(p.grp[g]);
    const long long ng = (long long)p.grp[g].tiles_m * p.grp[g].tiles_n;
    for (long long t = 0; t < ng; t++) {
      int best = 0;
      for (int w = 1; w < W; w++)
        if (load[w] < load[best]) best = w;
      load[best] += c;
      unsigned char& k = cnt[(size_t)best * MXG_MAX_GROUPS + g];
      if (k == 255) return;
      k++;
    }
  }
  int npat = 0, members[MX_MAX_PAT] = {};
  for (int w = 0; w < W; w++) {
    const unsigned char* cw = &cnt[(size_t)w * MXG_MAX_GROUPS];
    int pp = 0;
    for (; pp < npat; pp++)
      if (memcmp(p.pat_cnt[pp], cw, MXG_MAX_GROUPS) == 0) break;
    if (pp == npat) {
      if (npat == MX_MAX_PAT) return;
      memcpy(p.pat_cnt[pp], cw, MXG_MAX_GROUPS);
      npat++;
    }
    members[pp]++;
  }
  p.pat_start[0] = 0;
  for (int pp = 0; pp < npat; pp++) p.pat_start[pp + 1] = p.pat_start[pp] + members[pp];
  p.npat = npat;
}

struct MxSchedCache {
  int W = -1, G = 0;
  int shape[MXG_MAX_GROUPS][3];
  int npat = 0;
  int pat_start[MX_MAX_PAT + 1];
  unsigned char pat_cnt[MX_MAX_PAT][MXG_MAX_GROUPS];
};

}  // namespace

// Groups with rows need N % 128 == 0, K % 128 == 0 and aligned output rows; returns
// hipErrorNotSupported (nothing launched) otherwise.  The groups are reordered by
// decreasing item cost and the items dealt longest-first (see the file comment).
hipError_t gemm_nvfp4_mx_hetero(HeteroGemmArgs in, int epi, int cu_limit, hipStream_t s) {
  using namespace mx;
  if (epi != EPI_BF16 && epi != EPI_F32) return hipErrorNotSupported;
  const uintptr_t out_align = epi == EPI_BF16 ? 8 : 16;
  MxGemmArgs p{};
  int order[MXG_MAX_GROUPS], n = 0;
  for (int g = 0; g < in.G; g++) {
    const HeteroGroup& q = in.grp[g];
    if (q.M == 0) continue;
    if (q.N % BN != 0 || q.K % BK != 0 || q.K <= 0 || q.ldc % 4 != 0 ||
        ((uintptr_t)q.out & (out_align - 1)) != 0)
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
    q.tiles_m = (q.M + BM - 1) / BM;
    q.tiles_n = q.N / BN;
    q.tile_base = (int)items;
    items += (long long)q.tiles_m * q.tiles_n;
    p.grp[i] = q;
  }
  if (items > 0x7FFFFFFFLL) return hipErrorNotSupported;
  p.G = n;
  const void* k = epi == EPI_BF16 ? (const void*)k_gemm_nvfp4_mx<EPI_BF16> : (const void*)k_gemm_nvfp4_mx<EPI_F32>;
  const int grid = resident_grid(k, THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;

  // the schedule depends only on the shapes and the grid: computed once per shape set
  static thread_local MxSchedCache cache;
  bool hit = cache.W == grid && cache.G == n;
  for (int g = 0; g < n && hit; g++)
    hit = cache.shape[g][0] == p.grp[g].M && cache.shape[g][1] == p.grp[g].N && cache.shape[g][2] == p.grp[g].K;
  if (!hit) {
    if (items <= 65536) mx_schedule(p, grid);
    cache.W = grid;
    cache.G = n;
    for (int g = 0; g < n; g++) {
      cache.shape[g][0] = p.grp[g].M;
      cache.shape[g][1] = p.grp[g].N;
      cache.shape[g][2] = p.grp[g].K;
    }
    cache.npat = p.npat;
    memcpy(cache.pat_start, p.pat_start, sizeof(p.pat_start));
    memcpy(cache.pat_cnt, p.pat_cnt, sizeof(p.pat_cnt));
  } else {
    p.npat = cache.npat;
    memcpy(p.pat_start, cache.pat_start, sizeof(p.pat_start));
    memcpy(p.pat_cnt, cache.pat_cnt, sizeof(p.pat_cnt));
  }
  if (epi == EPI_BF16) hipLaunchKernelGGL((k_gemm_nvfp4_mx<EPI_BF16>), dim3(grid), dim3(THREADS), 0, s, p);
  else hipLaunchKernelGGL((k_gemm_nvfp4_mx<EPI_F32>), dim3(grid), dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace mxg
