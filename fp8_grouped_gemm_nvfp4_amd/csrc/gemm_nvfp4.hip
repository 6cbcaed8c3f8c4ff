// gemm_nvfp4.hip -- grouped NT GEMM over NVFP4 operands on gfx950 MFMA.
//
// Operation (masked batched GEMM with scale factors and alpha at output,
// "The CuteDSL Gamble", "The Message"):
//   C[g, m, n] = alpha_g * sum_k dec(A)[g, m, k] * dec(B)[g, n, k]
// with dec(X) = e2m1(code) * e4m3(scale of the 16-element block).
//
// MI355X design:
//  * NVFP4's per-16 e4m3 scales do not map onto the per-32 e8m0 scales of the
//    scaled f8f6f4 MFMA, and e2m1 * e4m3 needs up to 6 significant bits, which
//    fp8/fp4 cannot hold.  fp16 can: every decoded element is exact in fp16, so
//    the kernel decodes codes * block scale into fp16 and runs the fp16 MFMA
//    (v_mfma_f32_16x16x32_f16, fp32 accumulate).  Products of two fp16 values
//    are exact in fp32, so the only rounding is the fp32 accumulation.
//  * Decode happens once per element per workgroup, on the way from HBM into
//    LDS (global -> registers -> v_cvt_scalef32_pk_f16_fp4 + v_pk_mul_f16 ->
//    LDS), double-buffered, one barrier per 64-wide K step.  The raw bytes are
//    prefetched 3 steps ahead in a register ring.
//  * Tiles: BM x BN output per 256-thread workgroup, waves laid out WAVES_M x
//    WAVES_N, each wave a grid of 16x16 MFMA tiles.  A grid-stride loop over
//    tiles bounds the number of resident workgroups when a CU cap is given.
//  * Rows at or beyond a group's valid row count are neither read nor written.
//  * Epilogues: alpha * acc to bf16 (round to nearest even) or fp32, or the
//    fused SwiGLU + NVFP4 requantization of the MoE GEMM1.
#include "device_common.h"
#include "kernels.h"

namespace mxg {

constexpr int BK = 64;          // K elements per step (4 NVFP4 blocks)
constexpr int XCD_CHUNK = 8;    // consecutive tiles that run on one XCD
constexpr int LDS_PITCH = 72;   // fp16 elements per LDS row (64 + 8 pad)

struct TileJob {
  const uint8_t* a;     // group A codes, row 0
  const uint8_t* a_sf;
  const uint8_t* b;     // group B codes, row 0
  const uint8_t* b_sf;
  void* out;
  int M, N, K, ldc;     // valid rows, columns, depth, output row stride
  float alpha;
  int m0, n0;           // tile origin (for SwiGLU: n0 is the h column origin)
  size_t row0;          // row of the group's first row in the output/h tensors
};

// Resolve linear tile index t into a job; returns false if the tile has no valid rows.
template <int BM, int BN, bool SWIGLU>
__device__ __forceinline__ bool masked_tile(const MaskedGemmArgs& p, int t, TileJob& j) {
  int mt = t % p.tiles_m;
  int rest = t / p.tiles_m;
  int nt = rest % p.tiles_n;
  int g = rest / p.tiles_n;
  int mm = p.masked_m[g];
  mm = mm < 0 ? 0 : (mm > p.max_m ? p.max_m : mm);
  j.m0 = mt * BM;
  if (j.m0 >= mm) return false;
  j.M = mm;
  j.N = p.N;
  j.K = p.K;
  j.row0 = (size_t)g * p.max_m;
  j.ldc = SWIGLU ? p.N / 2 : p.N;
  j.n0 = nt * (SWIGLU ? BN / 2 : BN);
  j.a = p.a + (size_t)g * p.max_m * (p.K / 2);
  j.a_sf = p.a_sf + (size_t)g * p.max_m * (p.K / 16);
  j.b = p.b + (size_t)g * p.N * (p.K / 2);
  j.b_sf = p.b_sf + (size_t)g * p.N * (p.K / 16);
  j.alpha = (p.alpha ? p.alpha[g] : 1.0f) * p.alpha_scale;
  j.out = p.out;
  return true;
}

template <int BM, int BN>
__device__ __forceinline__ bool hetero_tile(const HeteroGemmArgs& p, int t, TileJob& j) {
  int g = 0;
  while (g + 1 < p.G && t >= p.grp[g + 1].tile_base) g++;
  const HeteroGroup& q = p.grp[g];
  int local = t - q.tile_base;
  int mt = local % q.tiles_m;
  int nt = local / q.tiles_m;
  j.m0 = mt * BM;
  j.n0 = nt * BN;
  j.M = q.M; j.N = q.N; j.K = q.K; j.ldc = q.ldc; j.row0 = 0;
  j.a = q.a; j.a_sf = q.a_sf; j.b = q.b; j.b_sf = q.b_sf;
  j.alpha = q.alpha;
  j.out = q.out;
  return j.m0 < q.M;
}

// Per-thread staging registers for one K step: 16 code bytes + 2 scale bytes
// per 16-byte chunk, CH_A chunks of A and CH_B of B.
template <int CH>
struct Stage {
  u32x4_t codes[CH];
  uint32_t sc[CH];
};

// Load chunk c (16 bytes = 32 elements) of a ROWS-row operand tile.  Row r of the tile
// is global row grow[i], already clamped into the operand's valid rows (rows beyond the
// valid range re-read a valid row; their results are never stored), so every load is
// unconditional and the compiler can keep several steps of loads in flight.
template <int ROWS, int CH>
__device__ __forceinline__ void load_tile(Stage<CH>& s, const uint8_t* codes, const uint8_t* sf,
                                          int K, int k0, const int* grow, int tid) {
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int c = tid + i * 256;
    if (ROWS * 2 >= 256 * (i + 1) || c < ROWS * 2) {
      const int h = c & 1;
      const uint8_t* src = codes + (size_t)grow[i] * (K / 2) + (k0 / 2) + h * 16;
      s.codes[i] = *(const u32x4_t*)src;
      s.sc[i] = *(const uint16_t*)(sf + (size_t)grow[i] * (K / 16) + (k0 / 16) + h * 2);
    }
  }
}

template <int ROWS, int CH>
__device__ __forceinline__ void store_tile(const Stage<CH>& s, _Float16* lds, int tid) {
#pragma unroll
  for (int i = 0; i < CH; i++) {
    int c = tid + i * 256;
    if (ROWS * 2 >= 256 * (i + 1) || c < ROWS * 2) {
      int r = c >> 1, h = c & 1;
      half2_t s0 = scale_e4m3_to_h2(s.sc[i] & 0xFFu);
      half2_t s1 = scale_e4m3_to_h2(s.sc[i] >> 8);
      half8_t v0 = decode8_e2m1_f16(s.codes[i][0], s0);
      half8_t v1 = decode8_e2m1_f16(s.codes[i][1], s0);
      half8_t v2 = decode8_e2m1_f16(s.codes[i][2], s1);
      half8_t v3 = decode8_e2m1_f16(s.codes[i][3], s1);
      half8_t* dst = (half8_t*)(lds + r * LDS_PITCH + h * 32);
      dst[0] = v0; dst[1] = v1; dst[2] = v2; dst[3] = v3;
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, int MODE>
__global__ __launch_bounds__(256) void k_gemm_nvfp4(const typename ArgsOf<MODE>::type p) {
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int CH_A = (BM * 2 + 255) / 256;
  constexpr int CH_B = (BN * 2 + 255) / 256;
  constexpr bool SWIGLU = (EPI == EPI_SWIGLU_NVFP4);
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile >= 16x16");

  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * (BM + BN) * LDS_PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int total = p.total_tiles;

  // A grid that covers every tile walks them XCD-aware: workgroup b runs on XCD b % 8,
  // chunks of XCD_CHUNK consecutive tiles (the M tiles of one B panel are adjacent) go
  // to the XCDs in turn, so a chunk shares one L2 and heavy tile ranges spread over all
  // XCDs.  A capped grid strides over the tiles.
  const bool cover = (int)gridDim.x >= total;
  for (int t0 = blockIdx.x; t0 < (cover ? (int)gridDim.x : total); t0 += gridDim.x) {
    int t = t0;
    if (cover) {
      const int xcd = t0 & 7, slot = t0 >> 3;
      t = ((slot / XCD_CHUNK) * 8 + xcd) * XCD_CHUNK + slot % XCD_CHUNK;
    }
    if (t >= total) continue;
    TileJob j;
    bool ok;
    if constexpr (MODE == MODE_MASKED) ok = masked_tile<BM, BN, SWIGLU>(p, t, j);
    else ok = hetero_tile<BM, BN>(p, t, j);
    if (!ok) continue;

    // global rows this thread stages, clamped into the valid rows
    int arow[CH_A], brow[CH_B];
#pragma unroll
    for (int i = 0; i < CH_A; i++) {
      const int r = (tid + i * 256) >> 1;
      arow[i] = (j.m0 + r < j.M) ? j.m0 + r : j.M - 1;
    }
#pragma unroll
    for (int i = 0; i < CH_B; i++) {
      const int r = (tid + i * 256) >> 1;
      int gr;
      if constexpr (SWIGLU) {
        const int half_n = j.N / 2;  // I
        int hc = j.n0 + (r < BN / 2 ? r : r - BN / 2);
        hc = hc < half_n ? hc : half_n - 1;
        gr = w13_row(r < BN / 2 ? hc : half_n + hc, half_n, p.w13_il16 != 0);
      } else {
        gr = (j.n0 + r < j.N) ? j.n0 + r : j.N - 1;
      }
      brow[i] = gr;
    }

    float4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int n = 0; n < TN; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Register ring: slot d holds the raw bytes of step kt+1 for kt = d (mod P), loaded P
    // steps before they are stored to LDS; loads are issued in consumption order, so the
    // compiler's in-order vmcnt waits keep the next P-1 steps in flight.
    constexpr int P = 3;
    const int KT = j.K / BK;
    auto load_step = [&](int kt, Stage<CH_A>& a, Stage<CH_B>& b) {
      kt = kt < KT ? kt : KT - 1;  // prefetches past the end re-read the last step
      load_tile<BM, CH_A>(a, j.a, j.a_sf, j.K, kt * BK, arow, tid);
      load_tile<BN, CH_B>(b, j.b, j.b_sf, j.K, kt * BK, brow, tid);
    };
    Stage<CH_A> sa[P];
    Stage<CH_B> sb[P];
    {
      Stage<CH_A> a0;
      Stage<CH_B> b0;
      load_step(0, a0, b0);
      store_tile<BM, CH_A>(a0, smem, tid);
      store_tile<BN, CH_B>(b0, smem + BM * LDS_PITCH, tid);
    }
#pragma unroll
    for (int d = 0; d < P; d++) {
      load_step(d + 1, sa[d], sb[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    for (int kt0 = 0; kt0 < KT; kt0 += P) {
#pragma unroll
      for (int d = 0; d < P; d++) {
        const int kt = kt0 + d;
        if (kt < KT) {
          const _Float16* As = smem + (kt & 1) * (BM + BN) * LDS_PITCH;
          const _Float16* Bs = As + BM * LDS_PITCH;
#pragma unroll
          for (int ks = 0; ks < BK / 32; ks++) {
            half8_t af[TM], bfr[TN];
            const int koff = ks * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < TM; i++)
              af[i] = *(const half8_t*)(As + (wm * WM + i * 16 + (lane & 15)) * LDS_PITCH + koff);
#pragma unroll
            for (int n = 0; n < TN; n++)
              bfr[n] = *(const half8_t*)(Bs + (wn * WN + n * 16 + (lane & 15)) * LDS_PITCH + koff);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
              for (int n = 0; n < TN; n++)
                acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr[n], acc[i][n], 0, 0, 0);
          }
        }
        // step kt+1 into the other buffer (its last readers finished before the previous
        // barrier); past the end this writes a buffer that is not read again
        _Float16* An = smem + ((kt + 1) & 1) * (BM + BN) * LDS_PITCH;
        store_tile<BM, CH_A>(sa[d], An, tid);
        store_tile<BN, CH_B>(sb[d], An + BM * LDS_PITCH, tid);
        __builtin_amdgcn_sched_barrier(0);
        load_step(kt + 1 + P, sa[d], sb[d]);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
      }
    }

    if constexpr (EPI == EPI_BF16 || EPI == EPI_F32) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int n = 0; n < TN; n++) {
          int col = j.n0 + wn * WN + n * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            int row = j.m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
            if (row < j.M && col < j.N) {
              float v = j.alpha * acc[i][n][r];
              size_t off = (j.row0 + row) * j.ldc + col;
              if constexpr (EPI == EPI_BF16) ((uint16_t*)j.out)[off] = (uint16_t)f32_to_bf16_rne(v);
              else ((float*)j.out)[off] = v;
            }
          }
        }
    } else {
      // Fused SwiGLU + NVFP4 requantization (MoE GEMM1).  Waves with wn == 0
      // hold gate columns, wn == 1 the matching up columns.  Exchange through
      // LDS as fp32, then each thread quantizes whole 16-column blocks.
      constexpr int HN = BN / 2;                // h columns per tile
      constexpr int CP = BN + 4;                // fp32 pitch
      static_assert(BM * CP * 4 <= 2 * (BM + BN) * LDS_PITCH * 2, "LDS reuse");
      float* cs = (float*)smem;
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int n = 0; n < TN; n++) {
          int c = wn * WN + n * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            int rr = wm * WM + i * 16 + (lane >> 4) * 4 + r;
            cs[rr * CP + c] = j.alpha * acc[i][n][r];
          }
        }
      __syncthreads();
      const int I = j.N / 2;
      const float gh = p.g_h, six_gh = 6.0f * gh;
      for (int q = tid; q < BM * (HN / 16); q += 256) {
        int rr = q / (HN / 16), cb = q % (HN / 16);
        int row = j.m0 + rr, hc0 = j.n0 + cb * 16;
        if (row >= j.M || hc0 >= I) continue;
        float h[16];
#pragma unroll
        for (int e = 0; e < 16; e++) {
          float gt = cs[rr * CP + cb * 16 + e];
          float up = cs[rr * CP + HN + cb * 16 + e];
          h[e] = gt / (1.0f + expf(-gt)) * up;
        }
        size_t hrow = j.row0 + row;
        float* dbg = p.dbg_h;
        if (dbg) {
#pragma unroll
          for (int e = 0; e < 16; e++) dbg[hrow * I + hc0 + e] = h[e];
        }
        if (float* g1 = p.dbg_g1) {
#pragma unroll
          for (int e = 0; e < 16; e++) {
            g1[hrow * 2 * I + hc0 + e] = cs[rr * CP + cb * 16 + e];
            g1[hrow * 2 * I + I + hc0 + e] = cs[rr * CP + HN + cb * 16 + e];
          }
        }
        uint32_t w[2];
        uint32_t s = quantize_block16(h, gh, six_gh, w);
        *(u32x2_t*)(p.h_codes + hrow * (I / 2) + hc0 / 2) = u32x2_t{w[0], w[1]};
        p.h_sf[hrow * (I / 16) + hc0 / 16] = (uint8_t)s;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------- launchers
template <int BM, int BN, int WM_, int WN_, int EPI, int MODE>
static hipError_t launch(const typename ArgsOf<MODE>::type& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_nvfp4<BM, BN, WM_, WN_, EPI, MODE>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Without a CU cap every tile gets a workgroup; the grid is a multiple of 8 chunks so that
// the kernel's XCD-aware remapping reaches every tile index.  With a cap the workgroups
// stride over the tiles.
static int grid_for(int total, int cu_limit) {
  if (cu_limit > 0) {
    int cap = cu_limit * 2;
    return total < cap ? total : cap;
  }
  return (total + 8 * XCD_CHUNK - 1) / (8 * XCD_CHUNK) * (8 * XCD_CHUNK);
}

hipError_t gemm_nvfp4_masked(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s) {
  // Decode-shaped groups (small row capacity) stream B into LDS by DMA in the skinny
  // kernel; larger groups use LDS-staged square tiles.
  if (p.max_m <= SKINNY_MAX_M && p.K % 512 == 0) {
    const hipError_t e = gemm_nvfp4_skinny(p, epi, cu_limit, s);
    if (e != hipErrorNotSupported) return e;
  }
  // Larger groups stream the weights through LDS in 256-row M tiles.
  if (p.max_m > SKINNY_MAX_M) {
    const hipError_t e = gemm_nvfp4_stream(p, epi, cu_limit, s);
    if (e != hipErrorNotSupported) return e;
  }

  if (epi == EPI_SWIGLU_NVFP4) {
    if (p.max_m <= 16) {
      p.tiles_m = (p.max_m + 15) / 16; p.tiles_n = (p.N / 2) / 128;
      p.total_tiles = p.G * p.tiles_m * p.tiles_n;
      return launch<16, 256, 1, 4, EPI_SWIGLU_NVFP4, MODE_MASKED>(p, grid_for(p.total_tiles, cu_limit), s);
    }
    p.tiles_m = (p.max_m + 127) / 128; p.tiles_n = (p.N / 2) / 64;
    p.total_tiles = p.G * p.tiles_m * p.tiles_n;
    return launch<128, 128, 2, 2, EPI_SWIGLU_NVFP4, MODE_MASKED>(p, grid_for(p.total_tiles, cu_limit), s);
  }
  if (p.max_m <= 16) {
    p.tiles_m = 1; p.tiles_n = (p.N + 255) / 256;
    p.total_tiles = p.G * p.tiles_m * p.tiles_n;
    int grid = grid_for(p.total_tiles, cu_limit);
    return epi == EPI_BF16 ? launch<16, 256, 1, 4, EPI_BF16, MODE_MASKED>(p, grid, s)
                           : launch<16, 256, 1, 4, EPI_F32, MODE_MASKED>(p, grid, s);
  }
  if (p.max_m <= 64) {
    p.tiles_m = (p.max_m + 63) / 64; p.tiles_n = (p.N + 127) / 128;
    p.total_tiles = p.G * p.tiles_m * p.tiles_n;
    int grid = grid_for(p.total_tiles, cu_limit);
    return epi == EPI_BF16 ? launch<64, 128, 2, 2, EPI_BF16, MODE_MASKED>(p, grid, s)
                           : launch<64, 128, 2, 2, EPI_F32, MODE_MASKED>(p, grid, s);
  }
  p.tiles_m = (p.max_m + 127) / 128; p.tiles_n = (p.N + 127) / 128;
  p.total_tiles = p.G * p.tiles_m * p.tiles_n;
  int grid = grid_for(p.total_tiles, cu_limit);
  return epi == EPI_BF16 ? launch<128, 128, 2, 2, EPI_BF16, MODE_MASKED>(p, grid, s)
                         : launch<128, 128, 2, 2, EPI_F32, MODE_MASKED>(p, grid, s);
}

hipError_t gemm_nvfp4_hetero(HeteroGemmArgs p, int epi, int cu_limit, hipStream_t s) {
  {
    const hipError_t e = gemm_nvfp4_stream_hetero(p, epi, cu_limit, s);
    if (e != hipErrorNotSupported) return e;
  }
  constexpr int BM = 128, BN = 128;
  int base = 0;
  for (int g = 0; g < p.G; g++) {
    HeteroGroup& q = p.grp[g];
    q.tiles_m = (q.M + BM - 1) / BM;
    q.tiles_n = (q.N + BN - 1) / BN;
    q.tile_base = base;
    base += q.tiles_m * q.tiles_n;
  }
  p.total_tiles = base;
  if (base == 0) return hipSuccess;
  int grid = grid_for(base, cu_limit);
  return epi == EPI_BF16 ? launch<BM, BN, 2, 2, EPI_BF16, MODE_HETERO>(p, grid, s)
                         : launch<BM, BN, 2, 2, EPI_F32, MODE_HETERO>(p, grid, s);
}

}  // namespace mxg
