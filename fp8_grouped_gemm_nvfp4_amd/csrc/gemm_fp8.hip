// gemm_fp8.hip -- the FP8 block-scaled GEMMs of the DeepSeek-V3-style expert
// path ("llm-assisted-kernel-dev" README, mixture-of-experts table: e4m3fn
// hidden states and weights with block scales; GEMM1 -> SwiGLU -> GEMM2 with a
// BF16 intermediate).
//
// GEMM1 + SwiGLU:  A = gathered e4m3 activations [G, max_m, H] with one fp32
//   scale per 1x128, B = W13 e4m3 [G, 2I, H] with fp32 scales per 128x128.
//   Each 128-wide K step is one scale block: the scaled f8f6f4 MFMA
//   (16x16x128, e8m0 scales fixed at 1.0) sums the 128 exact fp8 products into
//   a fresh fp32 tile, which is then promoted into the accumulator with the
//   row's activation scale times the block's weight scale.  Epilogue:
//   h = silu(gate) * up in fp32, stored as bf16 (round to nearest even).
// GEMM2:  A = h bf16 [G, max_m, I], B = W2 e4m3 [G, H, I] with 128x128 fp32
//   scales; fp8 is widened exactly to bf16 on the way into LDS and the bf16
//   MFMA (16x16x32) accumulates each 128-K scale block before promotion.
//   Output fp32 [G, max_m, H].
#include "device_common.h"
#include "kernels.h"

namespace mxg {

// XCD-aware tile order for a grid that covers every tile (workgroup b runs on XCD b % 8):
// chunks of 8 consecutive tiles (the M tiles of one weight panel are adjacent) go to the
// XCDs in turn.  A capped grid strides over the tiles in order.
constexpr int FP8_XCD_CHUNK = 8;
__device__ __forceinline__ int fp8_tile_of(int t0, bool cover) {
  if (!cover) return t0;
  const int xcd = t0 & 7, slot = t0 >> 3;
  return ((slot / FP8_XCD_CHUNK) * 8 + xcd) * FP8_XCD_CHUNK + slot % FP8_XCD_CHUNK;
}
static int fp8_grid(int total, int cu_limit) {
  if (cu_limit > 0) return total < cu_limit * 2 ? total : cu_limit * 2;
  return (total + 8 * FP8_XCD_CHUNK - 1) / (8 * FP8_XCD_CHUNK) * (8 * FP8_XCD_CHUNK);
}
constexpr int FP8_P = 3;   // K steps of raw bytes prefetched in a register ring (GEMM1)
constexpr int FP8_P2 = 2;  // the same for GEMM2, whose two accumulator sets leave fewer registers

// ----------------------------------------------------------------------------- GEMM1
namespace g1 {
constexpr int BM = 128, BN = 128, BK = 128, PITCH = 144;  // bytes per LDS row
constexpr int HN = BN / 2;                                 // h columns per tile
}

__global__ __launch_bounds__(256) void k_gemm_fp8_swiglu(const Fp8GemmArgs p) {
  using namespace g1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * PITCH + 2 * BM * 4 + 2 * 4 * 4];
  float* sa_lds = (float*)(smem + 2 * (BM + BN) * PITCH);  // [2][BM] activation scales
  float* sw_lds = sa_lds + 2 * BM;                          // [2][4] weight scale per wave

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int I = p.N / 2, K = p.K, KB = K / 128;

  const bool cover = (int)gridDim.x >= p.total_tiles;
  for (int t0 = blockIdx.x; t0 < (cover ? (int)gridDim.x : p.total_tiles); t0 += gridDim.x) {
    const int t = fp8_tile_of(t0, cover);
    if (t >= p.total_tiles) continue;
    int mt = t % p.tiles_m, rest = t / p.tiles_m;
    int nt = rest % p.tiles_n, g = rest / p.tiles_n;
    int mm = p.masked_m[g];
    mm = mm < 0 ? 0 : (mm > p.max_m ? p.max_m : mm);
    int m0 = mt * BM;
    if (m0 >= mm) continue;
    int n0 = nt * HN;  // h column origin
    const uint8_t* A = p.a + (size_t)g * p.max_m * K;
    const float* As_g = p.a_s + (size_t)g * p.max_m * KB;
    const uint8_t* B = p.b + (size_t)g * p.N * K;
    const float* Bs_g = p.b_s + (size_t)g * (p.N / 128) * KB;

    // each thread stages 4 chunks of A and 4 of B (16 B each): chunk c -> row c/8, col
    // (c%8)*16; rows are clamped into the valid ones (clamped rows are never stored), so
    // every load is unconditional
    int arow[4], brow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int c = tid + i * 256, r = c >> 3;
      arow[i] = (m0 + r < mm) ? m0 + r : mm - 1;
      int hc = n0 + (r < HN ? r : r - HN);
      hc = hc < I ? hc : I - 1;
      brow[i] = r < HN ? hc : I + hc;
    }
    const int srow = (m0 + (tid & (BM - 1)) < mm) ? m0 + (tid & (BM - 1)) : mm - 1;
    // weight scale row-blocks of this wave's columns (gate for wn = 0, up for wn = 1)
    const int bblk = (wn == 0 ? n0 : I + n0) / 128;

    struct Slot {
      u32x4_t a[4], b[4];
      float sa, sw;  // activation scale of row srow, weight scale of this wave's block
    };
    auto gload = [&](int kb, Slot& sl) {
      kb = kb < KB ? kb : KB - 1;  // prefetches past the end re-read the last block
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int c = tid + i * 256, col = (c & 7) * 16;
        sl.a[i] = *(const u32x4_t*)(A + (size_t)arow[i] * K + kb * 128 + col);
        sl.b[i] = *(const u32x4_t*)(B + (size_t)brow[i] * K + kb * 128 + col);
      }
      sl.sa = As_g[(size_t)srow * KB + kb];
      sl.sw = Bs_g[(size_t)bblk * KB + kb];
    };
    auto lstore = [&](int buf, const Slot& sl) {
      uint8_t* As = smem + buf * (BM + BN) * PITCH;
      uint8_t* Bs = As + BM * PITCH;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int c = tid + i * 256, r = c >> 3, col = (c & 7) * 16;
        *(u32x4_t*)(As + r * PITCH + col) = sl.a[i];
        *(u32x4_t*)(Bs + r * PITCH + col) = sl.b[i];
      }
      if (tid < BM) sa_lds[buf * BM + tid] = sl.sa;
      if ((tid & 63) == 0) sw_lds[buf * 4 + (tid >> 6)] = sl.sw;
    };

    float4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int n = 0; n < 4; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};

    // register ring: slot d holds block kb+1 for kb = d (mod P), issued in consumption order
    Slot ring[FP8_P];
    {
      Slot s0;
      gload(0, s0);
      lstore(0, s0);
    }
#pragma unroll
    for (int d = 0; d < FP8_P; d++) {
      gload(d + 1, ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    for (int kb0 = 0; kb0 < KB; kb0 += FP8_P) {
#pragma unroll
      for (int d = 0; d < FP8_P; d++) {
        const int kb = kb0 + d;
        const int buf = kb & 1;
        if (kb < KB) {
          const uint8_t* As = smem + buf * (BM + BN) * PITCH;
          const uint8_t* Bs = As + BM * PITCH;
          int8v_t af[4], bfr[4];
          const int koff = (lane >> 4) * 32;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const u32x4_t* pa = (const u32x4_t*)(As + (wm * 64 + i * 16 + (lane & 15)) * PITCH + koff);
            u32x4_t x0 = pa[0], x1 = pa[1];
            af[i] = int8v_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            const u32x4_t* pb = (const u32x4_t*)(Bs + (wn * 64 + i * 16 + (lane & 15)) * PITCH + koff);
            u32x4_t y0 = pb[0], y1 = pb[1];
            bfr[i] = int8v_t{(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3], (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
          }
          const float sbw = sw_lds[buf * 4 + wave];
          float4_t sav[4];
#pragma unroll
          for (int i = 0; i < 4; i++)
            sav[i] = *(const float4_t*)(sa_lds + buf * BM + wm * 64 + i * 16 + (lane >> 4) * 4);
#pragma unroll
          for (int i = 0; i < 4; i++)
#pragma unroll
            for (int n = 0; n < 4; n++) {
              float4_t tmp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  af[i], bfr[n], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
              for (int r = 0; r < 4; r++) acc[i][n][r] = __builtin_fmaf(tmp[r], sav[i][r] * sbw, acc[i][n][r]);
            }
        }
        // block kb+1 into the other buffer (its readers finished before the last barrier);
        // past the end this writes a buffer that is not read again
        lstore(buf ^ 1, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
        gload(kb + 1 + FP8_P, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
      }
    }

    // SwiGLU epilogue through LDS (fp32 tile, gate columns [0, HN), up [HN, BN))
    constexpr int CP = BN + 4;
    float* cs = (float*)smem;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int n = 0; n < 4; n++)
#pragma unroll
        for (int r = 0; r < 4; r++)
          cs[(wm * 64 + i * 16 + (lane >> 4) * 4 + r) * CP + wn * 64 + n * 16 + (lane & 15)] = acc[i][n][r];
    __syncthreads();
    uint16_t* H = (uint16_t*)p.out;
    for (int q = tid; q < BM * (HN / 2); q += 256) {
      int rr = q / (HN / 2), cp = (q % (HN / 2)) * 2;
      int row = m0 + rr, hc = n0 + cp;
      if (row >= mm || hc >= I) continue;
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 2; e++) {
        float gt = cs[rr * CP + cp + e], up = cs[rr * CP + HN + cp + e];
        float h = gt / (1.0f + expf(-gt)) * up;
        packed |= f32_to_bf16_rne(h) << (16 * e);
      }
      *(uint32_t*)(H + ((size_t)g * p.max_m + row) * I + hc) = packed;
    }
    __syncthreads();
  }
}

hipError_t gemm_fp8_swiglu(Fp8GemmArgs p, int cu_limit, hipStream_t s) {
  p.tiles_m = (p.max_m + g1::BM - 1) / g1::BM;
  p.tiles_n = (p.N / 2) / g1::HN;
  p.total_tiles = p.G * p.tiles_m * p.tiles_n;
  if (p.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemm_fp8_swiglu, dim3(fp8_grid(p.total_tiles, cu_limit)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- GEMM2
namespace g2 {
constexpr int BM = 128, BN = 128, BK = 64, PITCH = 72;  // bf16 elements per LDS row
}

__global__ __launch_bounds__(256) void k_gemm_bf16_fp8w(const Fp8GemmArgs p) {
  using namespace g2;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (BM + BN) * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K, KB = K / 128, N = p.N;

  const bool cover = (int)gridDim.x >= p.total_tiles;
  for (int t0 = blockIdx.x; t0 < (cover ? (int)gridDim.x : p.total_tiles); t0 += gridDim.x) {
    const int t = fp8_tile_of(t0, cover);
    if (t >= p.total_tiles) continue;
    int mt = t % p.tiles_m, rest = t / p.tiles_m;
    int nt = rest % p.tiles_n, g = rest / p.tiles_n;
    int mm = p.masked_m[g];
    mm = mm < 0 ? 0 : (mm > p.max_m ? p.max_m : mm);
    int m0 = mt * BM;
    if (m0 >= mm) continue;
    int n0 = nt * BN;
    const uint16_t* A = (const uint16_t*)p.a + (size_t)g * p.max_m * K;
    const uint8_t* B = p.b + (size_t)g * N * K;
    const float* Bs_g = p.b_s + (size_t)g * (N / 128) * KB;

    // A: 128 rows x 64 bf16 = 1024 chunks of 8 bf16 -> 4 per thread (row c/8, col (c%8)*8)
    // B: 128 rows x 64 fp8 = 512 chunks of 16 fp8 -> 2 per thread (row c/4, col (c%4)*16)
    // Rows are clamped into the valid ones (never stored), so every load is unconditional.
    int arow[4], brow[2];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int r = (tid + i * 256) >> 3;
      arow[i] = (m0 + r < mm) ? m0 + r : mm - 1;
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      int r = (tid + i * 256) >> 2;
      brow[i] = (n0 + r < N) ? n0 + r : N - 1;
    }
    struct Slot {
      u32x4_t a[4], b[2];
      float sw;  // weight scale of the step's 128 x 128 block
    };
    const int KT = K / BK;
    auto gload = [&](int kt, Slot& sl) {
      kt = kt < KT ? kt : KT - 1;  // prefetches past the end re-read the last step
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int c = tid + i * 256, col = (c & 7) * 8;
        sl.a[i] = *(const u32x4_t*)(A + (size_t)arow[i] * K + kt * BK + col);
      }
#pragma unroll
      for (int i = 0; i < 2; i++) {
        int c = tid + i * 256, col = (c & 3) * 16;
        sl.b[i] = *(const u32x4_t*)(B + (size_t)brow[i] * K + kt * BK + col);
      }
      sl.sw = Bs_g[(size_t)(n0 / 128) * KB + (kt >> 1)];
    };
    auto lstore = [&](int buf, const Slot& sl) {
      __bf16* As = smem + buf * (BM + BN) * PITCH;
      __bf16* Bs = As + BM * PITCH;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int c = tid + i * 256, r = c >> 3, col = (c & 7) * 8;
        *(u32x4_t*)(As + r * PITCH + col) = sl.a[i];
      }
#pragma unroll
      for (int i = 0; i < 2; i++) {
        int c = tid + i * 256, r = c >> 2, col = (c & 3) * 16;
        u32x4_t o0, o1;
#pragma unroll
        for (int w = 0; w < 4; w++) {
          bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(sl.b[i][w], 1.0f, false);
          bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(sl.b[i][w] >> 16, 1.0f, false);
          uint32_t ulo = *(uint32_t*)&lo, uhi = *(uint32_t*)&hi;
          if (w < 2) { o0[2 * w] = ulo; o0[2 * w + 1] = uhi; }
          else { o1[2 * (w - 2)] = ulo; o1[2 * (w - 2) + 1] = uhi; }
        }
        u32x4_t* dst = (u32x4_t*)(Bs + r * PITCH + col);
        dst[0] = o0;
        dst[1] = o1;
      }
    };

    float4_t acc[4][4], tmp[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int n = 0; n < 4; n++) { acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f}; tmp[i][n] = acc[i][n]; }

    // register ring: slot d holds step kt+1 for kt = d (mod P), issued in consumption order
    Slot ring[FP8_P2];
    float sw_cur;  // weight scale of the step being computed
    {
      Slot s0;
      gload(0, s0);
      lstore(0, s0);
      sw_cur = s0.sw;
    }
#pragma unroll
    for (int d = 0; d < FP8_P2; d++) {
      gload(d + 1, ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    for (int kt0 = 0; kt0 < KT; kt0 += FP8_P2) {
#pragma unroll
      for (int d = 0; d < FP8_P2; d++) {
        const int kt = kt0 + d;
        const int buf = kt & 1;
        if (kt < KT) {
          const __bf16* As = smem + buf * (BM + BN) * PITCH;
          const __bf16* Bs = As + BM * PITCH;
#pragma unroll
          for (int ks = 0; ks < BK / 32; ks++) {
            bf16x8_t af[4], bfr[4];
            const int koff = ks * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; i++) {
              af[i] = *(const bf16x8_t*)(As + (wm * 64 + i * 16 + (lane & 15)) * PITCH + koff);
              bfr[i] = *(const bf16x8_t*)(Bs + (wn * 64 + i * 16 + (lane & 15)) * PITCH + koff);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
              for (int n = 0; n < 4; n++)
                tmp[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[n], tmp[i][n], 0, 0, 0);
          }
          if ((kt & 1) == 1) {  // end of a 128-wide scale block: promote
            const float sbw = sw_cur;
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
              for (int n = 0; n < 4; n++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                  acc[i][n][r] = __builtin_fmaf(tmp[i][n][r], sbw, acc[i][n][r]);
                  tmp[i][n][r] = 0.f;
                }
          }
        }
        // step kt+1 into the other buffer; past the end this writes a buffer not read again
        sw_cur = ring[d].sw;
        lstore(buf ^ 1, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
        gload(kt + 1 + FP8_P2, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
      }
    }
    float* O = (float*)p.out;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int n = 0; n < 4; n++) {
        int col = n0 + wn * 64 + n * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; r++) {
          int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
          if (row < mm && col < N) O[((size_t)g * p.max_m + row) * N + col] = acc[i][n][r];
        }
      }
  }
}

hipError_t gemm_bf16_fp8w(Fp8GemmArgs p, int cu_limit, hipStream_t s) {
  p.tiles_m = (p.max_m + g2::BM - 1) / g2::BM;
  p.tiles_n = (p.N + g2::BN - 1) / g2::BN;
  p.total_tiles = p.G * p.tiles_m * p.tiles_n;
  if (p.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemm_bf16_fp8w, dim3(fp8_grid(p.total_tiles, cu_limit)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mxg
