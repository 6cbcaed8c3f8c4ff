// gemv_w4a16.hip -- NVFP4-weight x bf16-activation GEMV for decode batches (W4A16).
//
// Operation (the nvfp4_gemv row of the Helion pretuned-kernel table: NVFP4 decode GEMV
// at M = 1, W4A16 variant; single-stream decode in "The CuteDSL Gamble"):
//   out[m, n] = g_w * sum_k x[m, k] * dec(W)[n, k],  m < M <= 4, n < N,
// with x bf16 [M, K], W NVFP4 (codes [N, K/2], e4m3 scales [N, K/16]), fp32 sums.
//
// At batch 1 the work is a stream of the weight bytes; the layout is chosen so that
// every CU streams even when N is small:
//  * A unit is 16 output columns (16 weight rows, one 16x16x32 MFMA tile).  The 8 waves
//    of a workgroup split the unit's K range: wave w takes the 128-K chunks w, w + 8, ...
//    (K % 1024 == 0 gives every wave the same count), so a unit spreads over all 8 waves
//    and N / 16 units keep the grid busy.  Persistent grid, units blockIdx + i * grid.
//  * Each wave streams its chunks through a private ring of S LDS stages by DMA
//    (global_load_lds: 16 rows x 64 code bytes, then 16 rows x 8 scale bytes); the ring
//    runs across units, with S - 1 chunks in flight and explicit vmcnt waits.  No
//    workgroup barrier is needed inside a unit.
//  * The activations are read once per workgroup into LDS as fp16: row m is scaled by
//    2^s_m (s_m from the row's largest bf16 exponent, so that its largest magnitude is
//    below 2^15), which keeps every bf16 value exact in fp16 except those below
//    2^-28 times the row's largest magnitude.  The epilogue multiplies by 2^-s_m again.
//  * Weights are decoded exactly to fp16 (e2m1 * e4m3 has at most 6 significant bits);
//    products are exact in the fp32 MFMA accumulation.  The K order inside a chunk is
//    permuted identically on both operands (only the summation order changes).
//  * At a unit's end the 8 waves' partial tiles meet in LDS (double-buffered by unit
//    parity, one barrier per unit) and wave 0 adds them in wave order and stores.
// LDS layouts follow how gfx950 serves 16-byte reads (four passes of 16 lanes with the
// same lane bit 5 and the same parity of lane bits 2..4): weight code rows (64 bytes)
// hold 16-byte chunk c at c ^ 2 * (row bit 3); fp16 activation rows are padded by 16
// bytes; the two scale bytes a lane needs are read as one broadcast dword.
#include "device_common.h"
#include "kernels.h"

namespace mxg {

namespace gv {
constexpr int CK = 128;                          // K elements per chunk
constexpr int ROWS = 16;                         // weight rows (output columns) per unit
constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int S = 8;                             // ring stages per wave
constexpr int CODE = ROWS * (CK / 2);            // 1024 code bytes per stage
constexpr int STAGE = CODE + ROWS * (CK / 16);   // + 128 scale bytes
constexpr int APAD = 8;                          // fp16 padding per activation row
constexpr int ACT = GEMV_MAX_MK + GEMV_MAX_M * APAD;
}  // namespace gv

__device__ __forceinline__ int gv_swz(int r) { return (r >> 2) & 2; }

template <int EPI>
__global__ __launch_bounds__(gv::THREADS) void k_gemv_w4a16(const GemvArgs p) {
  using namespace gv;
  __shared__ __attribute__((aligned(16))) uint8_t ring[WAVES][S][STAGE];
  __shared__ __attribute__((aligned(16))) _Float16 act[ACT];
  __shared__ __attribute__((aligned(16))) float4_t red[2][WAVES][64];
  __shared__ uint32_t rowmax[GEMV_MAX_M];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.M, K = p.K, N = p.N;
  const int apitch = K + APAD;
  const int n_units = (N + ROWS - 1) / ROWS;
  const int grid = gridDim.x, bx = blockIdx.x;
  if (bx >= n_units) return;  // uniform over the workgroup
  const int nu = (n_units - 1 - bx) / grid + 1;
  const int cpw = K / CK / WAVES;  // chunks per wave per unit
  const int F = nu * cpw;

  // ---- weight DMA cursor: step f is chunk wave + 8 (f % cpw) of unit bx + (f / cpw) grid;
  // steps past the end repeat the last chunk so that every step issues the same ops
  const int r_dma = lane >> 2;        // code row of this lane
  const int r_sc = (lane & 31) >> 1;  // scale row of this lane (lanes < 32)
  int i_f = 0, j_f = 0, f_iss = 0;
  const uint8_t* csrc;
  const uint8_t* ssrc;
  auto set_unit = [&](int i) {
    const int n0 = (bx + i * grid) * ROWS;
    const int rc = n0 + r_dma < N ? n0 + r_dma : N - 1;  // rows past N re-read row N - 1 (never stored)
    const int rs = n0 + r_sc < N ? n0 + r_sc : N - 1;
    csrc = p.w + (size_t)rc * (K / 2) + (((lane & 3) ^ gv_swz(r_dma)) << 4);
    ssrc = p.w_sf + (size_t)rs * (K / 16) + (lane & 1) * 4;
  };
  set_unit(0);
  auto issue = [&]() {
    uint8_t* st = &ring[wave][f_iss % S][0];
    const int c = wave + WAVES * j_f;
    dma16(csrc + (size_t)c * (CK / 2), st);
    if (lane < 32) dma4(ssrc + (size_t)c * (CK / 16), st + CODE);
    f_iss++;
    if (f_iss < F) {
      if (++j_f == cpw) {
        j_f = 0;
        set_unit(++i_f);
      }
    }
  };
#pragma unroll
  for (int k = 0; k < S - 1; k++) issue();

  // ---- activations: one pass of 16-byte loads copies the bf16 rows into the fp16
  // buffer's place and takes the row maxima of |x| (wavefront reduction, then one LDS
  // atomic per wave and row); then each thread converts its own 16-byte units in place
  if (tid < GEMV_MAX_M) rowmax[tid] = 0;
  __syncthreads();
  const int upr = K / 8;  // 16-byte units (8 elements) per row
  for (int m = 0; m < M; m++) {
    uint32_t mx = 0;
    for (int u = tid; u < upr; u += THREADS) {
      const u32x4_t v = *(const u32x4_t*)(p.x + (size_t)m * K + 8 * u);
#pragma unroll
      for (int e = 0; e < 4; e++) mx = max(mx, max(v[e] & 0x7FFFu, (v[e] >> 16) & 0x7FFFu));
      *(u32x4_t*)(act + m * apitch + 8 * u) = v;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
    if (lane == 0) atomicMax(&rowmax[m], mx);
  }
  __syncthreads();
  auto row_shift = [&](int m) {
    const int e_field = (int)(rowmax[m] >> 7);            // biased exponent of the row maximum
    return 14 - ((e_field > 0 ? e_field : 1) - 127);      // largest magnitude lands below 2^15
  };
  for (int m = 0; m < M; m++) {
    const int sh = row_shift(m);
    for (int u = tid; u < upr; u += THREADS) {
      u32x4_t* cell = (u32x4_t*)(act + m * apitch + 8 * u);
      const u32x4_t v = *cell;
      u32x4_t h;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const _Float16 lo = (_Float16)__builtin_ldexpf(__uint_as_float(v[e] << 16), sh);
        const _Float16 hi = (_Float16)__builtin_ldexpf(__uint_as_float(v[e] & 0xFFFF0000u), sh);
        h[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *cell = h;
    }
  }
  __syncthreads();

  // ---- main loop
  const int n = lane & 15, q = lane >> 4;
  const int ma = n < M ? n : M - 1;  // activation row of this lane's MFMA column
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  int j_c = 0, i_c = 0;
  for (int f = 0; f < F; f++) {
    issue();
    wait_vmcnt<2 * (S - 1)>();  // chunk f landed; S - 1 chunks (2 DMAs each) behind it
    const uint8_t* st = &ring[wave][f % S][0];
    const u32x4_t raw = *(const u32x4_t*)(st + n * 64 + ((q ^ gv_swz(n)) << 4));
    const uint32_t sw = *(const uint32_t*)(st + CODE + n * 8 + (q >> 1) * 4);
    const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw >> (16 * (q & 1)), 1.0f, false);
    const half2_t s0 = half2_t{s01[0], s01[0]}, s1 = half2_t{s01[1], s01[1]};
    const int c = wave + WAVES * j_c;
    const _Float16* arow = act + ma * apitch + c * CK + 32 * q;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      // dword s of the lane's chunk: K 32 q + 8 s .. + 7 of the chunk, 16-block 2 q + s / 2
      const half8_t wv = decode8_e2m1_f16(raw[s], s < 2 ? s0 : s1);
      const half8_t av = *(const half8_t*)(arow + 8 * s);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, av, acc, 0, 0, 0);
    }
    if (++j_c == cpw) {
      // unit end: lane (n, q) holds rows 4q .. 4q + 3 of the 16 weight rows (output
      // columns n0 + 4q + r) for activation row n
      red[i_c & 1][wave][lane] = acc;
      acc = float4_t{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (wave == 0) {
        float4_t v = red[i_c & 1][0][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++) v += red[i_c & 1][w][lane];
        const int m = n, c0 = (bx + i_c * grid) * ROWS + 4 * q;
        if (m < M) {
          const int sh = row_shift(m);
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; r++) o[r] = __builtin_ldexpf(v[r] * p.g_w, -sh);
          const size_t base = (size_t)m * N + c0;
          if (c0 + 4 <= N && (N & 3) == 0) {
            if constexpr (EPI == EPI_BF16) {
              const uint32_t lo = bf16x2_rne(o[0], o[1]);
              const uint32_t hi = bf16x2_rne(o[2], o[3]);
              *(u32x2_t*)((uint16_t*)p.out + base) = u32x2_t{lo, hi};
            } else {
              *(float4_t*)((float*)p.out + base) = float4_t{o[0], o[1], o[2], o[3]};
            }
          } else {
            for (int r = 0; r < 4 && c0 + r < N; r++) {
              if constexpr (EPI == EPI_BF16) ((uint16_t*)p.out)[base + r] = (uint16_t)f32_to_bf16_rne(o[r]);
              else ((float*)p.out)[base + r] = o[r];
            }
          }
        }
      }
      j_c = 0;
      i_c++;
    }
  }
  wait_vmcnt<0>();  // the trailing re-reads land before the waves end
}

hipError_t gemv_nvfp4_w4a16(GemvArgs p, int epi, int cu_limit, hipStream_t s) {
  if (p.M < 1 || p.M > GEMV_MAX_M || p.M * p.K > GEMV_MAX_MK || p.K % (gv::CK * gv::WAVES) != 0 || p.N < 1)
    return hipErrorNotSupported;
  const void* k = epi == EPI_BF16 ? (const void*)k_gemv_w4a16<EPI_BF16> : (const void*)k_gemv_w4a16<EPI_F32>;
  int grid = resident_grid(k, gv::THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;
  const int n_units = (p.N + gv::ROWS - 1) / gv::ROWS;
  if (grid > n_units) grid = n_units;
  if (epi == EPI_BF16) hipLaunchKernelGGL(k_gemv_w4a16<EPI_BF16>, dim3(grid), dim3(gv::THREADS), 0, s, p);
  else hipLaunchKernelGGL(k_gemv_w4a16<EPI_F32>, dim3(grid), dim3(gv::THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace mxg
