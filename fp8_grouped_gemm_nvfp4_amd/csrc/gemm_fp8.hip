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
//   scales; fp8 is widened exactly to bf16 and the bf16 MFMA (16x16x32)
//   accumulates each 128-K scale block before promotion.  Output fp32 [G, max_m, H].
//
// Both kernels are persistent and stream the weights through LDS by DMA; at the
// prefill shapes they are bound by the L1 -> L2 request rate of the CUs, so every
// expert's weights are read once (256-row M tiles) and the activations, which the N
// tiles of an expert re-read, come from the L2 of one XCD.
#include "kernels.h"
#include "stream_common.h"

namespace mxg {

// ----------------------------------------------------------------------------- GEMM1
// Persistent and weight-streaming.  A work item (stream_common.h) is (expert g, 256-row M
// tile, 64 h columns): the item's 64 gate rows and 64 up rows of W13 against up to 256
// activation rows, so every weight panel is read from HBM once per expert whenever
// masked_m <= 256.
//
// Operands travel from HBM into LDS by DMA through two rings that run on across item
// boundaries: activations (and their row scales) two steps ahead, so that a step never
// waits out the round trip of a DMA issued in it, and weights (and the two block scales)
// DB = 2 steps ahead (the LDS holds three activation and three weight stages).  One step
// is one 128-wide K block.  Activation rows are read straight from the token rows of x
// (a table gives each expert row's token), so they are never copied per expert.  Rows
// past masked_m are not fetched at all in 8-row groups (the rest re-read the last valid
// row).  In LDS, 128-byte row r holds its eight 16-byte chunks XOR-permuted by
// (r ^ r >> 3) & 7, which keeps the MFMA operand reads free of bank conflicts.
//
// Waves: 12, in two roles.  Waves 8..11 (one per SIMD) issue every DMA; waves 0..7 (two
// per SIMD) only read fragments, run MFMAs and store h.  One barrier per step hands a
// step's stages from one role to the other.  MFMA wave w owns the 16-row groups 16 w
// and 16 w + 128 and every column of the item (its 64 gate and 64 up weight rows), so the
// SwiGLU epilogue runs in registers; interleaving the row groups keeps every MFMA wave
// busy when masked_m <= 128, and row groups that are entirely masked skip their MFMAs.
#ifndef MXG_F1_DB
#define MXG_F1_DB 2
#endif
// Wait until at most n (0..14) of this wave's vector memory operations are outstanding.
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    default: wait_vmcnt<14>(); break;
  }
}
namespace f1 {
constexpr int BM = 256, BN = 128, HN = BN / 2, BK = 128;
constexpr int MW = 8, DW = 4;  // MFMA waves, data waves
constexpr int WAVES = MW + DW, THREADS = WAVES * 64;
constexpr int A_STAGE = BM * BK + BM * 4;  // codes, then the fp32 row scales
constexpr int SA = 3;                      // activation slots: two steps in flight
constexpr int B_STAGE = BN * BK + 16;      // codes, then the {gate, up} block scales
constexpr int MAX_G = STREAM_MAX_G;
static_assert(BM == STREAM_BM, "M tile of the shared work distribution");
// DMA instructions per data wave per step: up to 8 of activations (the 8-row groups
// 8 pw + 32 j, so that the data waves share them evenly when masked_m is small), 4 of
// weights (32 rows); data wave 0 adds the activation row scales, data wave 1 the two
// weight block scales
constexpr int A_OPS = 8, B_OPS = 4;
// a data wave's DMAs in one step: activations, one scale block (activation or weight
// scales, never both), the tokens of an item, weights
static_assert(A_OPS + 1 + 1 + B_OPS <= 14, "one step's DMAs fit the waits of wait_vmcnt_le");
// Activation rows are read straight from the token rows of x: each data wave DMAs the
// tokens of its 64 rows of item k + 2 (one dword per lane) into a ring of three LDS slots
// when it sets up item k (k >= 1; the prologue loads items 0..2), and every set-up comes
// at least two steps after the DMA it reads, so a step's wait has covered it.
constexpr int TOK_SLOTS = 3;
}  // namespace f1

__device__ __forceinline__ int f1_swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int DB, bool SPLIT, bool DBG>
__global__ __launch_bounds__(f1::THREADS) void k_gemm_fp8_swiglu(const Fp8GemmArgs p) {
  using namespace f1;
  constexpr int SB = DB + 1;
  static_assert(DB >= 2, "B(s + 1) must be issued before A(s + 1)");
  __shared__ __attribute__((aligned(16))) uint8_t ringA[SA * A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ringB[SB * B_STAGE];
  __shared__ int tprefix[MAX_G + 1];
  __shared__ int mm_s[MAX_G];
  __shared__ int tok_s[TOK_SLOTS][DW][A_OPS * 8];  // per data wave: the tokens of its rows, per item

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int G = p.G, K = p.K, KB = K / BK, N = p.N, I = N / 2, cap = p.max_m, capS = p.a_s_stride;
  const int tiles_n = I / HN;

  stream_tile_prefix(p.masked_m, p.G, p.max_m, tprefix, mm_s, tid, true);
  const int total = __builtin_amdgcn_readfirstlane(tprefix[G]) * tiles_n;
  const int grid = gridDim.x;
  const int bx = stream_bx();
  if (bx >= total) return;
  const int n_items = (total - 1 - bx) / grid + 1;
  const int nsteps = n_items * KB;

  auto item_at = [&](int k) { return stream_item(bx + k * grid, tiles_n, G, tprefix, mm_s, HN, true); };

  if (wave >= MW) {
    // ======== data waves: activations two steps ahead, weights DB steps ahead ========
    const int pw = wave - MW;
    // DMA cursors: per-lane sources of the current item (rows past masked_m re-read the
    // last valid row, never stored); past the last step they stay on it
    // byte offsets of the token rows from x (below 2^32, checked by the host)
    uint32_t asrc[A_OPS];
    const float* asrc_s;
    int a_n = 0;  // activation DMAs per step: 8-row groups entirely past masked_m are skipped
    int tok_issued = 0;  // token DMAs issued by the last a_setup (0 or 1)
    // the tokens of this wave's rows 8 pw + 32 j + (l & 7), j = l >> 3, of item k into
    // slot k % TOK_SLOTS (rows past masked_m take the last valid row's token)
    auto issue_tok = [&](int k) {
      const StreamItem it = item_at(k);
      const int r = 8 * pw + 32 * (lane >> 3) + (lane & 7);
      const int row = it.m0 + r < it.mm ? it.m0 + r : it.mm - 1;
      dma4(p.a_tok + (size_t)it.g * cap + row, &tok_s[k % TOK_SLOTS][pw][0]);
    };
    // item k's DMA sources; its tokens are in slot k % TOK_SLOTS
    auto a_setup = [&](int k) {
      const StreamItem it = item_at(k);
      const int left = it.mm - it.m0 - 8 * pw;
      a_n = left <= 0 ? 0 : (left >= 32 * A_OPS ? A_OPS : (left + 31) / 32);
#pragma unroll
      for (int j = 0; j < A_OPS; j++) {
        const int r = 8 * pw + 32 * j + (lane >> 3);
        // clamped, so that any table entry addresses a row of x
        const int t = tok_s[k % TOK_SLOTS][pw][8 * j + (lane >> 3)];
        const int tok = t < 0 ? 0 : (t >= p.tokens ? p.tokens - 1 : t);
        asrc[j] = (uint32_t)tok * K + (((lane & 7) ^ f1_swz(r)) << 4);
      }
      const int rs = it.m0 + 4 * lane < capS - 4 ? it.m0 + 4 * lane : capS - 4;
      asrc_s = p.a_s + (size_t)it.g * KB * capS + rs;
      tok_issued = k >= 1 && k + 2 < n_items;  // the prologue loads the tokens of items 0..2
      if (tok_issued) issue_tok(k + 2);
    };
    uint32_t bsrc[B_OPS];
    const uint8_t* bbase = p.b;
    const float* bsrc_s;
    auto b_setup = [&](const StreamItem& it) {
      bbase = p.b + (size_t)it.g * N * K;
#pragma unroll
      for (int j = 0; j < B_OPS; j++) {
        const int r = 32 * pw + 8 * j + (lane >> 3);
        const int brow = r < HN ? it.n0 + r : I + it.n0 + (r - HN);
        bsrc[j] = (uint32_t)brow * K + (((lane & 7) ^ f1_swz(r)) << 4);
      }
      const int blk = (lane == 0 ? it.n0 : I + it.n0) / 128;
      bsrc_s = p.b_s + ((size_t)it.g * (N / 128) + blk) * KB;
    };
    int a_k = 0, a_kb = 0, a_step = 0, a_st = 0;
    int b_k = 0, b_kb = 0, b_step = 0, b_st = 0;
    int a_cnt = 0;  // DMA instructions of the last issue_a
    auto issue_a = [&]() {  // A(step) into slot step % SA
      uint8_t* st = ringA + a_st * A_STAGE;
#pragma unroll
      for (int j = 0; j < A_OPS; j++)
        if (j < a_n) dma16_s(p.a, asrc[j] + a_kb * BK, st + (8 * pw + 32 * j) * BK);
      if (pw == 0) dma16(asrc_s + (size_t)a_kb * capS, st + BM * BK);
      a_cnt = a_n + (pw == 0);
      a_st = a_st == SA - 1 ? 0 : a_st + 1;
      if (a_step + 1 < nsteps) {
        a_step++;
        if (++a_kb == KB) {
          a_kb = 0;
          a_setup(++a_k);
          a_cnt += tok_issued;
        }
      }
    };
    auto issue_b = [&]() {  // B(step) into stage step % SB: B_OPS (+ 1) instructions
      uint8_t* st = ringB + b_st * B_STAGE;
#pragma unroll
      for (int j = 0; j < B_OPS; j++) dma16_s(bbase, bsrc[j] + b_kb * BK, st + (32 * pw + 8 * j) * BK);
      if (pw == 1 && lane < 2) dma4(bsrc_s + b_kb, st + BN * BK);
      b_st = b_st + 1 == SB ? 0 : b_st + 1;
      if (b_step + 1 < nsteps) {
        b_step++;
        if (++b_kb == KB) {
          b_kb = 0;
          b_setup(item_at(++b_k));
        }
      }
    };
    for (int k = 0; k < TOK_SLOTS && k < n_items; k++) issue_tok(k);
    wait_vmcnt<0>();  // the tokens of items 0..2
    a_setup(0);
    b_setup(item_at(0));
#pragma unroll
    for (int i = 0; i < DB; i++) issue_b();
    issue_a();
    issue_a();
    // B(0 .. DB - 1), A(0) and any tokens issued with it have landed; A(1) (and tokens
    // issued with it) may stay outstanding
    wait_vmcnt_le(a_cnt);
    for (int s = 0; s < nsteps; s++) {
      // A(s) and B(s) are in LDS, and the MFMA waves are done with step s - 1, whose
      // activation slot and weight stage the next issues overwrite
      __syncthreads();
      issue_a();  // A(s + 2)
      issue_b();  // B(s + DB)
      // everything issued before this step (A(s + 1) and B(s + 1) among it) lands before
      // the next barrier; only this step's DMAs may stay outstanding
      wait_vmcnt_le(a_cnt + B_OPS + (pw == 1));
    }
    wait_vmcnt<0>();  // the trailing re-reads land before the workgroup ends
    return;
  }

  // ======== MFMA waves ========
  // Wave w owns the 16-row groups 16 w and 16 w + 128 of the M tile and all 128 weight
  // rows of the item (gate rows 0..63, up rows 64..127), so SwiGLU pairs fragment group
  // n with n + 4 in registers.  The weight fragments are read two groups ahead.
  float4_t acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int n = 0; n < 8; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};

  StreamItem cit = item_at(0);
  int c_k = 0, c_kb = 0, c_sb = 0, c_sa = 0;
  const int q = lane >> 4, rr = lane & 15;

  // h rows: with SPLIT they are 2I wide, hi = bf16(h) in columns [0, I), lo = bf16(h - hi)
  // in [I, 2I) (h - hi is exact in fp32, so hi + lo holds h to about 16 significant bits).
  // Masked rows store into the scratch row after the last expert.
  constexpr int PL = SPLIT ? 2 : 1;
  const int RS = PL * I;  // h row stride (elements)
  // Fragment of 16-byte chunks 2q, 2q + 1 (K 32 q .. 32 q + 31) of row 16 j + rr of a
  // stage: f1_swz(16 j + rr) = f1_swz(rr) ^ (2 j mod 8), so the lane's byte offset in the
  // row is its offset for j = 0 with (j mod 4) XORed into bits 5..6, and the second chunk
  // sits at the first one XOR 16.
  // The base is re-derived every step (an opaque copy), so the compiler does not keep
  // eight offsets live across the loop.
  const int frag_lane = rr * BK + (((2 * q) ^ f1_swz(rr)) << 4);
  int frag_off = frag_lane;
  auto frag = [&](const uint8_t* stage, int j) {
    const uint8_t* row = stage + 16 * j * BK;
    const int off = frag_off ^ ((j & 3) << 5);
    const u32x4_t x0 = *(const u32x4_t*)(row + off);
    const u32x4_t x1 = *(const u32x4_t*)(row + (off ^ 16));
    return int8v_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };

  for (int s = 0; s < nsteps; s++) {
    __syncthreads();  // A(s) and B(s) are in LDS
    frag_off = frag_lane;
    asm volatile("" : "+v"(frag_off));
    const int left = cit.mm - cit.m0 - 16 * wave;  // valid rows from this wave's first row
    const int nv = left <= 0 ? 0 : (left > 128 ? 2 : 1);
    if (nv > 0) {
      const uint8_t* As = ringA + c_sa * A_STAGE;
      const uint8_t* Bs = ringB + c_sb * B_STAGE;
      int8v_t af[2];
      float4_t sw[2][2];  // row scale x {gate, up} block scale
      const float* AS = (const float*)(As + BM * BK);
      const float* WS = (const float*)(Bs + BN * BK);
      const float wg = WS[0], wu = WS[1];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        if (i >= nv) break;
        af[i] = frag(As, wave + 8 * i);
        const float4_t sa = *(const float4_t*)(AS + 16 * wave + 128 * i + 4 * q);
        sw[i][0] = sa * wg;
        sw[i][1] = sa * wu;
      }
      int8v_t bf[8];
      bf[0] = frag(Bs, 0);
      bf[1] = frag(Bs, 1);
#pragma unroll
      for (int n = 0; n < 8; n++) {
        if (n + 2 < 8) bf[n + 2] = frag(Bs, n + 2);
#pragma unroll
        for (int i = 0; i < 2; i++) {
          if (i >= nv) break;
          // 128 exact e4m3 products summed in fp32 (unit e8m0 scales), then promoted with
          // the row's activation scale times the block's weight scale
          const float4_t t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf[n], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 4; r++) acc[i][n][r] = __builtin_fmaf(t[r], sw[i][n >> 2][r], acc[i][n][r]);
        }
      }
    }
    c_sb = c_sb + 1 == SB ? 0 : c_sb + 1;
    c_sa = c_sa == SA - 1 ? 0 : c_sa + 1;

    if (++c_kb == KB) {
      // SwiGLU in registers: lanes 2c and 2c+1 hold neighbouring columns of the same four
      // rows; one swap gives each lane both columns of two rows (rows +odd and +2+odd)
      if (nv > 0) {
        // the lane terms come from an opaque copy, so the compiler does not keep them
        // live (or spilled) across the step loop
        int el = lane;
        asm volatile("" : "+v"(el));
        const int q = el >> 4, rr = el & 15, odd = el & 1;
        uint16_t* H = (uint16_t*)p.out;
        uint16_t* scratch_row = H + (size_t)G * cap * RS;
#pragma unroll
        for (int i = 0; i < 2; i++) {
          if (i >= nv) break;
#pragma unroll
          for (int n = 0; n < 4; n++) {
            uint32_t b[PL][4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const float gt = acc[i][n][r], up = acc[i][n + 4][r];
              if constexpr (DBG) {  // the promoted GEMM1 sums, for stage checks only
                const int row = cit.m0 + 16 * wave + 128 * i + 4 * q + r;
                if (row < cit.mm) {
                  float* d = p.dbg_g1 + ((size_t)cit.g * cap + row) * N;
                  const int c = cit.n0 + 16 * n + rr;
                  d[c] = gt;
                  d[I + c] = up;
                }
              }
              const float h = gt / (1.0f + expf(-gt)) * up;
              b[0][r] = f32_to_bf16_rne(h);
              if constexpr (SPLIT) b[PL - 1][r] = f32_to_bf16_rne(h - __uint_as_float(b[0][r] << 16));
            }
            const int row0 = cit.m0 + 16 * wave + 128 * i + 4 * q;
            const int c = (cit.n0 + 16 * n + rr) & ~1;
            const int ra = row0 + odd, rb = row0 + 2 + odd;
            uint16_t* pa = ra < cit.mm ? H + ((size_t)cit.g * cap + ra) * RS + c : scratch_row + c;
            uint16_t* pb = rb < cit.mm ? H + ((size_t)cit.g * cap + rb) * RS + c : scratch_row + c;
#pragma unroll
            for (int pl = 0; pl < PL; pl++) {
              const uint32_t y0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? b[pl][0] : b[pl][1]), 0xB1, 0xF, 0xF, false);
              const uint32_t y1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? b[pl][2] : b[pl][3]), 0xB1, 0xF, 0xF, false);
              *(uint32_t*)(pa + pl * I) = odd ? (y0 | (b[pl][1] << 16)) : (b[pl][0] | (y0 << 16));
              *(uint32_t*)(pb + pl * I) = odd ? (y1 | (b[pl][3] << 16)) : (b[pl][2] | (y1 << 16));
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int n = 0; n < 8; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
      c_kb = 0;
      if (++c_k < n_items) cit = item_at(c_k);
    }
  }
}

template <int DB, bool SPLIT, bool DBG>
static hipError_t launch_fp8_swiglu(Fp8GemmArgs p, int cu_limit, hipStream_t s) {
  using namespace f1;
  if (p.G > MAX_G || (p.N / 2) % HN != 0 || p.K % BK != 0 || p.a_s_stride % 4 != 0 ||
      p.a_s_stride < p.max_m || p.a_s_stride < 4)
    return hipErrorNotSupported;
  if ((long long)p.G * ((p.max_m + BM - 1) / BM) * ((p.N / 2) / HN) > 0x7FFFFFFFLL) return hipErrorNotSupported;
  // the DMA offsets (of token rows, and from an expert's weight base) are 32-bit
  if ((unsigned long long)p.tokens * p.K >= (1ull << 32) || (unsigned long long)p.N * p.K >= (1ull << 32) ||
      !p.a_tok)
    return hipErrorNotSupported;
  const void* k = (const void*)k_gemm_fp8_swiglu<DB, SPLIT, DBG>;
  const int grid = resident_grid(k, THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_fp8_swiglu<DB, SPLIT, DBG>), dim3(grid), dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t gemm_fp8_swiglu(Fp8GemmArgs p, int cu_limit, hipStream_t s) {
  if (p.G <= 0 || p.max_m <= 0 || p.N <= 0 || p.K <= 0) return hipSuccess;
  if (p.dbg_g1)
    return p.h_split ? launch_fp8_swiglu<MXG_F1_DB, true, true>(p, cu_limit, s)
                     : launch_fp8_swiglu<MXG_F1_DB, false, true>(p, cu_limit, s);
  return p.h_split ? launch_fp8_swiglu<MXG_F1_DB, true, false>(p, cu_limit, s)
                   : launch_fp8_swiglu<MXG_F1_DB, false, false>(p, cu_limit, s);
}

// ----------------------------------------------------------------------------- GEMM2
// Persistent and weight-streaming like GEMM1.  A work item is (expert g, 256-row M tile,
// BN output columns); a step is 64 K: 256 bf16 h rows x 128 bytes and BN e4m3 weight rows
// x 64 bytes, both by DMA (h one step ahead, W2 DB steps ahead).  The weights are widened
// exactly to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8, scale 1) for the bf16 MFMA.
// The waves own interleaved 16-row groups as in GEMM1 and BN / 2 columns each, which lie in
// one 128-row block of W2's scales, so a wave's block scale c_k is one number per 128-K
// block.  Instead of summing each block apart and promoting it (a second set of
// accumulators), a wave keeps one sum in units of the current block's scale: before block
// k it multiplies the sum by c_{k-1} / c_k, and the epilogue multiplies by the last c_k.
// The sum equals sum_k c_k * P_k exactly up to those fp32 roundings (about three per
// block), and the freed registers pay for twice the columns per item, which halves the
// re-reads of h.  A block whose scale is zero contributes nothing and is skipped.  Row
// groups past masked_m hold zeros and are neither rescaled nor computed.  The MFMA takes
// the weights as its first operand, so it computes the transposed tile and each lane ends
// with four consecutive output columns of one row (16-byte stores, no transposition).
// Inside a step the K order is permuted identically on both operands (only the fp32
// summation order changes): lane quarter q takes K 16q .. 16q + 15 of the step, the first
// 8 in the first MFMA and the rest in the second, so that a lane's W2 bytes for the step
// are one 16-byte read and its h elements two.  LDS rows are XOR-swizzled (h: 16-byte
// chunk ^ (r ^ r >> 3) & 7; W2: 16-byte chunk ^ 2 * (r bit 3)).
namespace f2 {
constexpr int BM = 256, BK = 64;
constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int A_STAGE = BM * BK * 2;  // bf16 h rows, 128 bytes each
constexpr int DW = 4;                 // waves 0..3 issue every DMA
constexpr int A_OPS = 8;              // h DMAs per issuing wave per step (64 rows)
template <int NBW>
struct Cfg {
  static constexpr int BN = 32 * NBW;              // two waves across, 16 * NBW columns each
  static constexpr int B_STAGE = BN * BK + 16;     // e4m3 W2 rows, 64 bytes each, then two block scales
  static constexpr int B_OPS = BN * BK / (DW * 1024);  // weight DMAs per issuing wave per step
};
}  // namespace f2

// W2 rows (64 bytes): 16-byte chunk c sits at c ^ 2 * (r bit 3).  A 16-byte LDS read is
// served in four passes of 16 lanes (same lane bit 5, same parity of lane bits 2..4);
// with this permutation (and f1_swz on the 128-byte h rows) the lanes of a pass hit 16
// different slots of the 256-byte bank row.
__device__ __forceinline__ int f2_swz_b(int r) { return (r >> 2) & 2; }

template <int NBW, int DB>
__global__ __launch_bounds__(f2::THREADS) void k_gemm_bf16_fp8w(const Fp8GemmArgs p) {
  using namespace f2;
  constexpr int BN = Cfg<NBW>::BN, B_STAGE = Cfg<NBW>::B_STAGE, B_OPS = Cfg<NBW>::B_OPS;
  constexpr int WCOLS = 16 * NBW;
  static_assert(B_OPS >= 1 && WCOLS <= 128 && 128 % WCOLS == 0, "a wave's columns share one scale block");
  constexpr int SA = 2, SB = DB + 1;
  __shared__ __attribute__((aligned(16))) uint8_t ringA[SA * A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ringB[SB * B_STAGE];
  __shared__ int tprefix[f1::MAX_G + 1];
  __shared__ int mm_s[f1::MAX_G];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // K is the extent of A (h, or its hi and lo planes side by side); W2's K index wraps
  // at WK (= K, or I for the two planes)
  const int G = p.G, K = p.K, WK = p.b_k ? p.b_k : p.K, KB = WK / 128, N = p.N, cap = p.max_m;
  const int tiles_n = N / BN, KT = K / BK, WKT = WK / BK;

  stream_tile_prefix(p.masked_m, p.G, p.max_m, tprefix, mm_s, tid, false);
  const int total = __builtin_amdgcn_readfirstlane(tprefix[G]) * tiles_n;
  const int grid = gridDim.x;
  const int bx = stream_bx();
  if (bx >= total) return;
  const int n_items = (total - 1 - bx) / grid + 1;
  const int nsteps = n_items * KT;

  auto item_at = [&](int k) { return stream_item(bx + k * grid, tiles_n, G, tprefix, mm_s, BN, false); };

  // DMA sources: byte offsets from the item's expert base (below 2^32, checked by the host)
  uint32_t asrc[A_OPS];
  const uint8_t* abase = p.a;
  int a_n = 0;
  auto a_setup = [&](const StreamItem& it) {
    abase = p.a + (size_t)it.g * cap * K * 2;
    const int left = it.mm - it.m0 - 64 * wave;
    a_n = left <= 0 ? 0 : (left >= 8 * A_OPS ? A_OPS : (left + 7) / 8);
#pragma unroll
    for (int j = 0; j < A_OPS; j++) {
      const int r = 64 * wave + 8 * j + (lane >> 3);
      const int row = it.m0 + r < it.mm ? it.m0 + r : it.mm - 1;
      asrc[j] = (uint32_t)row * K * 2 + (((lane & 7) ^ f1_swz(r)) << 4);
    }
  };
  // issuing wave w DMAs weight rows 16 * (B_OPS * w + j) + lane / 4; lanes 0 and 1 of
  // wave 1 the scale blocks of the two column halves
  uint32_t bsrc[B_OPS];
  const uint8_t* bbase = p.b;
  uint32_t bsrc_s;  // byte offset of the item's first scale from b_s
  auto b_setup = [&](const StreamItem& it) {
    bbase = p.b + (size_t)it.g * N * WK;
#pragma unroll
    for (int j = 0; j < B_OPS; j++) {
      const int r = 16 * (B_OPS * wave + j) + (lane >> 2);
      bsrc[j] = (uint32_t)(it.n0 + r) * WK + (((lane & 3) ^ f2_swz_b(r)) << 4);
    }
    bsrc_s = 4u * (((uint32_t)it.g * (N / 128) + (it.n0 + (lane & 1) * WCOLS) / 128) * KB);
  };
  int a_k = 0, a_kt = 0, a_step = 0, a_st = 0;
  int b_k = 0, b_kt = 0, b_step = 0, b_st = 0;
  auto issue_a = [&]() {
    uint8_t* st = ringA + a_st * A_STAGE;
#pragma unroll
    for (int j = 0; j < A_OPS; j++)
      if (j < a_n) dma16_s(abase, asrc[j] + a_kt * (BK * 2), st + (64 * wave + 8 * j) * (BK * 2));
    a_st ^= 1;
    if (a_step + 1 < nsteps) {
      a_step++;
      if (++a_kt == KT) {
        a_kt = 0;
        a_setup(item_at(++a_k));
      }
    }
  };
  auto issue_b = [&]() {
    uint8_t* st = ringB + b_st * B_STAGE;
    const int wkt = b_kt < WKT ? b_kt : b_kt - WKT;  // W2 step of A step b_kt
#pragma unroll
    for (int j = 0; j < B_OPS; j++) dma16_s(bbase, bsrc[j] + wkt * BK, st + 16 * (B_OPS * wave + j) * BK);
    if (wave == 1 && lane < 2) dma4_s(p.b_s, bsrc_s + 4 * (wkt >> 1), st + BN * BK);
    b_st = b_st + 1 == SB ? 0 : b_st + 1;
    if (b_step + 1 < nsteps) {
      b_step++;
      if (++b_kt == KT) {
        b_kt = 0;
        b_setup(item_at(++b_k));
      }
    }
  };

  // Waves 0..3 issue every DMA while their SIMD partners 4..7 go straight to the MFMAs
  // after each barrier, which staggers the two waves of a SIMD (spreading the DMAs over
  // all eight waves measured 4% slower).
  const bool dw = wave < DW;
  if (dw) {
    const StreamItem it0 = item_at(0);
    a_setup(it0);
    b_setup(it0);
#pragma unroll
    for (int i = -DB; i < 0; i++) {
      if (i + 1 >= 0) issue_a();
      issue_b();
    }
  }

  // acc: the item's sums in units of the current block scale c_cur (0 before the first
  // block with a nonzero scale); between the end of an item and the next barrier, the
  // item's results (scaled)
  float4_t acc[4][NBW];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int n = 0; n < NBW; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
  float c_cur = 0.f;
  bool zblk = false;

  StreamItem cit = item_at(0);
  int c_k = 0, c_kt = 0, c_sa = 0, c_sb = 0;
  const int q = lane >> 4, rr = lane & 15;
  bool pend = false;
  StreamItem pit = cit;
  auto store_out = [&]() {
    float* O = (float*)p.out;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = pit.m0 + 16 * wm + 64 * i + rr;
#pragma unroll
      for (int n = 0; n < NBW; n++) {
        const int col = pit.n0 + WCOLS * wn + 16 * n + 4 * q;
        if (row < pit.mm) *(float4_t*)(O + ((size_t)pit.g * cap + row) * N + col) = acc[i][n];
        acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  for (int s = 0; s < nsteps; s++) {
    if (wave == 1) wait_vmcnt<B_OPS + 1>();
    else if (dw) wait_vmcnt<B_OPS>();
    __syncthreads();
    if (pend) {
      store_out();
      pend = false;
    }
    if (dw) {
      issue_a();
      issue_b();
    }

    const bool active = cit.m0 + 16 * wm < cit.mm;
    const uint8_t* Bs = ringB + c_sb * B_STAGE;
    if ((c_kt & 1) == 0) {  // first step of a 128-K scale block
      const float ck = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*(const float*)(Bs + BN * BK + 4 * wn))));
      zblk = ck == 0.f;
      if (!zblk) {
        if (active && c_cur != 0.f && c_cur != ck) {
          const float r = c_cur / ck;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if (cit.m0 + 16 * wm + 64 * i >= cit.mm) break;  // masked row groups hold zeros
#pragma unroll
            for (int n = 0; n < NBW; n++)
#pragma unroll
              for (int e = 0; e < 4; e++) acc[i][n][e] *= r;
          }
        }
        c_cur = ck;
      }
    }
    if (active && !zblk) {
      const uint8_t* As = ringA + c_sa * A_STAGE;
      u32x4_t braw[NBW];
#pragma unroll
      for (int n = 0; n < NBW; n++) {
        const int r = WCOLS * wn + 16 * n + rr;
        braw[n] = *(const u32x4_t*)(Bs + r * BK + ((q ^ f2_swz_b(r)) << 4));
      }
#pragma unroll
      for (int ks = 0; ks < BK / 32; ks++) {
        bf16x8_t af[4], bfr[NBW];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (cit.m0 + 16 * wm + 64 * i >= cit.mm) break;
          const int r = 16 * wm + 64 * i + rr;
          af[i] = *(const bf16x8_t*)(As + r * (BK * 2) + (((2 * q + ks) ^ f1_swz(r)) << 4));
        }
#pragma unroll
        for (int n = 0; n < NBW; n++) {
          const uint32_t lo = braw[n][2 * ks], hi = braw[n][2 * ks + 1];
          const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
          const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
          const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
          const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
          bfr[n] = bf16x8_t{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (cit.m0 + 16 * wm + 64 * i >= cit.mm) break;
#pragma unroll
          for (int n = 0; n < NBW; n++)
            acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[n], af[i], acc[i][n], 0, 0, 0);
        }
      }
    }
    c_sa ^= 1;
    c_sb = c_sb + 1 == SB ? 0 : c_sb + 1;

    if (++c_kt == KT) {
      if (active) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (cit.m0 + 16 * wm + 64 * i >= cit.mm) break;
#pragma unroll
          for (int n = 0; n < NBW; n++)
#pragma unroll
            for (int e = 0; e < 4; e++) acc[i][n][e] *= c_cur;
        }
        pend = true;
        pit = cit;
      }
      c_cur = 0.f;
      c_kt = 0;
      if (++c_k < n_items) cit = item_at(c_k);
    }
  }
  if (pend) store_out();
  wait_vmcnt<0>();  // the trailing re-reads land before the workgroup ends
}

template <int NBW, int DB>
static hipError_t launch_bf16_fp8w(const Fp8GemmArgs& p, int cu_limit, hipStream_t s) {
  using namespace f2;
  constexpr int BN = Cfg<NBW>::BN;
  if ((long long)p.G * ((p.max_m + BM - 1) / BM) * (p.N / BN) > 0x7FFFFFFFLL) return hipErrorNotSupported;
  const void* k = (const void*)k_gemm_bf16_fp8w<NBW, DB>;
  const int grid = resident_grid(k, THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_bf16_fp8w<NBW, DB>), dim3(grid), dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t gemm_bf16_fp8w(Fp8GemmArgs p, int cu_limit, hipStream_t s) {
  if (p.G <= 0 || p.max_m <= 0 || p.N <= 0 || p.K <= 0) return hipSuccess;
  if (p.G > f1::MAX_G || p.N % 128 != 0 || p.K % 128 != 0) return hipErrorNotSupported;
  if (p.b_k && (p.b_k % 128 != 0 || (p.K != p.b_k && p.K != 2 * p.b_k))) return hipErrorNotSupported;
  // the DMA offsets (from an expert's base, and of the scales from b_s) are 32-bit
  const unsigned long long wk = p.b_k ? p.b_k : p.K;
  if ((unsigned long long)p.max_m * p.K * 2 >= (1ull << 32) || (unsigned long long)p.N * wk >= (1ull << 32) ||
      4ull * p.G * (p.N / 128) * (wk / 128) >= (1ull << 32))
    return hipErrorNotSupported;
  // 256 columns per item where N allows it (half the h re-reads), else 128
  if (p.N % 256 == 0) return launch_bf16_fp8w<8, 4>(p, cu_limit, s);
  return launch_bf16_fp8w<4, 6>(p, cu_limit, s);
}

}  // namespace mxg
