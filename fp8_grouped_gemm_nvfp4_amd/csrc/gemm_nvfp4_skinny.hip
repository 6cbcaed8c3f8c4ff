// gemm_nvfp4_skinny.hip -- masked grouped NVFP4 NT GEMM for decode-shaped groups
// (at most 16 valid rows per M tile), where the time is the read of the active
// groups' B (expert weights) from HBM.
//
// Same operation as the tiled kernel (masked batched GEMM with scale factors and
// alpha at output, "The CuteDSL Gamble", "The Message"); the decode regime is the
// one the page's single-stream measurements sit in (M = 1 grouped GEMMs,
// "Assumptions Embedded in the Message").
//
// MI355X design:
//  * Weights go from HBM straight into LDS by DMA (global_load_lds_dwordx4, no
//    registers): each wave owns a ring of S LDS stages and keeps S - 1
//    chunks of 512 K-elements in flight ahead of its compute.
//  * Every DMA instruction covers 4 rows x 256 contiguous bytes of codes (the 16 rows'
//    32 scale bytes per chunk take one more): runs long enough for HBM to stream near
//    its peak.  The lane -> 16-byte-unit mapping is XOR-swizzled by row so that the
//    operand reads (16 rows, one unit each) are bank-conflict free.
//  * The ring runs across work units: a workgroup walks the flat (unit, chunk)
//    sequence of its units, so the pipeline never drains between units, and the
//    epilogue reads alpha through the scalar cache instead of a vector load.
//  * Weights are decoded e2m1 x e4m3 into exact fp16 (hardware fp4 and fp8 converts,
//    one packed multiply) and fed to v_mfma_f32_16x16x32_f16.  Inside a chunk, lane
//    group q owns elements j*128 + q*32 .. +32 of each 128-slice j; the activation
//    operand uses the same order.
//  * Activations (<= MR rows, MR = 8 or 16) arrive by DMA too (wave 0, DA - 1 chunks
//    ahead) and are decoded once per chunk by the workgroup into LDS as fp16 (double
//    buffered, one barrier per chunk).
//  * Output tile D[n][m] (weights x activations): lane l holds 4 consecutive n for one
//    m, so stores are 8-byte (bf16) or 16-byte (fp32) vectors.
//  * Fused SwiGLU + NVFP4 requantization (MoE GEMM1): waves 2k and 2k+1 stream the gate
//    rows and the matching up rows (8 waves, one tile each, as for the plain outputs);
//    at a unit's end the up wave hands its tile to the gate wave through LDS, which
//    forms h = silu(gate) * up in registers; the 16-column block amax is two cross-lane
//    shuffles away.  (A wave may also hold both tiles, NT = 2.)
//  * Persistent grid over a compacted list of (group, M tile) entries with valid rows,
//    built in LDS with wavefront ballots: idle groups cost nothing.
#include "device_common.h"
#include "kernels.h"

namespace mxg {

namespace sk {
constexpr int KC = 512;                         // K elements per chunk
constexpr int APITCH = KC + 8;                  // fp16 per LDS activation row
constexpr int CODE_BYTES = 16 * 256;            // codes of one 16-row weight tile chunk
constexpr int TILE_STAGE = CODE_BYTES + 512;    // + the 16 rows' scale bytes
constexpr int MAX_LIST = 512;                   // (group, M tile) entries kept in LDS
}

// Per-lane DMA source offsets of one weight tile: codes of rows 4i + lane/16 with the
// swizzled unit, scales of row lane/2 (lanes < 32 only).  A row's 32 scale bytes land
// with their 16-byte halves swapped for rows 8..15, so that the 4-byte scale reads of
// rows n and n + 8 fall in different banks.
struct TileSrc {
  size_t code[4];
  size_t scale;
};

// With il16 (SwiGLU tiles only, nlimit = I) the logical W13 row is mapped to its place
// in the gate/up-interleaved layout.
__device__ __forceinline__ TileSrc tile_src(int first_row, int nlimit, int row_off, int K, int lane,
                                            bool il16 = false) {
  TileSrc s;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    int r = 4 * i + (lane >> 4);
    int g = first_row + r;
    g = (g < nlimit ? g : nlimit - 1) + row_off;  // rows past the end re-read a valid row (never stored)
    g = w13_row(g, nlimit, il16);
    s.code[i] = (size_t)g * (K / 2) + (size_t)(((lane & 15) ^ r) * 16);
  }
  int r = (lane & 31) >> 1;
  int g = first_row + r;
  g = (g < nlimit ? g : nlimit - 1) + row_off;
  g = w13_row(g, nlimit, il16);
  s.scale = (size_t)g * (K / 16) + (size_t)(((lane & 1) ^ ((r >> 3) & 1)) * 16);
  return s;
}

template <int NT>
__device__ __forceinline__ void dma_w_chunk(uint8_t* stage, const uint8_t* B, const uint8_t* Bsf,
                                            const TileSrc* src, int chunk, int lane) {
#pragma unroll
  for (int t = 0; t < NT; t++) {
    uint8_t* st = stage + t * sk::TILE_STAGE;
#pragma unroll
    for (int i = 0; i < 4; i++) dma16(B + src[t].code[i] + (size_t)chunk * (sk::KC / 2), st + i * 1024);
    if (lane < 32) dma16(Bsf + src[t].scale + (size_t)chunk * (sk::KC / 16), st + sk::CODE_BYTES);
  }
}

// Raw activation chunk in LDS: codes [MR rows][256 B], then scales [MR][32 B].
template <int MR>
struct ARaw {
  static constexpr int BYTES = MR * 256 + MR * 32;
  static constexpr int OPS = MR / 4 + 1;  // DMA instructions per chunk
};

// DMA (by one wave) of the activation chunk of rows [0, MR) starting at A/Asf: code
// instruction i covers rows 4i .. 4i+3; rows past the valid count re-read row 0.
template <int MR>
__device__ __forceinline__ void dma_a_chunk(uint8_t* raw, const uint8_t* A, const uint8_t* Asf, int K,
                                            int rows, int chunk, int lane) {
#pragma unroll
  for (int i = 0; i < MR / 4; i++) {
    int r = 4 * i + (lane >> 4);
    r = r < rows ? r : 0;
    dma16(A + (size_t)r * (K / 2) + (size_t)chunk * (sk::KC / 2) + (lane & 15) * 16, raw + i * 1024);
  }
  int r = lane >> 1;
  r = r < rows ? r : 0;
  if (lane < 2 * MR) dma16(Asf + (size_t)r * (K / 16) + (size_t)chunk * (sk::KC / 16) + (lane & 1) * 16, raw + MR * 256);
}

// Decode a raw activation chunk into the fp16 buffer: thread t owns row t / TPR and EPT
// consecutive elements (threads of padding rows skip).
template <int THREADS, int MR>
__device__ __forceinline__ void decode_a_chunk(_Float16* As, const uint8_t* raw, int rows, int tid) {
  constexpr int TPR = THREADS / MR, EPT = sk::KC / TPR;  // 8, 16 or 32 elements
  static_assert(EPT == 8 || EPT == 16 || EPT == 32, "activation decode split");
  const int r = tid / TPR, seg = tid % TPR;
  if (r >= rows) return;
  half8_t* dst = (half8_t*)(As + r * sk::APITCH + seg * EPT);
  if constexpr (EPT == 32) {
    u32x4_t c = *(const u32x4_t*)(raw + r * 256 + seg * 16);
    uint32_t sc = *(const uint16_t*)(raw + MR * 256 + r * 32 + seg * 2);
    half2_t s0 = scale_e4m3_to_h2(sc & 0xFFu), s1 = scale_e4m3_to_h2(sc >> 8);
    dst[0] = decode8_e2m1_f16(c[0], s0);
    dst[1] = decode8_e2m1_f16(c[1], s0);
    dst[2] = decode8_e2m1_f16(c[2], s1);
    dst[3] = decode8_e2m1_f16(c[3], s1);
  } else if constexpr (EPT == 16) {
    u32x2_t c = *(const u32x2_t*)(raw + r * 256 + seg * 8);
    half2_t s0 = scale_e4m3_to_h2(raw[MR * 256 + r * 32 + seg]);
    dst[0] = decode8_e2m1_f16(c[0], s0);
    dst[1] = decode8_e2m1_f16(c[1], s0);
  } else {
    uint32_t c = *(const uint32_t*)(raw + r * 256 + seg * 4);
    dst[0] = decode8_e2m1_f16(c, scale_e4m3_to_h2(raw[MR * 256 + r * 32 + seg / 2]));
  }
}

// MFMA over one staged chunk.  Lane (n = l%16, q = l/16) reads unit 4j + q of row n (at
// swizzled position (4j+q) ^ n) and the two scale bytes of its elements' 16-blocks.
// Activation lanes of padding rows read the buffer's zero row zrow (their output columns
// are never stored): most decode tiles hold one valid row, and zero operands in the other
// fifteen MFMA columns draw less power than copies of a valid row, which matters once
// back-to-back launches run into the power limit.
template <int NT>
__device__ __forceinline__ void compute_chunk(float4_t (&acc)[NT], const uint8_t* stage, const _Float16* As,
                                              int lane, int rows, int zrow) {
  const int n = lane & 15, q = lane >> 4;
  const int ma = n < rows ? n : zrow;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    u32x4_t w[NT];
    half2_t sc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const uint8_t* st = stage + t * sk::TILE_STAGE;
      w[t] = *(const u32x4_t*)(st + n * 256 + (((4 * j + q) ^ n) * 16));
      // the dword holding this lane's two scale bytes (lanes q and q ^ 1 read the same
      // dword, a broadcast; 2-byte reads of its halves would be served apart)
      const uint32_t sw = *(const uint32_t*)(st + sk::CODE_BYTES + n * 32 + ((((j >> 1) ^ (n >> 3)) & 1) << 4) +
                                             (j & 1) * 8 + (q >> 1) * 4);
      const uint32_t sb = sw >> (16 * (q & 1));
      half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
      sc[t][0] = half2_t{s01[0], s01[0]};
      sc[t][1] = half2_t{s01[1], s01[1]};
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
      half8_t act = *(const half8_t*)(As + ma * sk::APITCH + j * 128 + q * 32 + s * 8);
#pragma unroll
      for (int t = 0; t < NT; t++) {
        half8_t wv = decode8_e2m1_f16(w[t][s], sc[t][s >> 1]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, act, acc[t], 0, 0, 0);
      }
    }
  }
}

// One work unit = (group g, MR-row M tile, N tile).  The workgroup's units are
// blockIdx.x + i * gridDim.x over the compacted list of (g, M tile) entries with valid
// rows times the N tiles.
struct Unit {
  int g, m0, rows, nt;
};

// Prologue shared by the persistent decode kernels: the compacted list of (group, M tile)
// entries with valid rows, built with wavefront ballots by wave 0 and packed as
// g << 7 | mt << 5 | rows (g < 512, mt < 4, rows <= 16), and the groups' alphas, copied
// to LDS so that no epilogue waits on a global or scalar load behind the weight stream.
template <int MR>
__device__ __forceinline__ void build_unit_list(const MaskedGemmArgs& p, uint16_t* list, int* list_n, float* alpha_s,
                                                int tid, int nthreads) {
  const int lane = tid & 63;
  for (int g = tid; g < p.G; g += nthreads) alpha_s[g] = (p.alpha ? p.alpha[g] : 1.0f) * p.alpha_scale;
  if (tid < 64) {
    int count = 0;
    for (int base = 0; base < p.G * p.tiles_m; base += 64) {
      const int idx = base + lane;  // idx = g * tiles_m + mt
      int rows = 0, g = 0, mt = 0;
      if (idx < p.G * p.tiles_m) {
        g = idx / p.tiles_m;
        mt = idx % p.tiles_m;
        int mm = p.masked_m[g];
        mm = mm < 0 ? 0 : (mm > p.max_m ? p.max_m : mm);
        rows = mm - mt * MR;
        rows = rows < 0 ? 0 : (rows > MR ? MR : rows);
      }
      const unsigned long long bal = __ballot(rows > 0);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (rows > 0) list[count + before] = (uint16_t)((g << 7) | (mt << 5) | rows);
      count += __popcll(bal);
    }
    if (lane == 0) *list_n = count;
  }
  __syncthreads();
}

// Walks the units blockIdx.x + i * gridDim.x, i = 0, 1, ... of a workgroup without
// divisions: (q, r) = (u / tiles_n, u % tiles_n) advance by (gridDim.x / tiles_n,
// gridDim.x % tiles_n) per unit.
struct UnitCursor {
  int q, r;
  __device__ __forceinline__ void start(int tiles_n) {
    q = (int)blockIdx.x / tiles_n;
    r = (int)blockIdx.x % tiles_n;
  }
  __device__ __forceinline__ void next(int gq, int gr, int tiles_n) {
    q += gq;
    r += gr;
    if (r >= tiles_n) {
      r -= tiles_n;
      q++;
    }
  }
  template <int MR>
  __device__ __forceinline__ Unit get(const uint16_t* list) const {
    const int e = list[q];
    Unit u;
    u.g = e >> 7;
    u.m0 = ((e >> 5) & 3) * MR;
    u.rows = e & 31;
    u.nt = r;
    return u;
  }
};

// Persistent kernel.  Each workgroup walks the flat sequence of (unit, chunk) steps of
// its units, f = i * nchunks + c, with the DMA ring running across unit boundaries:
// every wave keeps its weight chunks S-1 steps ahead and wave 0 keeps the activation
// chunks DA-1 steps ahead, so the pipeline never drains between units.
template <int MR, int NT, int EPI, int WAVES, int S, int DA>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_nvfp4_skinny(const MaskedGemmArgs p) {
  constexpr bool SWIGLU = (EPI == EPI_SWIGLU_NVFP4);
  // SwiGLU pairs a gate tile with the matching up tile: in one wave (NT = 2), or in the
  // waves 2k (gate) and 2k+1 (up) with one tile each (NT = 1, PAIRED)
  constexpr bool PAIRED = SWIGLU && NT == 1;
  constexpr int THREADS = WAVES * 64;
  static_assert(!SWIGLU || NT == 2 || (NT == 1 && WAVES % 2 == 0), "SwiGLU tile pairing");
  static_assert(!PAIRED || WAVES / 2 * 64 * 16 <= MR * sk::APITCH * 2, "exchange fits an activation buffer");
  static_assert(S >= DA - 1 && DA >= 3, "prefetch distances");
  constexpr int W_OPS = 5 * NT, A_OPS = ARaw<MR>::OPS;
  // vmcnt allowances (ops that may stay outstanding): see the issue order below
  constexpr int WAIT_W = (S - 1) * W_OPS;
  constexpr int WAIT_0a = (S - 1) * W_OPS + A_OPS;              // weights chunk f (first step is the tightest)
  constexpr int WAIT_0b = W_OPS + (DA - 2) * (A_OPS + W_OPS);   // activation chunk f+1
  constexpr int WAIT_0 = WAIT_0a < WAIT_0b ? WAIT_0a : WAIT_0b;
  constexpr int WAIT_PRO = (DA - 2) * A_OPS + (S - 1) * W_OPS;  // activation chunk 0 in the prologue

  __shared__ __attribute__((aligned(16))) _Float16 As[2][(MR + 1) * sk::APITCH];  // row MR: zeros
  __shared__ __attribute__((aligned(16))) uint8_t Araw[DA][ARaw<MR>::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Bst[WAVES][S][NT * sk::TILE_STAGE];
  __shared__ uint16_t list[sk::MAX_LIST];
  __shared__ float alpha_s[sk::MAX_LIST];
  __shared__ int list_n;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int q = lane >> 4;
  const int K = p.K, nchunks = K / sk::KC;
  const int tiles_n = p.tiles_n;

  for (int i = tid; i < 2 * (sk::APITCH / 8); i += THREADS)  // the zero rows (never written again)
    *(half8_t*)(&As[i / (sk::APITCH / 8)][MR * sk::APITCH + (i % (sk::APITCH / 8)) * 8]) = half8_t{};
  build_unit_list<MR>(p, list, &list_n, alpha_s, tid, THREADS);
  const int total = list_n * tiles_n;
  if ((int)blockIdx.x >= total) return;  // uniform over the workgroup
  const int nu = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int F = nu * nchunks;

  const int gq = (int)gridDim.x / tiles_n, gr = (int)gridDim.x % tiles_n;
  auto ncol0_of = [&](int nt) {
    if constexpr (PAIRED) return nt * (16 * (WAVES / 2)) + (wave >> 1) * 16;
    return SWIGLU ? nt * (16 * WAVES) + wave * 16 : nt * (16 * NT * WAVES) + wave * (16 * NT);
  };
  auto weight_src = [&](const Unit& un, TileSrc (&src)[NT]) {
    const int c0 = ncol0_of(un.nt);
    if constexpr (PAIRED) {
      const int I = p.N / 2;
      src[0] = tile_src(c0, I, (wave & 1) ? I : 0, K, lane, p.w13_il16 != 0);
    } else if constexpr (SWIGLU) {
      const int I = p.N / 2;
      src[0] = tile_src(c0, I, 0, K, lane, p.w13_il16 != 0);
      src[1] = tile_src(c0, I, I, K, lane, p.w13_il16 != 0);
    } else {
#pragma unroll
      for (int t = 0; t < NT; t++) src[t] = tile_src(c0 + 16 * t, p.N, 0, K, lane);
    }
  };

  // issue cursors: weights (this wave) and activations (wave 0); steps past the end
  // repeat the last chunk (an L2 re-read) so that every step issues the same ops
  int wc = 0;  // weight cursor chunk
  UnitCursor wcur;
  wcur.start(tiles_n);
  Unit wu = wcur.get<MR>(list);
  TileSrc src[NT];
  weight_src(wu, src);
  const uint8_t* wB = p.b + (size_t)wu.g * p.N * (K / 2);
  const uint8_t* wBsf = p.b_sf + (size_t)wu.g * p.N * (K / 16);
  int wf = 0;
  auto issue_w = [&]() {
    dma_w_chunk<NT>(&Bst[wave][wf % S][0], wB, wBsf, src, wc, lane);
    wf++;
    if (wf < F) {
      if (++wc == nchunks) {
        wc = 0;
        wcur.next(gq, gr, tiles_n);
        wu = wcur.get<MR>(list);
        weight_src(wu, src);
        wB = p.b + (size_t)wu.g * p.N * (K / 2);
        wBsf = p.b_sf + (size_t)wu.g * p.N * (K / 16);
      }
    }
  };
  int ac = 0, af = 0;
  UnitCursor acur;
  acur.start(tiles_n);
  Unit au = acur.get<MR>(list);
  auto issue_a = [&]() {
    const uint8_t* A = p.a + ((size_t)au.g * p.max_m + au.m0) * (K / 2);
    const uint8_t* Asf = p.a_sf + ((size_t)au.g * p.max_m + au.m0) * (K / 16);
    dma_a_chunk<MR>(&Araw[af % DA][0], A, Asf, K, au.rows, ac, lane);
    af++;
    if (af < F) {
      if (++ac == nchunks) {
        ac = 0;
        acur.next(gq, gr, tiles_n);
        au = acur.get<MR>(list);
      }
    }
  };

  // prologue: activation chunks 0 .. DA-2, weight chunks 0 .. S-2
  if (wave == 0)
    for (int k = 0; k < DA - 1; k++) issue_a();
  for (int k = 0; k < S - 1; k++) issue_w();
  if (wave == 0) wait_vmcnt<WAIT_PRO>();
  __syncthreads();
  int dc = 0;  // decode cursor
  UnitCursor dcur;
  dcur.start(tiles_n);
  Unit du = dcur.get<MR>(list);
  decode_a_chunk<THREADS, MR>(As[0], Araw[0], du.rows, tid);

  int cc = 0;  // compute cursor
  UnitCursor ccur;
  ccur.start(tiles_n);
  Unit cu = ccur.get<MR>(list);
  float4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; t++) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int f = 0; f < F; f++) {
    // Issue order of step f: wave 0 activation chunk f+DA-1, then each wave its weight
    // chunk f+S-1.  Then wait until this wave's weight chunk f (and, for wave 0, the
    // activation chunk f+1 decoded at the end of this step) has landed.
    if (wave == 0) issue_a();
    issue_w();
    if (wave == 0) wait_vmcnt<WAIT_0>();
    else wait_vmcnt<WAIT_W>();
    // After this barrier every wave has finished step f-1 (activation buffer (f+1)&1
    // and the raw stage of chunk f+DA may be rewritten), activation buffer f&1 is
    // complete and activation chunk f+1 is in LDS.
    __syncthreads();
    compute_chunk<NT>(acc, &Bst[wave][f % S][0], As[f & 1], lane, cu.rows, MR);

    if (cc == nchunks - 1) {
      // epilogue of the unit
      const int m = lane & 15;
      const int ncol0 = ncol0_of(cu.nt);
      const size_t orow = (size_t)cu.g * p.max_m + cu.m0 + m;
      const float alpha = alpha_s[cu.g];
      if constexpr (EPI == EPI_BF16 || EPI == EPI_F32) {
#pragma unroll
        for (int i = 0; i < NT; i++) {
          const int n = ncol0 + i * 16 + q * 4;
          if (m < cu.rows && n < p.N) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; r++) v[r] = alpha * acc[i][r];
            if (n + 4 <= p.N && (p.N & 3) == 0) {
              if constexpr (EPI == EPI_BF16) {
                uint32_t lo = bf16x2_rne(v[0], v[1]);
                uint32_t hi = bf16x2_rne(v[2], v[3]);
                *(u32x2_t*)((uint16_t*)p.out + orow * p.N + n) = u32x2_t{lo, hi};
              } else {
                *(float4_t*)((float*)p.out + orow * p.N + n) = float4_t{v[0], v[1], v[2], v[3]};
              }
            } else {
              for (int r = 0; r < 4 && n + r < p.N; r++) {
                if constexpr (EPI == EPI_BF16) ((uint16_t*)p.out)[orow * p.N + n + r] = (uint16_t)f32_to_bf16_rne(v[r]);
                else ((float*)p.out)[orow * p.N + n + r] = v[r];
              }
            }
          }
        }
      } else {
        const int I = p.N / 2;
        float4_t upv;
        if constexpr (PAIRED) {
          // The up wave hands its tile to the gate wave through activation buffer (f+1)&1:
          // its readers (step f-1) are past this step's barrier, and it is rewritten only
          // by the decode at the end of this step, after a second barrier.
          float4_t* xchg = (float4_t*)As[(f + 1) & 1];
          if (wave & 1) xchg[(wave >> 1) * 64 + lane] = acc[0];
          __syncthreads();
          upv = xchg[(wave >> 1) * 64 + lane];
        } else {
          upv = acc[1];
        }
        float h[4], gv[4], uv[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          float gt = alpha * acc[0][r], up = alpha * upv[r];
          gv[r] = gt;
          uv[r] = up;
          h[r] = gt / (1.0f + expf(-gt)) * up;
        }
        const int hc = ncol0 + q * 4;  // this lane's first h column
        if (p.dbg_h && m < cu.rows && hc < I && !(PAIRED && (wave & 1)))
          *(float4_t*)(p.dbg_h + orow * I + hc) = float4_t{h[0], h[1], h[2], h[3]};
        if (p.dbg_g1 && m < cu.rows && hc < I && !(PAIRED && (wave & 1))) {
          *(float4_t*)(p.dbg_g1 + orow * 2 * I + hc) = float4_t{gv[0], gv[1], gv[2], gv[3]};
          *(float4_t*)(p.dbg_g1 + orow * 2 * I + I + hc) = float4_t{uv[0], uv[1], uv[2], uv[3]};
        }
        uint32_t sbyte;
        uint32_t bits = quantize_block_x4(h, p.g_h, 6.0f * p.g_h, sbyte);
        uint32_t b1 = __shfl_xor(bits, 16);  // q ^ 1
        uint32_t b2 = __shfl_xor(bits, 32);  // q ^ 2
        uint32_t b3 = __shfl_xor(bits, 48);  // q ^ 3
        if (q == 0 && m < cu.rows && ncol0 < I && !(PAIRED && (wave & 1))) {
          uint32_t w0 = bits | (b1 << 16), w1 = b2 | (b3 << 16);
          *(u32x2_t*)(p.h_codes + orow * (I / 2) + ncol0 / 2) = u32x2_t{w0, w1};
          p.h_sf[orow * (I / 16) + ncol0 / 16] = (uint8_t)sbyte;
        }
        if constexpr (PAIRED) __syncthreads();  // the exchange is read before the decode below
      }
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (++cc == nchunks && f + 1 < F) {
      cc = 0;
      ccur.next(gq, gr, tiles_n);
      cu = ccur.get<MR>(list);
    }

    // decode activation chunk f+1 (its unit may be the next one)
    if (f + 1 < F) {
      if (++dc == nchunks) {
        dc = 0;
        dcur.next(gq, gr, tiles_n);
        du = dcur.get<MR>(list);
      }
      decode_a_chunk<THREADS, MR>(As[(f + 1) & 1], Araw[(f + 1) % DA], du.rows, tid);
    }
  }
  wait_vmcnt<0>();  // the trailing re-reads land before the waves end
}

int resident_grid(const void* kernel, int threads, int cu_limit) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  if (per_cu < 1) per_cu = 1;
  if (cu_limit > 0 && cu_limit < cus) cus = cu_limit;
  return cus * per_cu;
}

template <int MR, int NT, int EPI, int WAVES, int S, int DA>
static hipError_t launch_skinny(MaskedGemmArgs p, int cu_limit, hipStream_t s) {
  p.tiles_m = (p.max_m + MR - 1) / MR;
  if (p.G * p.tiles_m > sk::MAX_LIST || p.tiles_m > 4) return hipErrorNotSupported;
  constexpr int HCOLS = NT == 2 ? 16 * WAVES : 16 * (WAVES / 2);  // h columns per SwiGLU unit
  p.tiles_n = (EPI == EPI_SWIGLU_NVFP4) ? (p.N / 2 + HCOLS - 1) / HCOLS
                                        : (p.N + 16 * NT * WAVES - 1) / (16 * NT * WAVES);
  p.total_tiles = p.G * p.tiles_m * p.tiles_n;
  if (p.total_tiles == 0) return hipSuccess;
  const void* k = (const void*)k_gemm_nvfp4_skinny<MR, NT, EPI, WAVES, S, DA>;
  int grid = resident_grid(k, WAVES * 64, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;
  if (grid > p.total_tiles) grid = p.total_tiles;
  hipLaunchKernelGGL((k_gemm_nvfp4_skinny<MR, NT, EPI, WAVES, S, DA>), dim3(grid), dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

// Returns hipErrorNotSupported (nothing launched) for shapes the kernel does not take.
hipError_t gemm_nvfp4_skinny(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s) {
  if (p.max_m > SKINNY_MAX_M || p.K % sk::KC != 0) return hipErrorNotSupported;
  const bool small = p.max_m <= 8 || (p.sparse_rows && p.max_m <= 16);
  switch (epi) {
    case EPI_BF16:
      return small ? launch_skinny<8, 1, EPI_BF16, 8, 3, 4>(p, cu_limit, s) : launch_skinny<16, 1, EPI_BF16, 8, 3, 3>(p, cu_limit, s);
    case EPI_F32:
      return small ? launch_skinny<8, 1, EPI_F32, 8, 3, 4>(p, cu_limit, s) : launch_skinny<16, 1, EPI_F32, 8, 3, 3>(p, cu_limit, s);
    case EPI_SWIGLU_NVFP4:
      return small ? launch_skinny<8, 1, EPI_SWIGLU_NVFP4, 8, 3, 4>(p, cu_limit, s)
                   : launch_skinny<16, 1, EPI_SWIGLU_NVFP4, 8, 3, 3>(p, cu_limit, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mxg
