// gemm_nvfp4_stream.hip -- masked grouped NT GEMM over NVFP4 operands for groups with
// more rows than the decode kernel takes (MoE prefill), persistent and weight-streaming.
//
// Operation ("The CuteDSL Gamble", "The Message"; the MoE GEMM1 / GEMM2 of the
// "llm-assisted-kernel-dev" README's NVFP4 rows):
//   C[g, m, n] = alpha_g * sum_k dec(A)[g, m, k] * dec(B)[g, n, k],  m < masked_m[g],
// dec(X) = e2m1(code) * e4m3(scale of the 16-element block); with the SwiGLU epilogue
// h = silu(gate) * up is requantized to NVFP4 with the fixed global scale g_h.
//
// Work distribution as in stream_common.h: an item is (group, 256-row M tile, 128
// output columns or 64 gate + 64 up columns), so every weight panel is read from HBM
// once per group whenever masked_m <= 256.  One step is 128 K: per row 64 code bytes
// and 8 scale bytes.  Everything arrives by LDS DMA: the activation codes and scales
// one step ahead, the weight codes and scales DB steps ahead.
//
// LDS layouts follow how gfx950 serves 16-byte accesses (measured with the bank-conflict
// counters): a read is served in four passes of 16 lanes, a pass being the lanes with the
// same lane bit 5 and the same parity of lane bits 2..4, and is conflict-free when the
// lanes of a pass hit 16 different 16-byte slots of the 256-byte bank row; a write is
// served 8 consecutive lanes at a time over 128 bytes.  Activation code rows (64 bytes)
// have their 16-byte chunks XOR-permuted by 2 * (row bit 3); weight code rows are plain
// (the decode reads them 4 rows x 64 bytes per pass); the decoded fp16 weight rows (256
// bytes) hold K chunk c at slot c ^ sigma(r), sigma flipping row bit 3 with row bit 2.
//
// Compute: decoding is exact (e2m1 * e4m3 fits fp16; fp16 products are exact in fp32).
// The weight step is decoded once per workgroup into an fp16 LDS tile, one step ahead;
// for the activations each lane reads one 16-byte chunk (32 codes, two 16-blocks) per
// row and step and decodes it in registers, 8 elements per 16x16x32 fp16 MFMA.  The K
// order inside a step is permuted identically for both operands, which only reorders
// the fp32 sum.  The MFMA computes the transposed tile D = B A^T, so each lane ends
// with four consecutive output columns of one row: 16-byte fp32 stores, and the
// 16-column NVFP4 blocks of the SwiGLU epilogue sit in 4 lanes (quantize_block_x4).
// Waves: the two roles are split.  Waves 4..7 (one per SIMD; waves w and w + 4 share a
// SIMD) issue every DMA and decode the next weight step; waves 0..3 only read
// fragments, decode their activation rows and run MFMAs, each on a 64-row x 128-column
// register tile (wave c owns the 16-row groups 16 c + 64 i, so all four compute when
// masked_m > 48).  One barrier per step hands a step's buffers from one role to the
// other.  The MFMA waves cross it pipelined: the operands of their last sub-step are in
// registers before it, and the next step's fragment reads and first activation decode go
// out under that sub-step's MFMAs; each sub-step likewise decodes the next one's
// activation rows between its MFMAs.  Each item runs a loop specialised on the wave's
// valid row groups, so the MFMA stream has no branches; the loop keeps its pipeline
// state to itself (nothing crosses from one specialisation to another), which keeps the
// kernel free of register spills.
#include <type_traits>

#include "kernels.h"
#include "stream_common.h"

namespace mxg {

namespace ns {
constexpr int BM = STREAM_BM, BN = 128, BK = 128;
constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int CW = 4;                                       // MFMA waves; waves CW .. 7 move data
constexpr int RG = BM / 16 / CW;                            // 16-row groups per MFMA wave
constexpr int NB = BN / 16;                                 // 16-column groups per MFMA wave
constexpr int A_CODE = BM * 64, A_STAGE = A_CODE + BM * 8;  // codes [256][64], scales [256][8]
constexpr int B_CODE = BN * 64, B_STAGE = B_CODE + BN * 8;  // codes [128][64], scales [128][8]
constexpr int DB = 3;                                       // weight steps in flight
constexpr int SB = DB;                                      // raw weight stages
constexpr int B_DMAS = 3;                                   // weight DMAs of one data wave per step
}  // namespace ns

__device__ __forceinline__ int ns_swz_a(int r) { return (r >> 2) & 2; }          // activation code rows
__device__ __forceinline__ int ns_sigma(int r) { return (r & 15) ^ ((r & 4) << 1); }  // decoded weight rows

// Operands of one work item: the group's code / scale bases (row 0), the tile origin,
// the group's valid rows and its depth.
struct NsJob {
  const uint8_t *a, *a_sf, *b, *b_sf;
  int g, m0, mm, n0, K;
};

template <int EPI, int MODE>
__global__ __launch_bounds__(ns::THREADS) void k_gemm_nvfp4_stream(const typename ArgsOf<MODE>::type p) {
  using namespace ns;
  constexpr bool SWIGLU = (EPI == EPI_SWIGLU_NVFP4);
  // the contiguous layout is the masked one with each group's rows starting at row_start[g]
  constexpr bool CONTIG = (MODE == MODE_CONTIG);
  constexpr bool MASKED = (MODE == MODE_MASKED) || CONTIG;
  constexpr int MAXG = CONTIG ? STREAM_CONTIG_MAX_G : STREAM_MAX_G;
  static_assert(MASKED || !SWIGLU, "the SwiGLU epilogue is the MoE GEMM1's (masked)");
  static_assert(DB >= 3, "B(s + 1) must be issued before A(s)");
  __shared__ __attribute__((aligned(16))) uint8_t ringA[2 * A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ringB[SB * B_STAGE];
  __shared__ __attribute__((aligned(16))) _Float16 bdec[2][BN * BK];
  __shared__ int tprefix[MAXG + 1];
  __shared__ int mm_s[MAXG];
  __shared__ float alpha_s[MAXG];
  __shared__ int rs_s[CONTIG ? MAXG + 1 : 1];  // group row starts, clamped to [0, max_m] and non-decreasing

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int G = p.G;
  int N = 0, cap = 0, tiles_n = 0, total = 0;  // masked: common N, row capacity, N tiles
  const int ncols = SWIGLU ? BN / 2 : BN;      // output (h) columns per item
  if constexpr (MASKED) {
    N = p.N;
    cap = p.max_m;
    tiles_n = SWIGLU ? (N / 2) / ncols : N / ncols;
    for (int g = tid; g < G; g += THREADS) alpha_s[g] = (p.alpha ? p.alpha[g] : 1.0f) * p.alpha_scale;
    if constexpr (CONTIG) {
      // starts clamped to [0, max_m] and made non-decreasing (a running maximum, by wave
      // 0's shuffle scan), so every access stays inside the max_m rows whatever they hold
      for (int g = tid; g <= G; g += THREADS) {
        const int v = p.row_start[g];
        rs_s[g] = v < 0 ? 0 : (v > cap ? cap : v);
      }
      __syncthreads();
      if (tid < 64) {
        int run = 0;
        for (int base = 0; base <= G; base += 64) {
          const int g = base + tid;
          int x = g <= G ? rs_s[g] : 0;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (tid >= d) x = x > y ? x : y;
          }
          x = x > run ? x : run;
          if (g <= G) rs_s[g] = x;
          run = __shfl(x, 63);
        }
      }
      __syncthreads();
      stream_tile_prefix(p.masked_m, G, cap, tprefix, mm_s, tid, SWIGLU || p.K >= 4096, rs_s);
    } else {
      stream_tile_prefix(p.masked_m, G, cap, tprefix, mm_s, tid, SWIGLU || p.K >= 4096);
    }
    total = __builtin_amdgcn_readfirstlane(tprefix[G]) * tiles_n;
  }
  const int I = N / 2;
  const int grid = gridDim.x;
  const int bx = stream_bx();
  // heterogeneous groups with a schedule: tprefix[g] / mm_s[g] hold this workgroup's item
  // count and first local item of group g (consecutive items); without one, tprefix counts
  // the items (M tiles x N tiles) per group for the round-robin deal
  bool sched = false;
  if constexpr (!MASKED) {
    const HeteroSchedule& sc = p.sched;
    sched = sc.npat > 0;
    if (sched) {
      if (tid < G) {
        const int g = tid;
        int pp = 0, base = 0;
        while (pp + 1 < sc.npat && sc.pat_start[pp + 1] <= bx) pp++;
        for (int t = 0; t < pp; t++) base += (sc.pat_start[t + 1] - sc.pat_start[t]) * sc.pat_cnt[t][g];
        const int cnt = bx < sc.pat_start[sc.npat] ? sc.pat_cnt[pp][g] : 0;
        tprefix[g] = cnt;
        mm_s[g] = base + (bx - sc.pat_start[pp]) * cnt;
      }
    } else if (tid == 0) {
      int run = 0;
      for (int g = 0; g < G; g++) {
        tprefix[g] = run;
        run += (p.grp[g].M + BM - 1) / BM * (p.grp[g].N / BN);
      }
      tprefix[G] = run;
    }
    __syncthreads();
    if (!sched) total = __builtin_amdgcn_readfirstlane(tprefix[G]);
  }
  int n_items = 0;
  if (sched) {
    for (int g = 0; g < G; g++) n_items += __builtin_amdgcn_readfirstlane(tprefix[g]);
    if (n_items == 0) return;
  } else {
    if (bx >= total) return;
    n_items = (total - 1 - bx) / grid + 1;
  }

  auto job_at = [&](int k) {
    NsJob j;
    if constexpr (MASKED) {
      const StreamItem it = stream_item(bx + k * grid, tiles_n, G, tprefix, mm_s, ncols, SWIGLU || p.K >= 4096);
      j.g = it.g; j.m0 = it.m0; j.mm = it.mm; j.n0 = it.n0; j.K = p.K;
      const size_t r0 = CONTIG ? (size_t)__builtin_amdgcn_readfirstlane(rs_s[it.g]) : (size_t)it.g * cap;
      j.a = p.a + r0 * (p.K / 2);
      j.a_sf = p.a_sf + r0 * (p.K / 16);
      j.b = p.b + (size_t)it.g * N * (p.K / 2);
      j.b_sf = p.b_sf + (size_t)it.g * N * (p.K / 16);
    } else {
      int lo = 0, local = 0;
      if (sched) {  // this workgroup's k-th item: groups in order, consecutive items of each
        for (; lo < G; lo++) {
          const int c = __builtin_amdgcn_readfirstlane(tprefix[lo]);
          if (k < c) break;
          k -= c;
        }
        if (lo == G) lo = G - 1, k = 0;  // past the last item (not reached)
        local = __builtin_amdgcn_readfirstlane(mm_s[lo]) + k;
      } else {
        const int w = bx + k * grid;
        int hi = G;  // tprefix[lo] <= w < tprefix[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (__builtin_amdgcn_readfirstlane(tprefix[mid]) <= w) lo = mid;
          else hi = mid;
        }
        local = w - __builtin_amdgcn_readfirstlane(tprefix[lo]);
      }
      const HeteroGroup& q = p.grp[lo];
      const int tn = q.N / BN;
      const int mt = local / tn;
      j.g = lo; j.m0 = mt * BM; j.mm = q.M; j.n0 = (local - mt * tn) * BN; j.K = q.K;
      j.a = q.a; j.a_sf = q.a_sf; j.b = q.b; j.b_sf = q.b_sf;
    }
    return j;
  };
  int nsteps = 0;
  if constexpr (MASKED) nsteps = n_items * (p.K / BK);
  else
    for (int k = 0; k < n_items; k++) nsteps += job_at(k).K / BK;

  if (wave >= CW) {
    // ======== data waves: every DMA, and the weight decode one step ahead ========
    const int pw = wave - CW;
    // B row r of an item (stage row): SwiGLU rows [0, 64) are gate rows n0 + r, [64, 128)
    // the matching up rows I + n0 + r - 64
    auto b_row = [&](const NsJob& it, int r) {
      if constexpr (SWIGLU) return w13_row(r < BN / 2 ? it.n0 + r : I + it.n0 + (r - BN / 2), I, p.w13_il16 != 0);
      else return it.n0 + r;
    };
    // data wave pw moves activation rows [64 pw, 64 pw + 64) and weight rows [32 pw,
    // 32 pw + 32) of each step.  Rows past masked_m re-read the last valid row and are
    // never stored; 16-row code groups and 32-row scale groups entirely past it are not
    // fetched.
    const uint8_t* asrc[4];
    const uint8_t* asrc_s[2];
    int a_n = 0, a_ns = 0, a_KT = 0;
    auto a_setup = [&](const NsJob& it) {
      const int K = it.K;
      a_KT = K / BK;
      const int left = it.mm - it.m0 - 64 * pw;
      a_n = left <= 0 ? 0 : (left >= 64 ? 4 : (left + 15) >> 4);
      a_ns = left <= 0 ? 0 : (left > 32 ? 2 : 1);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int r = 64 * pw + 16 * j + (lane >> 2);
        const int row = it.m0 + r < it.mm ? it.m0 + r : it.mm - 1;
        asrc[j] = it.a + (size_t)row * (K / 2) + (((lane & 3) ^ ns_swz_a(r)) << 4);
      }
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int r = 64 * pw + 32 * j + (lane >> 1);
        const int row = it.m0 + r < it.mm ? it.m0 + r : it.mm - 1;
        asrc_s[j] = it.a_sf + (size_t)row * (K / 16) + (lane & 1) * 4;
      }
    };
    const uint8_t* bsrc[2];
    const uint8_t* bsrc_s;
    int b_KT = 0;
    auto b_setup = [&](const NsJob& it) {
      const int K = it.K;
      b_KT = K / BK;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int r = 32 * pw + 16 * j + (lane >> 2);
        bsrc[j] = it.b + (size_t)b_row(it, r) * (K / 2) + ((lane & 3) << 4);
      }
      bsrc_s = it.b_sf + (size_t)b_row(it, 32 * pw + (lane >> 1)) * (K / 16) + (lane & 1) * 4;
    };
    int a_k = 0, a_kt = 0, a_step = 0, a_st = 0;
    int b_k = 0, b_kt = 0, b_step = 0, b_st = 0;
    // A(step) into slot step & 1; past the last step the cursor stays and re-reads it
    auto issue_a = [&]() {
      uint8_t* st = ringA + a_st * A_STAGE;
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (j < a_n) dma16(asrc[j] + a_kt * (BK / 2), st + (64 * pw + 16 * j) * 64);
#pragma unroll
      for (int j = 0; j < 2; j++)
        if (j < a_ns) dma4(asrc_s[j] + a_kt * (BK / 16), st + A_CODE + (64 * pw + 32 * j) * 8);
      a_st ^= 1;
      if (a_step + 1 < nsteps) {
        a_step++;
        if (++a_kt == a_KT) {
          a_kt = 0;
          a_setup(job_at(++a_k));
        }
      }
    };
    // B(step) into stage step % SB: always B_DMAS instructions
    auto issue_b = [&]() {
      uint8_t* st = ringB + b_st * B_STAGE;
#pragma unroll
      for (int j = 0; j < 2; j++) dma16(bsrc[j] + b_kt * (BK / 2), st + (32 * pw + 16 * j) * 64);
      dma4(bsrc_s + b_kt * (BK / 16), st + B_CODE + 32 * pw * 8);
      b_st = b_st + 1 == SB ? 0 : b_st + 1;
      if (b_step + 1 < nsteps) {
        b_step++;
        if (++b_kt == b_KT) {
          b_kt = 0;
          b_setup(job_at(++b_k));
        }
      }
    };
    // Weight step decode into fp16: data wave pw takes rows 32 pw .. 32 pw + 31 in two
    // passes of 16; lane l takes row 16 t + (l & 7) + 8 (l >> 5) of pass t and 16-byte
    // code chunk cq = (l >> 3) & 3, so that 8 consecutive lanes write 8 rows of one chunk
    // column; row r's fp16 chunk c (K 8c .. 8c + 7 in the permuted order of the
    // activation side) sits at slot c ^ sigma(r).
    int d_st = 0;  // raw stage of the next weight step to decode
    auto decode_b = [&](int buf) {
      const uint8_t* st = ringB + d_st * B_STAGE;
      const int cq = (lane >> 3) & 3;
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int r = 32 * pw + 16 * t + (lane & 7) + 8 * (lane >> 5);
        const u32x4_t raw = *(const u32x4_t*)(st + r * 64 + (cq << 4));
        const uint32_t sb = *(const uint16_t*)(st + B_CODE + r * 8 + 2 * cq);
        const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
        const half2_t s0 = half2_t{s01[0], s01[0]}, s1 = half2_t{s01[1], s01[1]};
        _Float16* row = bdec[buf] + r * BK;
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
          *(half8_t*)(row + (((4 * cq + ks) ^ ns_sigma(r)) << 3)) = decode8_e2m1_f16(raw[ks], ks < 2 ? s0 : s1);
      }
      d_st = d_st + 1 == SB ? 0 : d_st + 1;
    };

    {
      const NsJob it0 = job_at(0);
      a_setup(it0);
      b_setup(it0);
    }
#pragma unroll
    for (int i = 0; i < DB; i++) issue_b();
    issue_a();
    wait_vmcnt<0>();
    __syncthreads();  // B(0 .. DB - 1) and A(0) are in LDS
    decode_b(0);
    for (int s = 0; s < nsteps; s++) {
      // A(s) and everything issued before it (B(s + 1) among them) have landed; only the
      // weight DMAs of B(s + DB - 1) may be outstanding
      wait_vmcnt<B_DMAS>();
      // every wave is done with step s - 1, whose activation slot and fp16 buffer the
      // next issues and decode overwrite; the decode of B(s) is visible
      __syncthreads();
      issue_a();                // A(s + 1)
      issue_b();                // B(s + DB), into the stage of B(s), decoded during step s - 1
      decode_b((s + 1) & 1);    // B(s + 1); past the end a stage that is not read again
    }
    __syncthreads();  // the MFMA waves' barrier after their last step
    wait_vmcnt<0>();  // the trailing re-reads land before the workgroup ends
    return;
  }

  // ======== MFMA waves: fragments, activation decode, MFMAs and the epilogue ========
  // Wave c owns the 16-row groups 16 c + 64 i (i < RG) of the M tile and all 128 columns,
  // so every MFMA wave computes whenever masked_m > 16 c.  Each item runs a loop
  // specialised on the wave's valid row groups (branch-free, its accumulators local to
  // it).  The step loop is pipelined across the barrier: the operands of sub-step 3 are
  // in registers before it, and after it the loads of the next step's fragments go out
  // under sub-step 3's MFMAs.
  const int c = wave;
  const int q = lane >> 4, rr = lane & 15;
  __syncthreads();  // the data waves' prologue

  // valid 16-row groups of this wave in an item
  auto nv_of = [&](const NsJob& it) {
    const int left = it.mm - it.m0 - 16 * c;
    return left <= 0 ? 0 : (left > 64 * (RG - 1) ? RG : (left + 63) >> 6);
  };
  // dword ks of a lane's chunk q holds K elements 32 q + 8 ks .. +7 of the step, in
  // 16-block 2 q + ks / 2
  // fp16 weight fragment n of sub-step ks: row 16 n + rr, chunk (4 q + ks) ^ sigma(rr) =
  // ((4 q) ^ sigma(rr)) ^ ks, i.e. the lane's byte offset for sub-step 0 with ks XORed
  // into bits 4..5.  The base is re-derived every step (an opaque copy), so the compiler
  // does not keep four offsets live across the loop.
  const int bf_lane = rr * (BK * 2) + (((4 * q) ^ ns_sigma(rr)) << 4);
  int bf_off = bf_lane;
  auto load_bf = [&](half8_t* bf, int s, int n, int ks) {
    const uint8_t* base = (const uint8_t*)bdec[s & 1] + 16 * n * (BK * 2);
    bf[n] = *(const half8_t*)(base + (bf_off ^ (ks << 4)));
  };
  // all RG row groups, valid or not (rows without valid data are never used); row
  // 16 c + 64 i + rr has the swizzle of rr, so the groups sit at fixed offsets
  const int a_off = (16 * c + rr) * 64 + ((q ^ ns_swz_a(rr)) << 4);
  const int as_off = A_CODE + (16 * c + rr) * 8 + 2 * q;
  auto load_a = [&](u32x4_t* araw, uint32_t* asc, int s) {
    const uint8_t* As = ringA + (s & 1) * A_STAGE;
#pragma unroll
    for (int i = 0; i < RG; i++) {
      araw[i] = *(const u32x4_t*)(As + a_off + 64 * 64 * i);
      asc[i] = *(const uint16_t*)(As + as_off + 64 * 8 * i);
    }
  };

  NsJob cit = job_at(0);
  int nv = nv_of(cit);
  int s = 0;  // global step
  __syncthreads();  // top of step 0

  for (int k = 0; k < n_items; k++) {
    const int ksteps = cit.K / BK;
    const NsJob nit = k + 1 < n_items ? job_at(k + 1) : cit;
    auto item = [&](auto nvc) {
      constexpr int NV = decltype(nvc)::value;
      constexpr int NA = NV > 0 ? NV : 1;
      // The pipeline state is the item's own: the barrier of its first step has been
      // passed (before step 0, or inside the previous item's last step), and that step's
      // buffers stay until this wave reaches the next barrier, so its fragments are read
      // again here rather than carried over from the previous item's last sub-step.
      half8_t bf[NB];
      u32x4_t araw[RG];
      uint32_t asc[RG];
      bf_off = bf_lane;
      asm volatile("" : "+v"(bf_off));
#pragma unroll
      for (int n = 0; n < NB; n++) load_bf(bf, s, n, 0);
      load_a(araw, asc, s);
      float4_t acc[NA][NB];
#pragma unroll
      for (int i = 0; i < NA; i++)
#pragma unroll
        for (int n = 0; n < NB; n++) acc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
      half2_t as2[NA][2];
      half8_t af[NA];
      auto cvt_scales = [&]() {
#pragma unroll
        for (int i = 0; i < NV; i++) {
          const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(asc[i], 1.0f, false);
          as2[i][0] = half2_t{s01[0], s01[0]};
          as2[i][1] = half2_t{s01[1], s01[1]};
        }
      };
      cvt_scales();
#pragma unroll
      for (int i = 0; i < NV; i++) af[i] = decode8_e2m1_f16(araw[i][0], as2[i][0]);
      for (int t = 0; t < ksteps; t++, s++) {
        bf_off = bf_lane;
        asm volatile("" : "+v"(bf_off));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 3; ks++) {
          half8_t afn[NA];
#pragma unroll
          for (int n = 0; n < NB; n++) {
#pragma unroll
            for (int i = 0; i < NV; i++)
              acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[n], af[i], acc[i][n], 0, 0, 0);
            load_bf(bf, s, n, ks + 1);
            // row group n / 2 of the next sub-step, decoded between the MFMAs
            if ((n & 1) && (n >> 1) < NV) afn[n >> 1] = decode8_e2m1_f16(araw[n >> 1][ks + 1], as2[n >> 1][(ks + 1) >> 1]);
          }
#pragma unroll
          for (int i = 0; i < NV; i++) af[i] = afn[i];
          __builtin_amdgcn_sched_barrier(0);  // keeps each sub-step's operands to one register set
        }
        // every LDS read of step s is in registers: the data waves may overwrite its
        // buffers once all MFMA waves pass this barrier (the top of step s + 1; after the
        // last step, the data waves' closing barrier, and the reads of a step that does
        // not exist are never used)
        __syncthreads();
        load_a(araw, asc, s + 1);
        half8_t afn[NA];
#pragma unroll
        for (int n = 0; n < NB; n++) {
#pragma unroll
          for (int i = 0; i < NV; i++)
            acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[n], af[i], acc[i][n], 0, 0, 0);
          load_bf(bf, s + 1, n, 0);
          // the next step's first sub-step: its scales, then row group n - 4
          if (n == NB / 2 - 1) cvt_scales();
          if (n >= NB / 2 && n - NB / 2 < NV) afn[n - NB / 2] = decode8_e2m1_f16(araw[n - NB / 2][0], as2[n - NB / 2][0]);
        }
#pragma unroll
        for (int i = 0; i < NV; i++) af[i] = afn[i];
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NV > 0) {
        // lane (rr, q) holds, for row group i, output row 16 c + 64 i + rr and the four
        // columns 4 q .. 4 q + 3 of each 16-column group n.  The lane terms come from an
        // opaque copy of the lane id, so that the compiler does not hoist the epilogue's
        // address arithmetic out of the step loop (it would spill it there, and the reload
        // would then wait for this item's output stores).
        int elane = lane;
        asm volatile("" : "+v"(elane));
        const int q = elane >> 4, rr = elane & 15;
        float alpha;
        void* obase;
        size_t ldo;
        if constexpr (MASKED) {
          alpha = alpha_s[cit.g];
          obase = p.out;
          ldo = N;
        } else {
          alpha = p.grp[cit.g].alpha;
          obase = p.grp[cit.g].out;
          ldo = p.grp[cit.g].ldc;
        }
#pragma unroll
        for (int i = 0; i < NV; i++) {
          const int m = cit.m0 + 16 * c + 64 * i + rr;
          const bool ok = m < cit.mm;
          const size_t orow = CONTIG ? (size_t)__builtin_amdgcn_readfirstlane(rs_s[cit.g]) + m
                              : MASKED ? (size_t)cit.g * cap + m : (size_t)m;
          if constexpr (SWIGLU) {
#pragma unroll
            for (int n = 0; n < NB / 2; n++) {
              float h[4], gv[4], uv[4];
#pragma unroll
              for (int r = 0; r < 4; r++) {
                const float gt = alpha * acc[i][n][r], up = alpha * acc[i][n + NB / 2][r];
                gv[r] = gt;
                uv[r] = up;
                h[r] = gt / (1.0f + expf(-gt)) * up;
              }
              const int hc0 = cit.n0 + 16 * n;  // first column of this lane's 16-block
              if (p.dbg_h && ok) *(float4_t*)(p.dbg_h + orow * I + hc0 + 4 * q) = float4_t{h[0], h[1], h[2], h[3]};
              if (p.dbg_g1 && ok) {
                *(float4_t*)(p.dbg_g1 + orow * 2 * I + hc0 + 4 * q) = float4_t{gv[0], gv[1], gv[2], gv[3]};
                *(float4_t*)(p.dbg_g1 + orow * 2 * I + I + hc0 + 4 * q) = float4_t{uv[0], uv[1], uv[2], uv[3]};
              }
              uint32_t sbyte;
              const uint32_t bits = quantize_block_x4(h, p.g_h, 6.0f * p.g_h, sbyte);
              const uint32_t b1 = __shfl_xor(bits, 16), b2 = __shfl_xor(bits, 32), b3 = __shfl_xor(bits, 48);
              if (q == 0 && ok) {
                *(u32x2_t*)(p.h_codes + orow * (I / 2) + hc0 / 2) = u32x2_t{bits | (b1 << 16), b2 | (b3 << 16)};
                p.h_sf[orow * (I / 16) + hc0 / 16] = (uint8_t)sbyte;
              }
            }
          } else {
#pragma unroll
            for (int n = 0; n < NB; n++) {
              const int col = cit.n0 + 16 * n + 4 * q;
              const float4_t v = acc[i][n] * alpha;
              if (!ok) continue;
              if constexpr (EPI == EPI_BF16) {
                const uint32_t lo = bf16x2_rne(v[0], v[1]);
                const uint32_t hi = bf16x2_rne(v[2], v[3]);
                *(u32x2_t*)((uint16_t*)obase + orow * ldo + col) = u32x2_t{lo, hi};
              } else {
                *(float4_t*)((float*)obase + orow * ldo + col) = v;
              }
            }
          }
        }
      }
    };
    switch (nv) {
      case 4: item(std::integral_constant<int, 4>{}); break;
      case 3: item(std::integral_constant<int, 3>{}); break;
      case 2: item(std::integral_constant<int, 2>{}); break;
      case 1: item(std::integral_constant<int, 1>{}); break;
      default: item(std::integral_constant<int, 0>{}); break;
    }
    cit = nit;
    nv = nv_of(nit);
  }
}

template <int EPI, int MODE>
static hipError_t launch_stream(const typename ArgsOf<MODE>::type& p, int cu_limit, hipStream_t s) {
  const void* k = (const void*)k_gemm_nvfp4_stream<EPI, MODE>;
  const int grid = resident_grid(k, ns::THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_nvfp4_stream<EPI, MODE>), dim3(grid), dim3(ns::THREADS), 0, s, p);
  return hipGetLastError();
}

// Returns hipErrorNotSupported (nothing launched) for shapes the kernel does not take.
hipError_t gemm_nvfp4_stream(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s) {
  using namespace ns;
  if (p.G <= 0 || p.G > STREAM_MAX_G || p.K % BK != 0 || p.K <= 0 || p.max_m <= 0) return hipErrorNotSupported;
  const int ncols = epi == EPI_SWIGLU_NVFP4 ? BN / 2 : BN;
  const int n_out = epi == EPI_SWIGLU_NVFP4 ? p.N / 2 : p.N;
  if (n_out % ncols != 0 || (epi == EPI_SWIGLU_NVFP4 && p.N % 2 != 0)) return hipErrorNotSupported;
  if ((long long)p.G * ((p.max_m + BM - 1) / BM) * (n_out / ncols) > 0x7FFFFFFFLL) return hipErrorNotSupported;
  switch (epi) {
    case EPI_BF16: return launch_stream<EPI_BF16, MODE_MASKED>(p, cu_limit, s);
    case EPI_F32: return launch_stream<EPI_F32, MODE_MASKED>(p, cu_limit, s);
    case EPI_SWIGLU_NVFP4: return launch_stream<EPI_SWIGLU_NVFP4, MODE_MASKED>(p, cu_limit, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_nvfp4_contiguous(MaskedGemmArgs p, int epi, int cu_limit, hipStream_t s) {
  using namespace ns;
  if (p.G <= 0 || p.G > STREAM_CONTIG_MAX_G || p.K % BK != 0 || p.K <= 0 || p.N % BN != 0 || p.N <= 0 ||
      p.max_m <= 0 || !p.row_start)
    return hipErrorNotSupported;
  if ((long long)((p.max_m + BM - 1) / BM + p.G) * (p.N / BN) > 0x7FFFFFFFLL) return hipErrorNotSupported;
  switch (epi) {
    case EPI_BF16: return launch_stream<EPI_BF16, MODE_CONTIG>(p, cu_limit, s);
    case EPI_F32: return launch_stream<EPI_F32, MODE_CONTIG>(p, cu_limit, s);
    default: return hipErrorNotSupported;
  }
}

// Heterogeneous groups: every group with rows needs N % 128 == 0, K % 128 == 0 and an
// output row stride and base that keep the 4-column stores aligned.  The groups are
// reordered by decreasing item cost and their items dealt longest-first onto the
// workgroups (hetero_lpt_schedule); the item cost is the item's K steps times (0.6 + its
// share of a full 256-row tile), the weight stream and decode being paid per step whatever
// the rows.
hipError_t gemm_nvfp4_stream_hetero(HeteroGemmArgs p, int epi, int cu_limit, hipStream_t s) {
  using namespace ns;
  if (epi != EPI_BF16 && epi != EPI_F32) return hipErrorNotSupported;
  const uintptr_t out_align = epi == EPI_BF16 ? 8 : 16;
  long long items = 0;
  for (int g = 0; g < p.G; g++) {
    const HeteroGroup& q = p.grp[g];
    if (q.M == 0) continue;
    if (q.N % BN != 0 || q.K % BK != 0 || q.ldc % 4 != 0 || ((uintptr_t)q.out & (out_align - 1)) != 0)
      return hipErrorNotSupported;
    items += (long long)(q.M + BM - 1) / BM * (q.N / BN);
  }
  if (items == 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL) return hipErrorNotSupported;
  auto cost = [&](const HeteroGroup& q) { return (q.K / BK) * (0.6 + (q.M < BM ? q.M : BM) / (double)BM); };
  HeteroGemmArgs r = p;
  bool taken[MXG_MAX_GROUPS] = {};
  double c[MXG_MAX_GROUPS];
  int n = 0;
  for (int pass = 0; pass < p.G; pass++) {  // stable selection by decreasing cost, empty groups dropped
    int best = -1;
    for (int g = 0; g < p.G; g++) {
      if (p.grp[g].M == 0 || taken[g]) continue;
      if (best < 0 || cost(p.grp[g]) > cost(p.grp[best])) best = g;
    }
    if (best < 0) break;
    HeteroGroup q = p.grp[best];
    q.tiles_m = (q.M + BM - 1) / BM;
    q.tiles_n = q.N / BN;
    c[n] = cost(q);
    r.grp[n++] = q;
    taken[best] = true;
  }
  r.G = n;
  const void* k = epi == EPI_BF16 ? (const void*)k_gemm_nvfp4_stream<EPI_BF16, MODE_HETERO>
                                  : (const void*)k_gemm_nvfp4_stream<EPI_F32, MODE_HETERO>;
  const int grid = resident_grid(k, ns::THREADS, cu_limit);
  if (grid <= 0) return hipErrorInvalidValue;
  hetero_lpt_schedule(r.grp, c, n, grid, r.sched);
  return epi == EPI_BF16 ? launch_stream<EPI_BF16, MODE_HETERO>(r, cu_limit, s)
                         : launch_stream<EPI_F32, MODE_HETERO>(r, cu_limit, s);
}

}  // namespace mxg
