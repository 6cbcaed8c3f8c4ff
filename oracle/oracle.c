/*
 * oracle.c -- plain, slow CPU oracle for the block-scaled grouped GEMM and the
 * mixture-of-experts expert path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include, link
 * or call this file; only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load it.  It shares no code, table or
 * constant generator with the GPU library.
 *
 * Arithmetic: every decoded operand value is an exact double; sums are fp64.
 * Encoders (e2m1, e4m3, bf16) are nearest-value searches over tables that are
 * built from the bit-field definitions, so they do not depend on any bit trick.
 *
 * Sources (the pages are cited by title and section):
 *  - "The CuteDSL Gamble: Chasing Kernel Efficiency on Blackwell GPUs",
 *    section "The Message": grouped_gemm_nt_masked is a masked, batched GEMM
 *    whose operands are (data, scale-factor) pairs, with dtype strings, an
 *    sf_vec_size, a per-group masked_m and optional alpha scaling at output.
 *  - same page, "Input Knowledge Required": NVFP4 is 4-bit floating point
 *    with block-level scale factors.
 *  - "llm-assisted-kernel-dev" README, section on mixture-of-experts
 *    (moe_fibench_ref.py and moe_fp8fpX_fused.py rows): DeepSeek-V3 no-aux
 *    routing (sigmoid(logits)+bias, grouped top-k, routed_scaling_factor),
 *    then per expert GEMM1 -> SwiGLU -> GEMM2 over e4m3fn data with block
 *    scales; BF16 is the optimized kernel's default intermediate precision.
 *  - The bit layouts of e2m1 (sign, 2 exponent bits with bias 1, 1 mantissa
 *    bit, no inf/NaN) and e4m3fn (sign, 4 exponent bits with bias 7,
 *    3 mantissa bits, S.1111.111 = NaN, no inf) are the standard OCP
 *    definitions; the pages name the formats but do not spell them out.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

static double E2M1[16];  /* value of every e2m1 code */
static double E4M3[256]; /* value of every e4m3fn code (NaN for 0x7F/0xFF) */

/* e2m1 code [s e1 e0 m]: e==0 -> m * 0.5 (subnormal), else 2^(e-1) * (1 + m/2). */
static double e2m1_from_bits(unsigned c) {
  unsigned s = (c >> 3) & 1u, e = (c >> 1) & 3u, m = c & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* e4m3fn code [s eeee mmm]: e==0 -> m * 2^-9, else (1 + m/8) * 2^(e-7); 0x7F/0xFF NaN. */
static double e4m3_from_bits(unsigned c) {
  unsigned s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

void orc_init(void) {
  for (unsigned c = 0; c < 16; c++) E2M1[c] = e2m1_from_bits(c);
  for (unsigned c = 0; c < 256; c++) E4M3[c] = e4m3_from_bits(c);
}

double orc_e2m1_value(int code) { return E2M1[code & 15]; }
double orc_e4m3_value(int code) { return E4M3[code & 255]; }

/* Nearest e2m1 code to v.  Ties go to the code whose last bit is 0 (round to
 * nearest even); magnitudes beyond 6 saturate to 6; the sign bit is signbit(v). */
int orc_encode_e2m1(double v) {
  double a = fabs(v);
  if (a > 6.0) return 7 | (signbit(v) ? 8 : 0); /* saturation (also for +-inf) */
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; c++) {
    double d = fabs(a - E2M1[c]);
    if (d < bestd || (d == bestd && (c & 1) == 0)) { best = c; bestd = d; }
  }
  return best | (signbit(v) ? 8 : 0);
}

/* Nearest finite e4m3fn code to v (ties to even code); |v| > 448 saturates. */
int orc_encode_e4m3_sat(double v) {
  double a = fabs(v);
  if (a > 448.0) return 0x7E | (signbit(v) ? 0x80 : 0); /* saturation (also for +-inf) */
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 127; c++) { /* 0x00..0x7E: every finite non-negative code */
    double d = fabs(a - E4M3[c]);
    if (d < bestd || (d == bestd && (c & 1) == 0)) { best = c; bestd = d; }
  }
  return best | (signbit(v) ? 0x80 : 0);
}

/* bf16 bits of v rounded once to nearest (ties to even), straight from fp64.
 * bf16 keeps 8 significant bits; its smallest normal is 2^-126 and its
 * subnormal step is 2^-133; anything that rounds past the largest finite
 * value (2 - 2^-7) * 2^127 becomes infinity. */
uint16_t orc_bf16_bits(double v) {
  if (isnan(v)) return 0x7FC0;
  int neg = signbit(v) != 0;
  double a = fabs(v);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    int ex;
    frexp(a, &ex);                    /* a = f * 2^ex, f in [0.5, 1) */
    int q = (ex - 1 >= -126) ? ex - 8 : -133; /* exponent of the last kept bit */
    r = ldexp(nearbyint(ldexp(a, -q)), q);    /* nearbyint: ties to even */
  }
  const double maxbf = ldexp(2.0 - ldexp(1.0, -7), 127);
  uint32_t bits;
  if (r > maxbf) {
    bits = 0x7F800000u;
  } else {
    float f = (float)r; /* exact: r has at most 8 significant bits */
    memcpy(&bits, &f, 4);
  }
  uint16_t out = (uint16_t)(bits >> 16);
  return neg ? (uint16_t)(out | 0x8000u) : out;
}

double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 operands                                                            */
/* Layout: codes [rows, K/2] bytes, element k of a row in byte k/2, low       */
/* nibble for even k; scales [rows, K/16] e4m3fn bytes, one per 16 elements. */
/* ------------------------------------------------------------------------ */

static double nvfp4_elem(const uint8_t* codes, const uint8_t* sf, int K, long row, int k) {
  uint8_t byte = codes[row * (long)(K / 2) + k / 2];
  unsigned c = (k & 1) ? (byte >> 4) : (byte & 15u);
  return E2M1[c] * E4M3[sf[row * (long)(K / 16) + k / 16]];
}

/* One A row against rows [0, nb) of B:
 *   y[n] = alpha * sum_k dec(A)[k] * dec(B)[n,k],  s[n] = |alpha| * sum_k |dec(A)[k] * dec(B)[n,k]|
 * where dec(X)[r,k] = e2m1(code) * e4m3(scale of the 16-block holding k). */
void orc_nvfp4_row_dot(const uint8_t* a, const uint8_t* a_sf, long a_row,
                       const uint8_t* b, const uint8_t* b_sf, int nb, int K, double alpha,
                       double* y, double* s) {
  double* ad = (double*)malloc(sizeof(double) * (size_t)K);
  for (int k = 0; k < K; k++) ad[k] = nvfp4_elem(a, a_sf, K, a_row, k);
#pragma omp parallel for schedule(static)
  for (int n = 0; n < nb; n++) {
    double acc = 0.0, accabs = 0.0;
    for (int k = 0; k < K; k++) {
      double p = ad[k] * nvfp4_elem(b, b_sf, K, n, k);
      acc += p;
      accabs += fabs(p);
    }
    if (y) y[n] = alpha * acc;
    if (s) s[n] = fabs(alpha) * accabs;
  }
  free(ad);
}

/* Selected A rows against rows [0, nb) of B: for m < M,
 *   y[m, n] = alpha * sum_k dec(A)[a_rows[m], k] * dec(B)[n, k],  s[m, n] likewise of |.|,
 * the same fp64 sums in k order as orc_nvfp4_row_dot, with each operand row decoded
 * once (a subset of tokens routed to one expert, evaluated together). */
void orc_gemm_nvfp4_rows(const uint8_t* a, const uint8_t* a_sf, const int32_t* a_rows, int M,
                         const uint8_t* b, const uint8_t* b_sf, int nb, int K, double alpha,
                         double* y, double* s) {
  double* ad = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
  for (int m = 0; m < M; m++)
    for (int k = 0; k < K; k++) ad[(size_t)m * K + k] = nvfp4_elem(a, a_sf, K, a_rows[m], k);
#pragma omp parallel
  {
    double* bd = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < nb; n++) {
      for (int k = 0; k < K; k++) bd[k] = nvfp4_elem(b, b_sf, K, n, k);
      for (int m = 0; m < M; m++) {
        const double* av = ad + (size_t)m * K;
        double acc = 0.0, accabs = 0.0;
        for (int k = 0; k < K; k++) {
          double p = av[k] * bd[k];
          acc += p;
          accabs += fabs(p);
        }
        if (y) y[(size_t)m * nb + n] = alpha * acc;
        if (s) s[(size_t)m * nb + n] = fabs(alpha) * accabs;
      }
    }
    free(bd);
  }
  free(ad);
}

/* Masked grouped NT GEMM over NVFP4 operands (the masked batched GEMM with
 * scale factors and alpha at output of "The CuteDSL Gamble", "The Message").
 *   A [G, max_m, K], B [G, N, K] (NVFP4 as above), alpha [G] (NULL -> 1),
 *   masked_m [G], clamped to [0, max_m].
 * For g < G, m < masked_m[g], n < N:
 *   y[g,m,n] = alpha[g] * sum_k dec(A)[g,m,k] * dec(B)[g,n,k]   (fp64, unrounded)
 *   s[g,m,n] = |alpha[g]| * sum_k |dec(A) * dec(B)|
 *   out[g,m,n] = bf16 bits of y rounded once to nearest even.
 * Rows m >= masked_m[g] of y, s and out are never written.  Any of y, s, out
 * may be NULL. */
void orc_gemm_nvfp4_masked(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                           const uint8_t* b_sf, const float* alpha, const int32_t* masked_m,
                           int G, int max_m, int N, int K, double* y, double* s, uint16_t* out) {
  double* yr = (double*)malloc(sizeof(double) * (size_t)N);
  double* sr = (double*)malloc(sizeof(double) * (size_t)N);
  for (int g = 0; g < G; g++) {
    int mm = masked_m[g];
    if (mm < 0) mm = 0;
    if (mm > max_m) mm = max_m;
    double al = alpha ? (double)alpha[g] : 1.0;
    const uint8_t* ag = a + (size_t)g * max_m * (K / 2);
    const uint8_t* asg = a_sf + (size_t)g * max_m * (K / 16);
    const uint8_t* bg = b + (size_t)g * N * (K / 2);
    const uint8_t* bsg = b_sf + (size_t)g * N * (K / 16);
    for (int m = 0; m < mm; m++) {
      orc_nvfp4_row_dot(ag, asg, m, bg, bsg, N, K, al, yr, sr);
      size_t base = ((size_t)g * max_m + m) * N;
      for (int n = 0; n < N; n++) {
        if (y) y[base + n] = yr[n];
        if (s) s[base + n] = sr[n];
        if (out) out[base + n] = orc_bf16_bits(yr[n]);
      }
    }
  }
  free(yr);
  free(sr);
}

/* ------------------------------------------------------------------------ */
/* FP8 block-scaled operands (DeepSeek-V3 style, the mixture-of-experts row  */
/* of the "llm-assisted-kernel-dev" README): activations e4m3fn [M, K] with  */
/* one fp32 scale per 1x128; weights e4m3fn [N, K] with one fp32 scale per    */
/* 128x128 block, scales [N/128, K/128].                                      */
/* ------------------------------------------------------------------------ */

/* y[m,n] = sum_k (e4m3(qa[m,k]) * sa[m,k/128]) * (e4m3(qb[n,k]) * sb[n/128,k/128])
 * s[m,n] = the same sum of absolute values.  Rows of qa/sa are given by a
 * row-index list (NULL -> rows 0..M-1) so one token subset can be evaluated.
 * Each selected A row and each B row is decoded once into exact doubles; every
 * (m, n) is then the plain fp64 sum over k = 0..K-1 in order. */
void orc_gemm_fp8_block(const uint8_t* qa, const float* sa, const int32_t* a_rows, int M,
                        const uint8_t* qb, const float* sb, int N, int K, double* y, double* s) {
  int KB = K / 128;
  double* ad = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
  for (int m = 0; m < M; m++) {
    long ar = a_rows ? a_rows[m] : m;
    for (int k = 0; k < K; k++)
      ad[(size_t)m * K + k] = E4M3[qa[ar * K + k]] * (double)sa[ar * KB + k / 128];
  }
#pragma omp parallel
  {
    double* bd = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; n++) {
      for (int k = 0; k < K; k++) bd[k] = E4M3[qb[(long)n * K + k]] * (double)sb[(n / 128) * KB + k / 128];
      for (int m = 0; m < M; m++) {
        const double* av = ad + (size_t)m * K;
        double acc = 0.0, accabs = 0.0;
        for (int k = 0; k < K; k++) {
          double p = av[k] * bd[k];
          acc += p;
          accabs += fabs(p);
        }
        y[(size_t)m * N + n] = acc;
        if (s) s[(size_t)m * N + n] = accabs;
      }
    }
    free(bd);
  }
  free(ad);
}

/* Dense activations (given as exact doubles, e.g. bf16 values) times FP8
 * 128x128-block-scaled weights: y[m,n] = sum_k a[m,k] * e4m3(qb[n,k]) * sb[n/128,k/128],
 * each term evaluated as (a * e4m3) * scale, summed in k order. */
void orc_gemm_dense_fp8w(const double* a, int M, const uint8_t* qb, const float* sb, int N, int K,
                         double* y, double* s) {
  int KB = K / 128;
#pragma omp parallel
  {
    double* be = (double*)malloc(sizeof(double) * (size_t)K);
    double* bs = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; n++) {
      for (int k = 0; k < K; k++) {
        be[k] = E4M3[qb[(long)n * K + k]];
        bs[k] = (double)sb[(n / 128) * KB + k / 128];
      }
      for (int m = 0; m < M; m++) {
        const double* av = a + (long)m * K;
        double acc = 0.0, accabs = 0.0;
        for (int k = 0; k < K; k++) {
          double p = av[k] * be[k] * bs[k];
          acc += p;
          accabs += fabs(p);
        }
        y[(size_t)m * N + n] = acc;
        if (s) s[(size_t)m * N + n] = accabs;
      }
    }
    free(be);
    free(bs);
  }
}

/* NVFP4-weight x bf16-activation GEMV (W4A16, the nvfp4_gemv row of the Helion
 * pretuned-kernel table):
 *   y[m,n] = g * sum_k bf16(x[m,k]) * dec(W)[n,k],  s[m,n] = |g| * sum_k |bf16(x) * dec(W)|
 * x: bf16 bits [M, K]; W: NVFP4 codes [N, K/2], scales [N, K/16]; g: W's global
 * dequantization scale.  fp64, unrounded. */
void orc_gemv_nvfp4_w4a16(const uint16_t* x, int M, const uint8_t* w, const uint8_t* w_sf, int N, int K,
                          double g, double* y, double* s) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < (long)M * N; i++) {
    long m = i / N, n = i % N;
    double acc = 0.0, accabs = 0.0;
    for (int k = 0; k < K; k++) {
      double p = orc_bf16_value(x[m * K + k]) * nvfp4_elem(w, w_sf, K, n, k);
      acc += p;
      accabs += fabs(p);
    }
    y[i] = g * acc;
    if (s) s[i] = fabs(g) * accabs;
  }
}

/* ------------------------------------------------------------------------ */
/* NVFP4 quantizer (reading: block scale = e4m3(amax / (6 g)), block dequant   */
/* scale d = scale * g, code = e2m1(x * (1/d)); every step an fp32 operation   */
/* rounded to nearest).  g is the tensor's fp32 global dequantization scale.  */
/* ------------------------------------------------------------------------ */
void orc_quantize_nvfp4(const float* x, long rows, int K, float g, uint8_t* codes, uint8_t* sf) {
  const float six_g = 6.0f * g;
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; r++) {
    for (int blk = 0; blk < K / 16; blk++) {
      const float* xb = x + r * K + blk * 16;
      float amax = 0.0f;
      for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(xb[i]));
      float q = amax / six_g;
      int scode = orc_encode_e4m3_sat((double)q);
      sf[r * (K / 16) + blk] = (uint8_t)scode;
      float sval = (float)E4M3[scode];
      int c[16];
      if (sval == 0.0f) {
        for (int i = 0; i < 16; i++) c[i] = signbit(xb[i]) ? 8 : 0;
      } else {
        float d = sval * g;
        float rcp = 1.0f / d;
        for (int i = 0; i < 16; i++) c[i] = orc_encode_e2m1((double)(xb[i] * rcp));
      }
      for (int i = 0; i < 16; i += 2)
        codes[r * (K / 2) + blk * 8 + i / 2] = (uint8_t)(c[i] | (c[i + 1] << 4));
    }
  }
}

/* ------------------------------------------------------------------------ */
/* DeepSeek-V3 no-aux router (the mixture-of-experts row of the               */
/* "llm-assisted-kernel-dev" README: sigmoid(logits) + bias, grouped top-k,    */
/* routed_scaling_factor).  Readings: the sigmoid is evaluated in fp64 and    */
/* rounded once to fp32; selection uses s + bias (fp32), groups are            */
/* contiguous blocks of E/n_group experts scored by the fp32 sum of their two  */
/* largest s + bias; the topk_group best groups are kept; the top_k best      */
/* experts inside them are taken; ties go to the lower index everywhere; the  */
/* weights use s without the bias, divided by the fp32 slot-order sum of the  */
/* selected s, then multiplied by routed_scaling_factor.                       */
/* ------------------------------------------------------------------------ */
void orc_route_noaux(const float* logits, const float* bias, int T, int E, int n_group,
                     int topk_group, int top_k, float rsf, int32_t* ids, float* w) {
  int gsize = E / n_group;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; t++) {
    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    float* sb = (float*)malloc(sizeof(float) * (size_t)E);
    float* gs = (float*)malloc(sizeof(float) * (size_t)n_group);
    char* gkeep = (char*)calloc((size_t)n_group, 1);
    char* taken = (char*)calloc((size_t)E, 1);
    for (int e = 0; e < E; e++) {
      s[e] = (float)(1.0 / (1.0 + exp(-(double)logits[(long)t * E + e])));
      sb[e] = s[e] + bias[e];
    }
    for (int q = 0; q < n_group; q++) {
      /* the two largest values of the group (the same value may appear twice) */
      int i1 = -1;
      for (int e = q * gsize; e < (q + 1) * gsize; e++)
        if (i1 < 0 || sb[e] > sb[i1]) i1 = e;
      int i2 = -1;
      for (int e = q * gsize; e < (q + 1) * gsize; e++)
        if (e != i1 && (i2 < 0 || sb[e] > sb[i2])) i2 = e;
      gs[q] = (gsize >= 2) ? sb[i1] + sb[i2] : sb[i1];
    }
    for (int r = 0; r < topk_group; r++) {
      int best = -1;
      for (int q = 0; q < n_group; q++)
        if (!gkeep[q] && (best < 0 || gs[q] > gs[best])) best = q;
      gkeep[best] = 1;
    }
    int sel[64];
    for (int j = 0; j < top_k; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        if (taken[e] || !gkeep[e / gsize]) continue;
        if (best < 0 || sb[e] > sb[best]) best = e;
      }
      taken[best] = 1;
      sel[j] = best;
    }
    float den = 0.0f;
    for (int j = 0; j < top_k; j++) den = den + s[sel[j]];
    for (int j = 0; j < top_k; j++) {
      ids[(long)t * top_k + j] = sel[j];
      float q = s[sel[j]] / den;
      w[(long)t * top_k + j] = q * rsf;
    }
    free(s); free(sb); free(gs); free(gkeep); free(taken);
  }
}

/* Token -> expert permutation for the masked layout: the (t, j) slot routed to
 * expert e = ids[t,j] gets row[t,j] = number of earlier tokens routed to e
 * (a stable counting sort in token order); masked_m[e] = min(count_e, max_m).
 * Slots whose row is >= max_m do not fit the capacity and are dropped. */
void orc_dispatch(const int32_t* ids, int T, int E, int top_k, int max_m, int32_t* masked_m,
                  int32_t* row) {
  int32_t* count = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int t = 0; t < T; t++)
    for (int j = 0; j < top_k; j++) {
      int e = ids[(long)t * top_k + j];
      row[(long)t * top_k + j] = count[e];
      count[e] += 1;
    }
  for (int e = 0; e < E; e++) masked_m[e] = count[e] < max_m ? count[e] : max_m;
  free(count);
}

/* SwiGLU on one stacked GEMM1 output (the "GEMM1 -> SwiGLU -> GEMM2" step of
 * the same README row): gate = columns [0, I), up = columns [I, 2I);
 * h = silu(gate) * up with silu(v) = v / (1 + exp(-v)), in fp64. */
void orc_swiglu(const double* gate_up, int rows, int I, double* h) {
  for (long r = 0; r < rows; r++)
    for (int i = 0; i < I; i++) {
      double gt = gate_up[r * 2 * I + i], up = gate_up[r * 2 * I + I + i];
      h[r * I + i] = gt / (1.0 + exp(-gt)) * up;
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Array forms of the scalar encoders, for the Python wrapper. */
void orc_bf16_bits_array(const double* v, long n, uint16_t* out) {
  for (long i = 0; i < n; i++) out[i] = orc_bf16_bits(v[i]);
}
void orc_encode_e2m1_array(const double* v, long n, uint8_t* out) {
  for (long i = 0; i < n; i++) out[i] = (uint8_t)orc_encode_e2m1(v[i]);
}
void orc_encode_e4m3_array(const double* v, long n, uint8_t* out) {
  for (long i = 0; i < n; i++) out[i] = (uint8_t)orc_encode_e4m3_sat(v[i]);
}
