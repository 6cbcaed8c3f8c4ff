// device_common.h -- gfx950 device helpers shared by the library's kernels:
// vector types, NVFP4 / e4m3 / bf16 conversions and the NVFP4 block quantizer.
//
// Formats (the pages name them -- NVFP4 as 4-bit floats with block scale
// factors in "The CuteDSL Gamble", "Input Knowledge Required"; e4m3fn scales
// in the "llm-assisted-kernel-dev" README's mixture-of-experts table -- the bit
// layouts are the OCP ones): e2m1 = [s e1 e0 m], bias 1, no inf/NaN;
// e4m3fn = [s eeee mmm], bias 7, S.1111.111 = NaN, no inf, max 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef int int4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// e4m3fn byte -> fp32 value.  Placing the 7 magnitude bits at fp32 bit 20
// gives the value times 2^-120 (normals and subnormals alike, since both
// formats continue their subnormal ranges linearly); one exact multiply
// restores it.  The NaN codes map to NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t mag = c & 0x7Fu;
  float v = __uint_as_float(((c & 0x80u) << 24) | (mag << 20)) * 0x1p120f;
  return mag == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
}

// fp32 -> bf16 bits, round to nearest even; a NaN becomes the quiet NaN with the upper
// half of its bits (u >> 16 | 0x40).  gfx950's v_cvt_pk_bf16_f32 does exactly this: it
// matched that bit-level definition on every one of the 2^32 fp32 inputs.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values in one instruction: lo in bits 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

// Round a fp32 value to the nearest finite e4m3fn code (ties to even mantissa),
// saturating magnitudes above 448 to 448 (code 0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = __builtin_fabsf(v);
  if (a != a) return sign | 0x7Fu;
  if (a >= 464.0f) return sign | 0x7Eu;
  if (a < 0x1p-6f) {
    // subnormal range: multiples of 2^-9; a * 512 is exact, rintf rounds ties to even.
    // A result of 8 is 2^-6, whose code (exponent field 1, mantissa 0) is also 8.
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  uint32_t u = __float_as_uint(a);
  int e = (int)(u >> 23) - 127;           // -6 .. 8
  uint32_t mant = u & 0x7FFFFFu;
  uint32_t m3 = mant >> 20, rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) m3 += 1;
  if (m3 == 8) { m3 = 0; e += 1; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | m3;
  if (code > 0x7Eu) code = 0x7Eu;          // (448, 464) rounds to 448
  return sign | code;
}

// Round a fp32 value to the nearest e2m1 code: magnitudes {0,.5,1,1.5,2,3,4,6};
// at a midpoint the code with last bit 0 wins; beyond 6 saturates; sign kept.
__device__ __forceinline__ uint32_t f32_to_e2m1_rne_sat(float v) {
  uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  float a = __builtin_fabsf(v);
  uint32_t c = a <= 0.25f ? 0u
             : a < 0.75f ? 1u
             : a <= 1.25f ? 2u
             : a < 1.75f ? 3u
             : a <= 2.5f ? 4u
             : a < 3.5f ? 5u
             : a <= 5.0f ? 6u : 7u;
  return sign | c;
}

// NVFP4 quantization of one 16-element block (fp32 values, fp32 arithmetic with
// round-to-nearest at every step): S = e4m3(amax / (6 g)), d = S * g,
// code_i = e2m1(x_i * (1 / d)).  Returns the scale byte; codes packed two per
// byte (element 2i in the low nibble) into out[0..1] (little-endian dwords).
__device__ __forceinline__ uint32_t quantize_block16(const float* x, float g, float six_g,
                                                     uint32_t out[2]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  float q = amax / six_g;
  uint32_t s = f32_to_e4m3_rne_sat(q);
  float sval = e4m3_to_f32(s);
  uint32_t w0 = 0, w1 = 0;
  if (sval == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      uint32_t c = (__float_as_uint(x[i]) >> 28) & 0x8u;
      if (i < 8) w0 |= c << (4 * i); else w1 |= c << (4 * (i - 8));
    }
  } else {
    float d = sval * g;
    float r = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      uint32_t c = f32_to_e2m1_rne_sat(x[i] * r);
      if (i < 8) w0 |= c << (4 * i); else w1 |= c << (4 * (i - 8));
    }
  }
  out[0] = w0;
  out[1] = w1;
  return s;
}

// Decode one dword of 8 e2m1 codes (element 0 in the low nibble) times the
// block scale s (fp16, exact: e4m3 values fit fp16's normal range) into 8 fp16
// values.  e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688], so every product is exact in fp16.
__device__ __forceinline__ half8_t decode8_e2m1_f16(uint32_t w, half2_t s2) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ half2_t scale_e4m3_to_h2(uint32_t c) {
  _Float16 h = (_Float16)e4m3_to_f32(c);
  half2_t r = {h, h};
  return r;
}

// NVFP4 quantization of one 16-column block spread over the 4 lanes
// {m, m+16, m+32, m+48} (4 values each, element (lane/16)*4 + r).  Same operation
// sequence as quantize_block16.  Returns this lane's 16 code bits (element order)
// and the scale byte.
__device__ __forceinline__ uint32_t quantize_block_x4(const float h[4], float g, float six_g,
                                                      uint32_t& scale) {
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; r++) amax = __builtin_fmaxf(amax, __builtin_fabsf(h[r]));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
  float qv = amax / six_g;
  uint32_t s = f32_to_e4m3_rne_sat(qv);
  float sval = e4m3_to_f32(s);
  uint32_t bits = 0;
  if (sval == 0.0f) {
#pragma unroll
    for (int r = 0; r < 4; r++) bits |= ((__float_as_uint(h[r]) >> 28) & 0x8u) << (4 * r);
  } else {
    float d = sval * g;
    float rc = 1.0f / d;
#pragma unroll
    for (int r = 0; r < 4; r++) bits |= f32_to_e2m1_rne_sat(h[r] * rc) << (4 * r);
  }
  scale = s;
  return bits;
}

// Physical row of logical W13 row r (gate rows [0, I), up rows [I, 2I)): r itself in
// the stacked layout; with gate and up interleaved in 16-row blocks, gate row j sits at
// 32 (j / 16) + j % 16 and up row j 16 rows after it.
__device__ __forceinline__ int w13_row(int r, int I, bool il16) {
  if (!il16) return r;
  const bool up = r >= I;
  const int j = up ? r - I : r;
  return ((j >> 4) << 5) + (up ? 16 : 0) + (j & 15);
}

// LDS DMA (global_load_lds_*): 64 lanes each copy 16 (or 4) bytes from their own global
// address into LDS at base + lane * 16 (or 4), without passing through registers.  The
// streaming kernels issue every asynchronous operation of their main loops this way and
// wait with explicit partial vmcnt waits: the compiler, which cannot see these loads,
// would otherwise drain all outstanding loads (vmcnt(0)) before each LDS read.  No
// register-destination load is issued with inline assembly, so no register can be
// overwritten behind the compiler's back.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  // the LDS base is wave-uniform; readfirstlane puts it in an SGPR for M0
  uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}

// The same DMAs with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte
// offset (the saddr form), which keeps per-lane addresses to one VGPR each.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, void* lds) {
  uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, void* lds) {
  uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace mxg
