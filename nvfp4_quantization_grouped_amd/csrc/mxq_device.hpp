// Device-side building blocks shared by the libmxq kernels (gfx950 / CDNA4).
//
// Element conversions use gfx950's scaled conversion instructions
// (v_cvt_scalef32_pk_*): towards fp4/fp8 they divide by the given scale and
// round to nearest-even, saturating e2m1 at 6; back from fp4/fp8 they
// multiply by the scale.  For power-of-two scales these are exactly the
// element steps of the pages' formats, with two sign-of-zero conventions
// fixed up here: the pages' e2m1 table ("nemo_automodel.components.
// quantization.mxfp4", Data: _FP4_E2M1_TABLE) decodes code 8 to +0.0, and a
// code's sign bit stands for x < 0, so -0.0 encodes as code 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) short i16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum : int { FMT_FP8 = 0, FMT_MXFP4 = 1, FMT_NVFP4 = 2 };

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Exact 2^k as an fp32 value for k in [-149, 127] (subnormal below -126).
__device__ __forceinline__ float pow2f(int k) {
  return k >= -126 ? as_f32((uint32_t)(k + 127) << 23) : as_f32(1u << (k + 149));
}

// E8M0 byte -> fp32 scale 2^(b-127); 0xFF is NaN (float8_e8m0fnu).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 255u ? as_f32(0x7FC00000u) : pow2f((int)b - 127);
}

// ---------------------------------------------------------------- scale rules
// quantize_mxfp4 ("nemo_automodel.components.quantization.mxfp4",
// quantize_mxfp4): e = floor(log2(amax)) - 2, exact, clamped to the E8M0
// range [-127, 127]; an all-zero block takes the bottom of the range.
// amax_bits: fp32 bit pattern of a non-negative finite amax.
__device__ __forceinline__ int floor_rule_exponent(uint32_t amax_bits) {
  int fl;
  if (amax_bits >= 0x00800000u) fl = (int)(amax_bits >> 23) - 127;           // normal
  else if (amax_bits != 0u) fl = (31 - __builtin_clz(amax_bits)) - 149;      // subnormal
  else return -127;
  int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// quantize_cache ("nemo_automodel.components.models.deepseek_v41.quantization",
// quantize_cache and _power_of_two_ceiling): s = 2^k, the power-of-two
// ceiling of max(amax / fmax, 2^-126).  With amax = (1 + m/2^23) 2^E and
// fmax = c 2^j (6 = 1.5*4, 448 = 1.75*256) the ceiling is 2^(E-j) when the
// significand is <= c and 2^(E-j+1) otherwise; the fp32 quotient the page
// forms rounds to the same power of two (no quotient lands within half an ulp
// above a power of two).  nvfp4 clamps to the E4M3 powers 2^-9 .. 2^8.
template <int FMT>
__device__ __forceinline__ int ceil_rule_exponent(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 23) - 127;          // subnormal/zero: E = -127
  const uint32_t m = amax_bits & 0x7FFFFFu;
  int k;
  if (FMT == FMT_FP8) k = E - 8 + (m > 0x600000u ? 1 : 0);   // 448 = 1.75 * 2^8
  else                k = E - 2 + (m > 0x400000u ? 1 : 0);   // 6 = 1.5 * 2^2
  if (k < -126) k = -126;
  if (FMT == FMT_NVFP4) k = k < -9 ? -9 : (k > 8 ? 8 : k);
  return k;
}

// ------------------------------------------------------- lane-group reductions
// Max over aligned groups of L consecutive lanes (L a power of two <= 64),
// by DPP within rows of 16 and cross-row shuffles above that.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (L >= 2) v = max(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v = max(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v = max(v, dpp<0x141>(v));   // row_half_mirror
  if constexpr (L >= 16) v = max(v, dpp<0x140>(v));  // row_mirror
  if constexpr (L >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (L >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// ------------------------------------------------------ sign-of-zero fix-ups
// Eight e2m1 codes in a dword: clear the sign bit of every code whose
// magnitude is 0 (code 8 -> code 0), so it decodes to +0.0 as the table does.
__device__ __forceinline__ uint32_t clear_negzero_codes(uint32_t c) {
  const uint32_t mag = c & 0x77777777u;
  const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;  // bit 3 set iff magnitude != 0
  return mag | (c & nz);
}
// Two 16-bit floats in a dword: turn -0.0 halves into +0.0 (x < 0 is false for -0.0).
__device__ __forceinline__ uint32_t canon_negzero_h2(uint32_t w) {
  const uint32_t mag = w & 0x7FFF7FFFu;
  const uint32_t nz = (mag + 0x7FFF7FFFu) & 0x80008000u;  // bit 15 set iff magnitude != 0
  return mag | (w & nz);
}

// ------------------------------------------------------------ element codecs
// Two 16-bit inputs (one dword) -> two e2m1 codes in byte SEL of `old`.
template <int DT, int SEL>
__device__ __forceinline__ uint32_t enc_fp4_h2(uint32_t old, uint32_t w, float scale) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2_t, w), scale, SEL);
  else
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(old, __builtin_bit_cast(f16x2_t, w), scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t enc_fp4_f2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}
// Byte SEL of `codes` (two e2m1 codes) -> two bf16 / f16 values in a dword.
template <int SEL>
__device__ __forceinline__ uint32_t dec_fp4_bf16x2(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL));
}
template <int SEL>
__device__ __forceinline__ uint32_t dec_fp4_f16x2(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, SEL));
}
// fp8 (E4M3): two inputs -> two codes in 16-bit word WSEL of `old`.
template <bool WSEL>
__device__ __forceinline__ uint32_t enc_fp8_bf16x2(uint32_t old, uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      __builtin_bit_cast(i16x2_t, old), __builtin_bit_cast(bf16x2_t, w), scale, WSEL));
}
template <bool WSEL>
__device__ __forceinline__ uint32_t enc_fp8_f2(uint32_t old, float a, float b, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
      __builtin_bit_cast(i16x2_t, old), a, b, scale, WSEL));
}
template <bool WSEL>
__device__ __forceinline__ uint32_t dec_fp8_bf16x2(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, WSEL));
}
template <bool WSEL>
__device__ __forceinline__ f32x2_t dec_fp8_f2(uint32_t codes, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, scale, WSEL);
}

// 16-bit float pairs <-> fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
// fp32 -> f16 pair, nearest-even (hardware conversion, denormals kept).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const unsigned short lo = __builtin_bit_cast(unsigned short, (_Float16)a);
  const unsigned short hi = __builtin_bit_cast(unsigned short, (_Float16)b);
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Magnitude max of two 16-bit floats held in a dword, per half.
__device__ __forceinline__ uint32_t mag_max_h2(uint32_t acc, uint32_t w) {
  u16x2_t a = __builtin_bit_cast(u16x2_t, acc);
  u16x2_t b = __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

}  // namespace mxq
