// Device helpers shared by the quantize / dequantize / GEMM kernels (gfx950).
//
// Numerics follow the format definitions of aisyndicate.ch "FP4 auf
// Blackwell" (section "Was NVFP4 von frueheren 4-Bit-Formaten
// unterscheidet") and pimento.cloud "FP8, NVFP4 czy AWQ?" (section "Czym
// roznia sie FP8, NVFP4, MXFP4 i AWQ?"): E2M1 elements, E4M3 / E8M0 block
// scales, FP32 tensor scale.  Every translation unit that includes this
// file is compiled with -ffp-contract=off and IEEE fp32 division and
// denormals, so each expression below rounds exactly once per operation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// ---- bit casts -------------------------------------------------------------
__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// bf16 pair in one dword -> two fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// ---- cross-lane (DPP quad permutes; all lanes of the quad must be active) --
// quad_perm [1,0,3,2]: partner lane ^ 1;  [2,3,0,1]: partner lane ^ 2.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return as_f((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u(v), CTRL, 0xF, 0xF, true));
}

// ---- E4M3 (scale byte, non-negative) --------------------------------------
// Nearest E4M3 value to u >= 0 with ties to the even code, saturating at 448
// (code 0x7E); never NaN.  Subnormal grid step 2^-9 below 2^-6.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float u) {
  if (!(u < 448.0f)) return 0x7Eu;                 // includes +inf
  if (u < 0.015625f) {                             // below 2^-6
    return (uint32_t)__builtin_rintf(u * 512.0f);  // exact scaling, RNE; 8 -> 0x08
  }
  uint32_t b = as_u(u);
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);    // RNE to 3 mantissa bits
  return (r >> 20) - (120u << 3);                  // exponent bias 127 -> 7
}

// E4M3 code 0..126 -> its fp32 value (exact).
__device__ __forceinline__ float e4m3_decode_pos(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  return e ? as_f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Any E4M3 byte -> its fp32 value: sign in bit 7, S.1111.111 is NaN (the
// format has no infinity).  Every kernel that reads caller-supplied NVFP4
// block-scale bytes decodes them through this (or through the hardware
// fp8 conversion, which has the same rule).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const float v = ((c & 0x7Fu) == 0x7Fu) ? __builtin_nanf("") : e4m3_decode_pos(c & 0x7Fu);
  return (c & 0x80u) ? -v : v;
}

// ---- E2M1 ------------------------------------------------------------------
// Two fp32 -> two E2M1 codes (round to nearest even, ties to the even code,
// saturating at 6, sign of zero kept) written into byte `SEL` of `old`.
// With scale 1.0 the hardware conversion divides by 2^0; it was checked
// against the nearest-even definition on every tie, its fp32 neighbours,
// subnormals, +-0 and values beyond 6.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Byte SEL of `w` (two E2M1 codes) -> two fp32 values (scale 1: exact).
template <int SEL>
__device__ __forceinline__ v2f e2m1_unpack2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// ---- FP8 E4M3 output --------------------------------------------------------
// Four fp32 values -> four E4M3 bytes, round to nearest even after a clamp to
// +-448 (the hardware conversion rounds correctly inside that range but
// returns NaN beyond it).
__device__ __forceinline__ uint32_t pack_e4m3x4(const float* y) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(y[i], -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (uint32_t)w;
}

// Block scale byte -> its fp32 value.  NVFP4 (NV = true): E4M3 with its
// sign, 0x7F / 0xFF NaN.  MXFP4: E8M0 2^(c-127), the byte 0 giving 2^-127,
// 0xFF NaN.
template <bool NV>
__device__ __forceinline__ float block_scale_value(uint32_t sbyte) {
  if (NV) return e4m3_decode(sbyte);
  if (sbyte == 0xFFu) return __builtin_nanf("");
  return sbyte ? as_f(sbyte << 23) : as_f(0x00400000u);
}

// ---- MXFP4 block exponent --------------------------------------------------
// Smallest k with a <= 6 * 2^k for a > 0, clamped to [-127, 127].  With
// a = 1.f * 2^(E-127) = m * 2^e, m in [0.5, 1), e = E - 126: k = e - 3 when
// m <= 0.75 (mantissa field <= 0x400000), else e - 2.  A subnormal a has
// E = 0 and always lands on the clamp -127.
__device__ __forceinline__ int mx_block_exponent(float a) {
  uint32_t b = as_u(a);
  int E = (int)(b >> 23);
  int k = E - 129 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

}  // namespace fp4dev
