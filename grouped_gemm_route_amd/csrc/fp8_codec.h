// OCP FP8 E4M3 codes for the exchange payload (device helpers).
//
// "MoE 推理服务工程真相 2026", section 6.3: the all-to-all token data goes as
// FP8 instead of BF16, halving its bytes.  Rows are cut into groups of
// kFp8Group columns; a group is stored as e4m3 codes of x * (448 / amax)
// (zero codes if amax < 2^-100) with the fp32 scale amax / 448 and read back
// as code value * scale.  Every step is one fp32 operation with
// round-to-nearest-even (the division is IEEE-correct), so the codes are an
// exact function of the inputs.
//
// E4M3: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0 holds the
// subnormals m * 2^-9; S.1111.111 is NaN and the largest finite value is
// 1.75 * 2^8 = 448.  gfx950's conversion instructions (v_cvt_pk_fp8_f32,
// v_cvt_pk_f32_fp8) use this OCP format; encoding rounds to nearest even.
// Inputs are clamped to +-448 first, so no saturation rule is involved.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kFp8Group = 128;  // columns per scale
constexpr float kE4m3Max = 448.0f;

typedef __attribute__((ext_vector_type(2))) float f32x2;

// Codes of (a, b) written into the low or high 16 bits of `old` (high if
// kHigh), the other half kept.
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHigh);
}

// Values of the two codes in the low or high 16 bits of w.
template <bool kHigh>
__device__ __forceinline__ f32x2 e4m3_decode2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHigh);
}

// Quantizes one 16-byte piece (8 bf16 values) of a row whose 16 pieces per
// group sit in 16 consecutive lanes (lane groups aligned to 16): returns the
// 8 codes packed little-endian in a uint2 and the group's scale.
__device__ __forceinline__ uint2 quantize_piece(const uint4 raw, float* scale) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = (float)x[i];
    amax = fmaxf(amax, fabsf(f[i]));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  // groups below 2^-100 (zero, or too small for 448 / amax to stay finite)
  // get zero codes
  const float r = amax >= 0x1p-100f ? kE4m3Max / amax : 0.0f;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(f[i] * r, -kE4m3Max), kE4m3Max);
  uint32_t lo = e4m3_encode2<false>(v[0], v[1], 0u);
  lo = e4m3_encode2<true>(v[2], v[3], lo);
  uint32_t hi = e4m3_encode2<false>(v[4], v[5], 0u);
  hi = e4m3_encode2<true>(v[6], v[7], hi);
  *scale = amax / kE4m3Max;
  return make_uint2(lo, hi);
}

}  // namespace moe
