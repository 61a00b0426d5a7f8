// OCP FP8 E4M3 codes for the exchange payload (device helpers).
//
// "MoE 推理服务工程真相 2026", section 6.3: the all-to-all token data goes as
// FP8 instead of BF16, halving its bytes.  Rows are cut into groups of
// kFp8Group columns; a group is stored as e4m3 codes of x * (448 / amax)
// (zero codes if amax < 2^-100) with the fp32 scale amax / 448 and read back
// as code value * scale.  Every
// step is one fp32 operation with round-to-nearest-even (the division is
// IEEE-correct), so the codes are an exact function of the inputs.
//
// E4M3: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0 holds the
// subnormals m * 2^-9; S.1111.111 is NaN and the largest finite value is
// 1.75 * 2^8 = 448.  Conversions are done in integer/float arithmetic here
// (no conversion instruction) so their rounding is the one stated.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kFp8Group = 128;  // columns per scale
constexpr float kE4m3Max = 448.0f;

// Code of v, |v| <= 448 (callers clamp), round-to-nearest-even.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t mag;
  if (a < 0x1p-6f) {
    // subnormal step 2^-9: a * 512 is exact, rintf rounds half to even; a
    // result of 8 is the code of 2^-6, the smallest normal
    mag = (uint32_t)rintf(a * 512.0f);
  } else {
    // round the fp32 mantissa to 3 bits, half to even; a carry moves into
    // the exponent, which is what the format wants
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    mag = ((((b >> 23) - 127u + 7u) << 3) | ((b >> 20) & 7u));
  }
  return sign | mag;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 7u;
  const float mag = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
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
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = fminf(fmaxf(f[i] * r, -kE4m3Max), kE4m3Max);
    const uint32_t c = e4m3_encode(v);
    if (i < 4) lo |= c << (8 * i);
    else hi |= c << (8 * (i - 4));
  }
  *scale = amax / kE4m3Max;
  return make_uint2(lo, hi);
}

}  // namespace moe
