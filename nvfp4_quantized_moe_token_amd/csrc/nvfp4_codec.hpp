// NVFP4 encoding of one 1x16 block: global scale, E4M3 block scale and
// E2M1 codes (device functions shared by the quantizer and the fused
// quantize-scatter of the permutation).
//
// Steps (per block with amax a, global scale g): t = a/6, u = t/g,
// S = E4M3_RNE_satfinite(u), d = decode(S) * g, code = sign(x) |
// E2M1_RNE_satfinite(fl32(|x|/d)).  The format is the one the library
// implements for the NVFP4 of "miniTE ускоряет RL в NVFP4 на B300" (1x16
// blocks along K, E4M3 block scale, FP32 tensor scale, E2M1 elements).
//
// Exactness.  Every step follows the IEEE fp32 definition: t = a/6 and
// u = t/g use correctly rounded division (this file is built without fast
// math and with contraction off).  The element ratio fl32(x/d) is formed as
// RN32(RN64(x * RN64(1/d))): x and d have 24-bit significands, so x/d is
// either exactly representable or at least 2^-49 (relative) away from any
// fp32 rounding midpoint, while the fp64 product is within 2^-52 of x/d;
// rounding it to fp32 therefore gives exactly fl32(x/d).  The E2M1 rounding
// of that fp32 ratio uses the hardware converter with a unit scale (RNE,
// saturating to 6, sign kept, including -0 and +-inf), checked against the
// oracle over every rounding threshold.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

constexpr float kGlobalDiv = 2688.0f;  // 6 * 448

__device__ __forceinline__ float global_scale(float amax) {
  return amax > 0.0f ? amax / kGlobalDiv : 1.0f;
}

// OCP E4M3FN code of u >= 0 (u may be +inf): round to nearest even,
// saturate at 448 (0x7E); subnormal step 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode(float u) {
  u = fminf(u, 448.0f);
  if (u < 0.015625f) return (uint32_t)__builtin_rintf(u * 512.0f);  // 0..8, exact scaling
  uint32_t b = __float_as_uint(u);
  b += 0x7FFFFu + ((b >> 20) & 1u);  // RNE to 3 mantissa bits
  return (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_decode(uint32_t S) { return __builtin_amdgcn_cvt_f32_fp8((int)S, 0); }

// Block scale from the block amax a and global scale g: the E4M3 code S and
// the decode factor d = decode(S) * g (IEEE fp32, correctly rounded).
__device__ __forceinline__ void block_scale(float a, float g, uint32_t& S, float& d) {
  const float t = a / 6.0f;
  const float u = t > 0.0f ? t / g : 0.0f;
  S = e4m3_encode(u);
  d = e4m3_decode(S) * g;
}

// E2M1 codes of 8 values (element 2j in the low nibble of nibble pair j):
// RNE of fl32(v/d), formed as RN32(RN64(v * RN64(1/d))).
__device__ __forceinline__ uint32_t encode8(const float* v, float d) {
  const double inv = d > 0.0f ? 1.0 / (double)d : 0.0;  // d == 0: every ratio becomes +-0
  uint32_t w = 0;
#define NVQ_PAIR(I, SEL)                                                                       \
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, (float)((double)v[I] * inv), (float)((double)v[(I) + 1] * inv), \
                                               1.0f, SEL)
  NVQ_PAIR(0, 0);
  NVQ_PAIR(2, 1);
  NVQ_PAIR(4, 2);
  NVQ_PAIR(6, 3);
#undef NVQ_PAIR
  return w;
}

// Quantize the 16 fp32 values v of one block with global scale g.
__device__ __forceinline__ void quantize_block(const float (&v)[16], float g, uint2& codes, uint32_t& S) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
  float d;
  block_scale(a, g, S, d);
  codes = make_uint2(encode8(v, d), encode8(v + 8, d));
}

}  // namespace nvfp4moe
