// MX (microscaling) encoding shared by the MX quantizer and the W4A8
// gate+up epilogue that requantizes H: the E8M0 shared exponent of a block
// and the E4M3 element encoding.  The rule (the published microscaling one;
// the pages do not define MX): for a block with amax a > 0 the shared scale
// is X = 2^(floor(log2 a) - emax) (emax = 8 for E4M3, 2 for E2M1), clamped
// to 2^[-127, 127], and 2^-127 for an all-zero block; every element is V / X
// rounded to nearest even, saturated to 448 (E4M3).
#pragma once

#include "common.hpp"

namespace nvfp4moe {

typedef __attribute__((ext_vector_type(2))) short s16x2_t;

// Unbiased shared exponent of a block with amax a: floor(log2 a) - emax,
// clamped to [-127, 127]; -127 when a == 0 (also when a is an fp32
// subnormal, whose exponent is below -126: the clamp gives -127 there).
template <int EMAX>
__device__ __forceinline__ int shared_exp(float a) {
  if (!(a > 0.0f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(a) - 1 - EMAX;  // a = m * 2^(e+1), m in [0.5, 1)
  return e < -127 ? -127 : e > 127 ? 127 : e;
}

// 4 fp32 values to E4M3 codes (one word, element i in byte i): scaled by
// 2^-se (exact), clamped to +-448 (the format saturates; the converter would
// otherwise overflow), then rounded to nearest even by the hardware
// converter with a unit scale.
__device__ __forceinline__ uint32_t encode4_e4m3(const float* v, int se) {
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = __builtin_ldexpf(v[i], -se);
    r[i] = __builtin_copysignf(fminf(fabsf(s), 448.0f), s);
  }
  s16x2_t p = {0, 0};
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, r[0], r[1], 1.0f, false);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, r[2], r[3], 1.0f, true);
  return __builtin_bit_cast(uint32_t, p);
}

}  // namespace nvfp4moe
