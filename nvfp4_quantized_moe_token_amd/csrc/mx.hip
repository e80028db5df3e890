// MX quantization for the W4A8 variant: MXFP8 (E4M3 elements) activations
// and MXFP4 (E2M1 elements) weights, each 32 consecutive elements along K
// sharing one E8M0 (power-of-two) scale.
//
// The W4A8 activation-precision variant is the one the report's ablation
// sets between W4A16 and W4A4 ("miniTE報告、NVFP4強化学習の安定性を検証",
// third paragraph).  The pages do not define MX; the library follows the
// published microscaling rule: for a block with amax a > 0 the shared scale
// is X = 2^(floor(log2 a) - emax) (emax = 8 for E4M3, 2 for E2M1), clamped to
// 2^[-127, 127], and 2^-127 for an all-zero block; every element is V / X
// rounded to nearest, ties to even, saturated to 448 (E4M3) or 6 (E2M1), its
// sign bit the sign of V.  V / X is a power-of-two scaling, exact in fp32
// except where it falls below the normal range, where the element rounds to
// zero in both formats anyway.
//
// Layout: two lanes per 32-block, each reading 16 consecutive elements (32
// bytes of bf16 or 64 of fp32); the block amax is the max of the pair, taken
// with one lane shuffle.  Codes: 16 bytes (E4M3) or 8 bytes (E2M1) per lane,
// so a wave stores one contiguous run; the even lane of a pair stores the
// scale byte.  The grid covers the tensor once (grid-stride only past the
// launch limit), as the NVFP4 quantizer does.
#include "mx_codec.hpp"

namespace nvfp4moe {
namespace {

// 16 fp32 values of a half-block to E4M3 codes (16 bytes).
__device__ __forceinline__ uint4 encode16_e4m3(const float (&v)[16], int se) {
  return make_uint4(encode4_e4m3(v, se), encode4_e4m3(v + 4, se), encode4_e4m3(v + 8, se), encode4_e4m3(v + 12, se));
}

// 16 fp32 values to E2M1 codes (8 bytes, element 2j in the low nibble of
// pair j): scaled by 2^-se, rounded by the hardware converter with a unit
// scale (RNE, saturating to 6, sign kept).
__device__ __forceinline__ uint2 encode16_e2m1(const float (&v)[16], int se) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#define MXQ_PAIR(I, SEL)                                                                                       \
  w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], __builtin_ldexpf(v[8 * h + (I)], -se),                  \
                                                  __builtin_ldexpf(v[8 * h + (I) + 1], -se), 1.0f, SEL)
    MXQ_PAIR(0, 0);
    MXQ_PAIR(2, 1);
    MXQ_PAIR(4, 2);
    MXQ_PAIR(6, 3);
#undef MXQ_PAIR
  }
  return make_uint2(w[0], w[1]);
}

// One thread per 16-element half-block; half-blocks 2b and 2b+1 (lanes of
// one wave: the count is even) form block b.
template <int NT, bool BF16, bool E4M3>
__global__ __launch_bounds__(NT) void mx_quantize_kernel(const uint4* __restrict__ x, int64_t nhalf,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  constexpr int EMAX = E4M3 ? 8 : 2;
  for (int64_t hb = blockIdx.x * (int64_t)NT + threadIdx.x; hb < nhalf; hb += (int64_t)gridDim.x * NT) {
    float v[16];
    if (BF16) {
      const uint4 w0 = x[2 * hb], w1 = x[2 * hb + 1];
      const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(ws[i]);
        v[2 * i + 1] = bf16_hi(ws[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 w = x[4 * hb + i];
        v[4 * i] = __uint_as_float(w.x);
        v[4 * i + 1] = __uint_as_float(w.y);
        v[4 * i + 2] = __uint_as_float(w.z);
        v[4 * i + 3] = __uint_as_float(w.w);
      }
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));  // the partner half of the block
    const int se = shared_exp<EMAX>(a);
    if (E4M3)
      reinterpret_cast<uint4*>(q)[hb] = encode16_e4m3(v, se);
    else
      reinterpret_cast<uint2*>(q)[hb] = encode16_e2m1(v, se);
    if ((hb & 1) == 0) scales[hb >> 1] = (uint8_t)(se + 127);
  }
}

// MXFP8 (E4M3) quantization fused with the token permutation, by scatter:
// each 16-element half-block of X is read once, encoded once, and its codes
// (and, from the even lane of the pair, its block's scale byte) are written
// to the k permuted rows dest[t*k+j] of its token.  Rows past offsets[E]
// (skipped assignments) are written as zeros, the encoding of a zero row.
// Equal bit for bit to mx_quantize of X followed by the row gathers of the
// codes and of the scales.
template <int NT, bool BF16>
__global__ __launch_bounds__(NT) void mx_quantize_scatter_kernel(const uint4* __restrict__ x, int64_t T, int k,
                                                                 int64_t hpr, const int32_t* __restrict__ dest,
                                                                 const int32_t* __restrict__ offsets, int E,
                                                                 int64_t R, uint4* __restrict__ q,
                                                                 uint8_t* __restrict__ scales) {
  const int64_t nhalf = T * hpr;
  const int64_t tid = blockIdx.x * (int64_t)NT + threadIdx.x, stride = (int64_t)gridDim.x * NT;
  for (int64_t hb = tid; hb < nhalf; hb += stride) {
    const int64_t t = hb / hpr, j = hb - t * hpr;  // token, half-block of its row
    float v[16];
    if (BF16) {
      const uint4 w0 = x[2 * hb], w1 = x[2 * hb + 1];
      const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(ws[i]);
        v[2 * i + 1] = bf16_hi(ws[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 w = x[4 * hb + i];
        v[4 * i] = __uint_as_float(w.x);
        v[4 * i + 1] = __uint_as_float(w.y);
        v[4 * i + 2] = __uint_as_float(w.z);
        v[4 * i + 3] = __uint_as_float(w.w);
      }
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));  // the partner half of the block (hpr is even)
    const int se = shared_exp<8>(a);
    const uint4 codes = encode16_e4m3(v, se);
    for (int jj = 0; jj < k; ++jj) {
      const int32_t r = dest[t * k + jj];
      if (r < 0) continue;
      const int64_t oh = (int64_t)r * hpr + j;
      q[oh] = codes;
      if ((j & 1) == 0) scales[oh >> 1] = (uint8_t)(se + 127);
    }
  }
  int64_t valid = offsets[E];
  valid = valid < 0 ? 0 : valid > R ? R : valid;
  for (int64_t h = valid * hpr + tid; h < R * hpr; h += stride) {
    q[h] = make_uint4(0u, 0u, 0u, 0u);
    if ((h & 1) == 0) scales[h >> 1] = 0;
  }
}

}  // namespace

// Enqueue the MXFP8 quantize-scatter of T token rows of D elements into the
// permuted rows given by dest (metadata already enqueued; D % 32 == 0).
int mx_quantize_scatter_launch(const void* x, int x_dtype, int64_t T, int k, int64_t D, const int32_t* dest,
                               const int32_t* offsets, int E, uint8_t* q, uint8_t* scales, hipStream_t st) {
  constexpr int NT = 256;
  const int64_t R = T * k, hpr = D / 16;
  int64_t grid = cdiv(T * hpr > 0 ? T * hpr : 1, NT);
  if (grid > kMaxStreamGrid) grid = kMaxStreamGrid;
  if (x_dtype == NVFP4MOE_BF16)
    mx_quantize_scatter_kernel<NT, true><<<(unsigned)grid, NT, 0, st>>>(
        reinterpret_cast<const uint4*>(x), T, k, hpr, dest, offsets, E, R, reinterpret_cast<uint4*>(q), scales);
  else
    mx_quantize_scatter_kernel<NT, false><<<(unsigned)grid, NT, 0, st>>>(
        reinterpret_cast<const uint4*>(x), T, k, hpr, dest, offsets, E, R, reinterpret_cast<uint4*>(q), scales);
  return launch_status();
}

// Enqueue the MX quantizer (arguments validated; rows * K > 0).
int mx_quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t K, int elem, uint8_t* q, uint8_t* scales,
                       hipStream_t st) {
  constexpr int NT = 256;
  const int64_t nhalf = rows * (K / 16);
  int64_t grid = cdiv(nhalf, NT);
  if (grid > kMaxStreamGrid) grid = kMaxStreamGrid;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const bool bf = x_dtype == NVFP4MOE_BF16, e4 = elem == NVFP4MOE_MX_E4M3;
  if (bf && e4) mx_quantize_kernel<NT, true, true><<<(unsigned)grid, NT, 0, st>>>(xv, nhalf, q, scales);
  else if (bf) mx_quantize_kernel<NT, true, false><<<(unsigned)grid, NT, 0, st>>>(xv, nhalf, q, scales);
  else if (e4) mx_quantize_kernel<NT, false, true><<<(unsigned)grid, NT, 0, st>>>(xv, nhalf, q, scales);
  else mx_quantize_kernel<NT, false, false><<<(unsigned)grid, NT, 0, st>>>(xv, nhalf, q, scales);
  return launch_status();
}

}  // namespace nvfp4moe

extern "C" int mx_quantize(const void* x, int x_dtype, int64_t rows, int64_t K, int elem, uint8_t* q,
                           uint8_t* scales, nvfp4moe_stream_t stream) {
  using namespace nvfp4moe;
  if (rows < 0 || K < 0) return NVFP4MOE_EINVAL;
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (elem != NVFP4MOE_MX_E4M3 && elem != NVFP4MOE_MX_E2M1) return NVFP4MOE_EINVAL;
  if (rows * K > 0 && (!x || !q || !scales)) return NVFP4MOE_EINVAL;
  if (K % 32 != 0) return NVFP4MOE_ESHAPE;
  if (rows * K > 0 && (!aligned(x, 16) || !aligned(q, elem == NVFP4MOE_MX_E4M3 ? 16 : 8))) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (rows * K == 0) return NVFP4MOE_OK;
  return mx_quantize_launch(x, x_dtype, rows, K, elem, q, scales, as_stream(stream));
}
