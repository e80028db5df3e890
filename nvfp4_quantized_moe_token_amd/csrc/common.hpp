// Shared host/device helpers for the nvfp4moe HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4moe.h"

namespace nvfp4moe {

// ---------------------------------------------------------------- host side
// Returns NVFP4MOE_OK when the current device is gfx950, NVFP4MOE_EARCH
// otherwise.  The answer is cached per device ordinal.
int check_arch();

// Compute units of the current device (cached per device ordinal).
int device_cu_count();

inline hipStream_t as_stream(nvfp4moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NVFP4MOE_OK : NVFP4MOE_ELAUNCH;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int dtype_bytes(int dt) {
  return dt == NVFP4MOE_F32 ? 4 : dt == NVFP4MOE_BF16 ? 2 : dt == NVFP4MOE_U8 ? 1 : 0;
}

// Number of workgroups for grid-stride HBM-bound kernels: enough waves to
// keep every CU busy without a huge tail.
constexpr int kStreamBlocks = 256 * 8;

// Grid limit of the one-pass streaming kernels (quantize, quantize-scatter,
// combine, SiLU backward): they launch one thread (or one workgroup) per
// unit of work and keep a grid-stride loop only for inputs beyond this many
// workgroups of 256 threads (2^28 work-items, below the dispatch's 2^32).
// On MI355X a grid that covers the tensor once streams 13-15% faster than a
// grid capped at a few thousand workgroups that loops (measured on a cold
// 268 MB bf16 quantize: 6.0 against 5.3 TB/s).
constexpr int64_t kMaxStreamGrid = int64_t(1) << 20;

// Grid limit of the streaming kernels that also reduce a max with one
// same-address atomic per workgroup (those serialize: 2048 of them on one
// address cost ~17 us).
constexpr int64_t kAmaxGrid = 256 * 8;

// -------------------------------------------------------------- device side
// Raw buffer resources: accesses at or past `bytes` (or at kOOB) are not
// made -- loads read zeros, stores are dropped.
constexpr uint32_t kOOB = 0x80000000u;       // a buffer offset past every range
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRawBufferWord3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs): the gfx950
// conversion instruction v_cvt_pk_bf16_f32, two values per instruction.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// SiLU gate of one element pair, fp32: silu(g) * u with silu(g) = g / (1 + e^-g)
// evaluated as g * rcp(1 + e^-g) (hardware exp2 and reciprocal, about 1 ulp
// each).  Shared by the standalone SiLU-gate kernels and the fused GEMM
// epilogue so that both produce the same bits.
__device__ __forceinline__ float sigmoid_f32(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_gate(float g, float u) { return g * sigmoid_f32(g) * u; }

// Non-negative floats order like their bit patterns: max-reduce |x| with
// unsigned integer atomics.
__device__ __forceinline__ void atomic_max_abs(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(fabsf(v)));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Block-wide max of non-negative values followed by one atomicMax per block.
// All threads of the block must call it.
template <int NT>
__device__ __forceinline__ void block_atomic_max(float* dst, float v) {
  __shared__ float red[NT / 64];
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i]);
    atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(m));
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n);

// max |x| per row-group (quantize.hip); amax_out is cleared first.
int launch_amax(const void* x, int x_dtype, int64_t n16_per_group, int64_t groups, float* amax_out, hipStream_t st);
// MX quantizer (mx.hip); arguments validated, rows * K > 0.
// MXFP8 quantize-scatter of T token rows into their permuted rows (mx.hip);
// arguments validated, D % 32 == 0, the routing metadata already enqueued.
int mx_quantize_scatter_launch(const void* x, int x_dtype, int64_t T, int k, int64_t D, const int32_t* dest,
                               const int32_t* offsets, int E, uint8_t* q, uint8_t* scales, hipStream_t st);
int mx_quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t K, int elem, uint8_t* q, uint8_t* scales,
                       hipStream_t st);
// The same without clearing amax_out (an earlier launch on the stream did).
int launch_amax_uncleared(const void* x, int x_dtype, int64_t n16_per_group, int64_t groups, float* amax_out,
                          hipStream_t st);

}  // namespace nvfp4moe
