// NVFP4 quantization: amax reduction and the 1x16-block quantizer.
//
// The scaling scheme and the NVFP4 kernels are where naive FP4 loses its
// speed ("miniTE ускоряет RL в NVFP4 на B300", section "Диагностика,
// выравнивание и быстрые ядра"); the global amax is computed once and
// reused ("miniTE報告、NVFP4強化学習の安定性を検証", fourth paragraph).
//
// Layout: one lane owns one 16-element block: it reads the block (32 bytes
// of bf16 or 64 of fp32), reduces its amax in registers, derives the E4M3
// scale, and writes 8 bytes of codes plus 1 scale byte.  Consecutive lanes
// own consecutive blocks, so the code stores of a wave are one contiguous
// 512-byte run and the loads cover one contiguous 2 KiB (bf16) span.  The
// grid covers the tensor once (one block per thread): with a cold cache
// this moves a 268 MB bf16 tensor at ~6.0 TB/s on MI355X, against ~5.3 TB/s
// for a capped grid-stride loop; two or four blocks per thread, non-temporal
// loads or stores, lane-contiguous loads, shared per-pair scales and deeper
// prefetch all measured slower.
//
#include <stdlib.h>

#include "nvfp4_codec.hpp"

namespace nvfp4moe {
namespace {

__device__ __forceinline__ float amax16(const uint4 w, int is_bf16) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float m = 0.0f;
  if (is_bf16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[j])), fabsf(bf16_hi(ws[j]))));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(__uint_as_float(ws[j])));
  }
  return m;
}

// max |x| of each row-group (blockIdx.y); four independent 16-byte loads in
// flight per thread, one atomic per workgroup.
template <int NT>
__global__ __launch_bounds__(NT) void amax_kernel(const uint4* __restrict__ x, int64_t n16_per_group,
                                                  int is_bf16, float* __restrict__ amax) {
  const uint4* g = x + (int64_t)blockIdx.y * n16_per_group;
  const int64_t stride = (int64_t)gridDim.x * NT;
  float m = 0.0f;
  int64_t i = blockIdx.x * (int64_t)NT + threadIdx.x;
  for (; i + 3 * stride < n16_per_group; i += 4 * stride) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = g[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) m = fmaxf(m, amax16(w[u], is_bf16));
  }
  for (; i < n16_per_group; i += stride) m = fmaxf(m, amax16(g[i], is_bf16));
  block_atomic_max<NT>(&amax[blockIdx.y], m);
}

template <int NT, bool BF16>
__global__ __launch_bounds__(NT) void quantize_kernel(const uint4* __restrict__ x, int64_t nblk, int64_t blk_per_group,
                                                      int64_t groups, const float* __restrict__ amax,
                                                      uint2* __restrict__ q, uint8_t* __restrict__ scales,
                                                      float* __restrict__ gscale) {
  const int64_t tid = blockIdx.x * (int64_t)NT + threadIdx.x;
  for (int64_t i = tid; i < groups; i += (int64_t)gridDim.x * NT) gscale[i] = global_scale(amax[i]);
  for (int64_t b = tid; b < nblk; b += (int64_t)gridDim.x * NT) {
    // The block's loads are issued before the amax read and the global
    // scale's division, so that their latencies overlap.
    float v[16];
    if (BF16) {
      const uint4 w0 = x[2 * b], w1 = x[2 * b + 1];
      const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(ws[i]);
        v[2 * i + 1] = bf16_hi(ws[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 w = x[4 * b + i];
        v[4 * i] = __uint_as_float(w.x);
        v[4 * i + 1] = __uint_as_float(w.y);
        v[4 * i + 2] = __uint_as_float(w.z);
        v[4 * i + 3] = __uint_as_float(w.w);
      }
    }
    const float g = global_scale(amax[groups == 1 ? 0 : b / blk_per_group]);
    uint2 codes;
    uint32_t S;
    quantize_block(v, g, codes, S);
    q[b] = codes;
    scales[b] = (uint8_t)S;
  }
}


// One-pass quantizer of row-groups (expert weights): each group is read
// once, instead of once for its amax and once more to encode it.
//
// A group's 16-element blocks are cut into P slices of kOnePassSliceBlocks
// (kOnePassPerThread consecutive-lane blocks per thread).  The grid holds R
// teams of P workgroups; team i takes groups i, i + R, i + 2R, ...  A
// workgroup loads its slice of a group into registers, reduces its amax and
// publishes it in its own slot of `part` (the slots start at -1, so "not
// yet" and any amax >= 0 differ by sign).  It loads and publishes its slice
// of the team's next group before it waits for the current group's P slots;
// once none is negative, their max is the group's amax, and the slice is
// encoded from the registers that hold it.  No atomics are used: every slot
// has one writer.
//
// The wait is only fast when the whole team is resident; the launch sizes
// R * P to what the occupancy of this kernel allows on the device.  It is
// never needed for correctness: past a bound of kOnePassPollLimit polls (a
// group's slices are normally all published within a few microseconds) the
// workgroup reads the whole group and takes its amax itself, so every wave
// always exits and the results never depend on which workgroups ran at once
// (other work on the device, or two such calls on different streams).
constexpr int kOnePassThreads = 256;
constexpr int kOnePassPerThread = 4;
constexpr int kOnePassSliceBlocks = kOnePassThreads * kOnePassPerThread;
constexpr int kOnePassPollLimit = 4096;

template <bool BF16>
__global__ __launch_bounds__(kOnePassThreads) void quantize_onepass_kernel(
    const uint4* __restrict__ x, int64_t bpg, int64_t groups, int P, int R, float* __restrict__ part,
    float* __restrict__ amax_out, uint2* __restrict__ q, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    int poll_limit) {
  constexpr int NT = kOnePassThreads, NB = kOnePassPerThread, W = BF16 ? 2 : 4;  // 16-byte words per block
  __shared__ float red[NT / 64], red2[NT / 64];
  const int team = blockIdx.x / P, si = blockIdx.x % P;
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int64_t b0 = (int64_t)si * kOnePassSliceBlocks;  // the slice's first block in its group
  // This thread's words of group e's slice.  A block past the group's end
  // reads the group's last block instead, which leaves the group's amax
  // unchanged and is not stored; so every load is issued without a branch.
  auto load = [&](int64_t e, uint4 (&w)[NB][W]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t bl = b0 + j * NT + t;
      const int64_t src = e * bpg + (bl < bpg ? bl : bpg - 1);
#pragma unroll
      for (int u = 0; u < W; ++u) w[j][u] = x[src * W + u];
    }
  };
  // Publish the amax of this workgroup's slice of group e (every thread calls).
  auto publish = [&](int64_t e, const uint4 (&w)[NB][W]) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int u = 0; u < W; ++u) m = fmaxf(m, amax16(w[j][u], BF16));
    m = wave_max(m);
    if (lane == 0) red[wid] = m;
    __syncthreads();
    if (t == 0) {
      float mm = red[0];
#pragma unroll
      for (int i = 1; i < NT / 64; ++i) mm = fmaxf(mm, red[i]);
      __hip_atomic_store(part + e * P + si, mm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // red is read before the next publish writes it
  };
  // A workgroup publishes its slice of the team's next group before it waits
  // for the current one, so the wait has a whole group's time in hand.
  uint4 w[NB][W], wn[NB][W];
  if (team < groups) {
    load(team, w);
    publish(team, w);
  }
  for (int64_t e = team; e < groups; e += R) {
    const int64_t gb = e * bpg;
    if (e + R < groups) {
      load(e + R, wn);
      publish(e + R, wn);
    }
    const float* slots = part + e * P;
    // Wait until every slice of the group has published its amax.
    float v;
    for (int it = 0;; ++it) {
      v = 0.0f;
      if (it >= poll_limit) {
        // the group's amax from the group itself (the same value)
        for (int64_t i = t; i < bpg * W; i += NT) v = fmaxf(v, amax16(x[gb * W + i], BF16));
        break;
      }
      int ready = 1;
      for (int i = t; i < P; i += NT) {
        const float pv = __hip_atomic_load(slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready &= pv >= 0.0f ? 1 : 0;
        v = fmaxf(v, pv);
      }
      if (__syncthreads_and(ready)) break;
      __builtin_amdgcn_s_sleep(4);
    }
    v = wave_max(v);
    if (lane == 0) red2[wid] = v;
    __syncthreads();
    float a = red2[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) a = fmaxf(a, red2[i]);
    const float g = global_scale(a);
    if (si == 0 && t == 0) {
      amax_out[e] = a;
      gscale[e] = g;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t bl = b0 + j * NT + t;
      if (bl < bpg) {
        float vals[16];
#pragma unroll
        for (int u = 0; u < W; ++u) {
          const uint32_t ws[4] = {w[j][u].x, w[j][u].y, w[j][u].z, w[j][u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (BF16) {
              vals[8 * u + 2 * i] = bf16_lo(ws[i]);
              vals[8 * u + 2 * i + 1] = bf16_hi(ws[i]);
            } else {
              vals[4 * u + i] = __uint_as_float(ws[i]);
            }
          }
        }
        uint2 codes;
        uint32_t S;
        quantize_block(vals, g, codes, S);
        q[gb + bl] = codes;
        scales[gb + bl] = (uint8_t)S;
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int u = 0; u < W; ++u) w[j][u] = wn[j][u];
  }
}

}  // namespace

// Enqueue max |x| of each of `groups` equal consecutive parts of n16 16-byte
// words (bf16 or fp32) into amax_out[groups] (cleared first).
int launch_amax(const void* x, int x_dtype, int64_t n16_per_group, int64_t groups, float* amax_out, hipStream_t st) {
  fill_u32_kernel<<<(unsigned)cdiv(groups, 256), 256, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, groups);
  return launch_amax_uncleared(x, x_dtype, n16_per_group, groups, amax_out, st);
}

// The same into an amax_out that an earlier launch on the stream cleared.
int launch_amax_uncleared(const void* x, int x_dtype, int64_t n16_per_group, int64_t groups, float* amax_out,
                          hipStream_t st) {
  constexpr int NT = 1024;
  if (n16_per_group > 0) {
    // At most ~256 workgroups of 1024 threads in all: every workgroup ends
    // in one atomic on its group's amax, and same-address atomics serialize
    // (2048 of them cost ~17 us on a 33 MB tensor, measured).  On that
    // tensor 256 x 1024 threads take 12 us against 15 us for 512 x 256; on
    // the expert weights (128 groups) the two shapes run alike.
    int64_t bx = cdiv(n16_per_group, NT * 4);
    const int64_t cap = groups >= 256 ? 1 : 256 / groups;
    if (bx > cap) bx = cap;
    amax_kernel<NT><<<dim3((unsigned)bx, (unsigned)groups), NT, 0, st>>>(
        reinterpret_cast<const uint4*>(x), n16_per_group, x_dtype == NVFP4MOE_BF16, amax_out);
  }
  return launch_status();
}

// Enqueue the quantizer (and the amax reduction when amax_in is NULL).
// Arguments are already validated.
static int quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t groups,
                           const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales, float* gscale,
                           hipStream_t st) {
  constexpr int NT = 256;
  const int64_t rpg = rows / groups;
  const float* amax = amax_in;
  if (!amax_in) {
    const int rc = launch_amax(x, x_dtype, rpg * K * dtype_bytes(x_dtype) / 16, groups, amax_out, st);
    if (rc != NVFP4MOE_OK) return rc;
    amax = amax_out;
  }
  const int64_t nblk = rows * (K / 16);
  const int64_t work = nblk > groups ? nblk : groups;
  int64_t grid = cdiv(work, NT);
  if (grid > kMaxStreamGrid) grid = kMaxStreamGrid;
  const int64_t bpg = rpg * (K / 16) > 0 ? rpg * (K / 16) : 1;
  if (x_dtype == NVFP4MOE_BF16)
    quantize_kernel<NT, true><<<(unsigned)grid, NT, 0, st>>>(reinterpret_cast<const uint4*>(x), nblk, bpg, groups,
                                                             amax, reinterpret_cast<uint2*>(q), scales, gscale);
  else
    quantize_kernel<NT, false><<<(unsigned)grid, NT, 0, st>>>(reinterpret_cast<const uint4*>(x), nblk, bpg, groups,
                                                              amax, reinterpret_cast<uint2*>(q), scales, gscale);
  return launch_status();
}


// Slices per group of the one-pass quantizer.
static int64_t onepass_slices(int64_t rows, int64_t K, int64_t groups) {
  const int64_t bpg = rows / groups * (K / 16);
  return bpg > 0 ? cdiv(bpg, kOnePassSliceBlocks) : 0;
}

// Workgroups of the one-pass quantizer that may run at once on the current
// device (cached per device ordinal).
static int onepass_capacity(bool bf16) {
  static int cache[2][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& c = cache[bf16 ? 1 : 0][dev];
  if (c == 0) {
    int per_cu = 0;
    const hipError_t rc = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                     &per_cu, quantize_onepass_kernel<true>, kOnePassThreads, 0)
                               : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                     &per_cu, quantize_onepass_kernel<false>, kOnePassThreads, 0);
    c = rc == hipSuccess && per_cu > 0 ? per_cu * device_cu_count() : -1;
  }
  return c;
}

static int quantize_onepass_launch(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t groups,
                                   float* amax_out, uint8_t* q, uint8_t* scales, float* gscale, void* workspace,
                                   hipStream_t st) {
  const bool bf16 = x_dtype == NVFP4MOE_BF16;
  const int64_t P = onepass_slices(rows, K, groups);
  const int cap = P > 0 ? onepass_capacity(bf16) : 0;
  // Empty groups, or groups too large for a team to be resident: the
  // two-pass quantizer (amax pass, then the encoder).
  if (P == 0 || cap <= 0 || P > cap)
    return quantize_launch(x, x_dtype, rows, K, groups, nullptr, amax_out, q, scales, gscale, st);
  int64_t R = cap / P;
  if (R > groups) R = groups;
  float* part = reinterpret_cast<float*>(workspace);
  fill_u32_kernel<<<(unsigned)cdiv(groups * P, 256), 256, 0, st>>>(reinterpret_cast<uint32_t*>(part), 0xBF800000u,
                                                                   groups * P);  // -1.0f: not yet published
  const int64_t bpg = rows / groups * (K / 16);
  // NVFP4MOE_ONEPASS_POLL_LIMIT overrides the wait's bound (tests force the
  // path that reads the whole group with 0)
  int poll_limit = kOnePassPollLimit;
  if (const char* env = getenv("NVFP4MOE_ONEPASS_POLL_LIMIT")) poll_limit = atoi(env);
  if (bf16)
    quantize_onepass_kernel<true><<<(unsigned)(R * P), kOnePassThreads, 0, st>>>(
        reinterpret_cast<const uint4*>(x), bpg, groups, (int)P, (int)R, part, amax_out,
        reinterpret_cast<uint2*>(q), scales, gscale, poll_limit);
  else
    quantize_onepass_kernel<false><<<(unsigned)(R * P), kOnePassThreads, 0, st>>>(
        reinterpret_cast<const uint4*>(x), bpg, groups, (int)P, (int)R, part, amax_out,
        reinterpret_cast<uint2*>(q), scales, gscale, poll_limit);
  return launch_status();
}

}  // namespace nvfp4moe

extern "C" int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t groups,
                              const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales, float* gscale,
                              int32_t* status, nvfp4moe_stream_t stream) {
  using namespace nvfp4moe;
  (void)status;
  if (rows < 0 || K < 0 || groups < 1) return NVFP4MOE_EINVAL;
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!gscale || (!amax_in && !amax_out)) return NVFP4MOE_EINVAL;
  if (rows * K > 0 && (!x || !q || !scales)) return NVFP4MOE_EINVAL;
  if (K % 16 != 0 || rows % groups != 0) return NVFP4MOE_ESHAPE;
  if (rows * K > 0 && (!aligned(x, 16) || !aligned(q, 8))) return NVFP4MOE_ESHAPE;
  if (!aligned(gscale, 4) || (amax_in && !aligned(amax_in, 4)) || (amax_out && !aligned(amax_out, 4)))
    return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  return quantize_launch(x, x_dtype, rows, K, groups, amax_in, amax_out, q, scales, gscale, as_stream(stream));
}


extern "C" size_t nvfp4_quantize_onepass_workspace_size(int64_t rows, int64_t K, int64_t groups) {
  using namespace nvfp4moe;
  if (rows < 0 || K < 0 || groups < 1 || K % 16 != 0 || rows % groups != 0) return 0;
  return (size_t)(groups * onepass_slices(rows, K, groups)) * sizeof(float);
}

extern "C" int nvfp4_quantize_onepass(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t groups,
                                      float* amax_out, uint8_t* q, uint8_t* scales, float* gscale, void* workspace,
                                      size_t workspace_bytes, nvfp4moe_stream_t stream) {
  using namespace nvfp4moe;
  if (rows < 0 || K < 0 || groups < 1) return NVFP4MOE_EINVAL;
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!gscale || !amax_out) return NVFP4MOE_EINVAL;
  if (rows * K > 0 && (!x || !q || !scales)) return NVFP4MOE_EINVAL;
  if (K % 16 != 0 || rows % groups != 0) return NVFP4MOE_ESHAPE;
  if (rows * K > 0 && (!aligned(x, 16) || !aligned(q, 8))) return NVFP4MOE_ESHAPE;
  if (!aligned(gscale, 4) || !aligned(amax_out, 4)) return NVFP4MOE_ESHAPE;
  const size_t need = nvfp4_quantize_onepass_workspace_size(rows, K, groups);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVFP4MOE_EWORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  return quantize_onepass_launch(x, x_dtype, rows, K, groups, amax_out, q, scales, gscale, workspace,
                                 as_stream(stream));
}
