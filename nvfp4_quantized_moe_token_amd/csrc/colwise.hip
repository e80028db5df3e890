// Column-wise NVFP4 quantization: the reduction operands of the NVFP4
// backward variant's weight-gradient GEMMs (blocks of 16 consecutive rows of
// one column inside each expert's row segment), and the expert weights
// quantized along their input dimension for its data-gradient GEMMs.
//
// The NVFP4 backward is this library's reading of the headline learner
// speed-up of "miniTE ускоряет RL в NVFP4 на B300" (intro, key-facts list)
// as including quantized backward GEMMs; the learner of "miniTE報告、NVFP4強化
// 学習の安定性を検証" (first paragraph) keeps its backward in BF16, which is
// this library's default.
//
// Output layouts (codes two per byte along the reduction, element 2j in the
// low nibble; one E4M3 scale byte per 16):
//  * grouped (activations): q_t [N][Kp/2], s_t [N][Kp/16]; expert e's
//    segment starts at column poff_e = 64 * (floor(off_e / 64) + e) and is
//    zero-padded to a multiple of 64, which never reaches poff_{e+1}; one
//    global scale for the tensor.
//  * uniform (weights [E][L][N]): q_t [E][N][L/2], s_t [E][N][L/16]; one
//    global scale per expert.
// The encoding of each block is the row quantizer's (nvfp4_codec.hpp), on
// the same fp32 values, so a segment's codes equal those of the row
// quantizer applied to its transpose.
//
// Work: one workgroup per 64 padded rows x 256 columns.  The tile is read
// with 16-byte row-contiguous loads into LDS (bf16), then each thread takes
// one column: 4 blocks of 16 rows, 32 bytes of codes and a 4-byte scale word
// written to that column's output row.  Padded rows read as zeros.
#include "nvfp4_codec.hpp"

namespace nvfp4moe {
namespace {

constexpr int kColTileRows = 64;
constexpr int kColTileCols = 256;

// The expert whose padded segment holds padded row pr (grouped layout): the
// last e with poff_e <= pr, offsets clamped to [0, M].
__device__ int find_padded_segment(const int32_t* __restrict__ off, int E, int64_t M, int64_t pr) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    int64_t o = off[mid];
    o = o < 0 ? 0 : o > M ? M : o;
    const int64_t p = 64 * (o / 64 + mid);
    if (p <= pr)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__global__ void fill_gscale_kernel(const float* __restrict__ amax, float* __restrict__ g, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) g[i] = global_scale(amax[i]);
}

template <bool UNIFORM>
__global__ __launch_bounds__(256) void colwise_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                      const int32_t* __restrict__ off, int E, int64_t L,
                                                      const float* __restrict__ amax, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s, float* __restrict__ gscale, int64_t Kp) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kColTileRows][kColTileCols];
  __shared__ int64_t seg[4];  // expert, first source row, rows in the segment, segment-relative first row
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;              // 64-row tile of the padded row space
  const int64_t n0 = (int64_t)blockIdx.y * kColTileCols;
  if (tid == 0) {
    if (UNIFORM) {
      const int64_t tps = L / kColTileRows;
      seg[0] = t / tps;
      seg[1] = seg[0] * L;
      seg[2] = L;
      seg[3] = (t % tps) * kColTileRows;
    } else {
      const int e = find_padded_segment(off, E, M, t * kColTileRows);
      int64_t lo = off[e], hi = off[e + 1];
      lo = lo < 0 ? 0 : lo > M ? M : lo;
      hi = hi < lo ? lo : hi > M ? M : hi;
      seg[0] = e;
      seg[1] = lo;
      seg[2] = hi - lo;
      seg[3] = t * kColTileRows - 64 * (lo / 64 + e);
    }
  }
  __syncthreads();
  const int e = (int)seg[0];
  const int64_t src0 = seg[1], cnt = seg[2], j0 = seg[3];
  const float g = global_scale(amax[UNIFORM ? e : 0]);
  if (tid == 0 && blockIdx.y == 0 && j0 == 0) gscale[UNIFORM ? e : 0] = g;
  const int64_t padded = (cnt + 63) / 64 * 64;
  if (j0 >= padded) return;  // a gap between padded segments: nothing to write (uniform: never)

  // Load: 64 rows x 32 chunks of 16 bytes, 8 per thread; rows past the
  // segment and columns past N read as zeros.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 5, ch = c & 31;
    const int64_t row = j0 + r, col = n0 + ch * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < cnt && col < N) v = *reinterpret_cast<const uint4*>(x + (src0 + row) * N + col);
    *reinterpret_cast<uint4*>(&tile[r][ch * 8]) = v;
  }
  __syncthreads();

  const int64_t n = n0 + tid;
  if (n >= N) return;
  uint32_t codes[8];
  uint32_t sw = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __uint_as_float((uint32_t)tile[16 * b + i][tid] << 16);
    uint2 c2;
    uint32_t S;
    quantize_block(v, g, c2, S);
    codes[2 * b] = c2.x;
    codes[2 * b + 1] = c2.y;
    sw |= S << (8 * b);
  }
  // element (segment e, column n, segment row j) sits at base + n * ld + j
  const int64_t base = UNIFORM ? (int64_t)e * N * L : 64 * (src0 / 64 + e);
  const int64_t ld = UNIFORM ? L : Kp;
  uint8_t* qd = q + (base + n * ld + j0) / 2;
  reinterpret_cast<uint4*>(qd)[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
  reinterpret_cast<uint4*>(qd)[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
  *reinterpret_cast<uint32_t*>(s + (base + n * ld + j0) / 16) = sw;
}

}  // namespace
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" int nvfp4_quantize_colwise(const void* x, int x_dtype, int64_t M_total, int64_t N,
                                      const int32_t* expert_offsets, int E, const float* amax_in, uint8_t* q_t,
                                      uint8_t* s_t, float* gscale, int64_t Kp, nvfp4moe_stream_t stream) {
  if (M_total < 0 || N < 0 || E < 1 || Kp < 0) return NVFP4MOE_EINVAL;
  if (x_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!expert_offsets || !amax_in || !gscale) return NVFP4MOE_EINVAL;
  if (N > 0 && (!q_t || !s_t || (M_total > 0 && !x))) return NVFP4MOE_EINVAL;
  if (N % 8 != 0 || Kp % 64 != 0 || Kp < 64 * (M_total / 64 + (int64_t)E)) return NVFP4MOE_ESHAPE;
  if (!aligned(x, 16) || !aligned(q_t, 16) || !aligned(s_t, 4) || !aligned(gscale, 4)) return NVFP4MOE_ESHAPE;
  if (M_total > 0x7FFFFFFFLL || Kp / 64 > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  const int64_t tiles = Kp / 64 > 0 ? Kp / 64 : 1;
  const int64_t ny = cdiv(N > 0 ? N : 1, kColTileCols);
  if (ny > 65535) return NVFP4MOE_ESHAPE;
  // Every tile is launched (also with N == 0: tile 0 writes the global scale).
  colwise_kernel<false><<<dim3((unsigned)tiles, (unsigned)ny), 256, 0, st>>>(
      reinterpret_cast<const uint16_t*>(x), M_total, N, expert_offsets, E, 0, amax_in, q_t, s_t, gscale, Kp);
  return launch_status();
}

extern "C" int nvfp4_quantize_transposed(const void* x, int x_dtype, int64_t groups, int64_t L, int64_t N,
                                         const float* amax_in, float* amax_out, uint8_t* q_t, uint8_t* s_t,
                                         float* gscale, nvfp4moe_stream_t stream) {
  if (groups < 1 || L < 0 || N < 0) return NVFP4MOE_EINVAL;
  if (x_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!gscale || (!amax_in && !amax_out)) return NVFP4MOE_EINVAL;
  if (L * N > 0 && (!x || !q_t || !s_t)) return NVFP4MOE_EINVAL;
  if (L % 64 != 0 || N % 8 != 0) return NVFP4MOE_ESHAPE;
  if (!aligned(x, 16) || !aligned(q_t, 16) || !aligned(s_t, 4) || !aligned(gscale, 4) ||
      (amax_in && !aligned(amax_in, 4)) || (amax_out && !aligned(amax_out, 4)))
    return NVFP4MOE_ESHAPE;
  if (groups * (L / 64) > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  const float* amax = amax_in;
  if (!amax_in) {
    const int rc = launch_amax(x, NVFP4MOE_BF16, L * N * 2 / 16, groups, amax_out, st);
    if (rc != NVFP4MOE_OK) return rc;
    amax = amax_out;
  }
  if (L == 0 || N == 0) {
    // no blocks: only the global scales
    fill_gscale_kernel<<<(unsigned)cdiv(groups, 256), 256, 0, st>>>(amax, gscale, groups);
    return launch_status();
  }
  const int64_t ny = cdiv(N, kColTileCols);
  if (ny > 65535) return NVFP4MOE_ESHAPE;
  colwise_kernel<true><<<dim3((unsigned)(groups * (L / 64)), (unsigned)ny), 256, 0, st>>>(
      reinterpret_cast<const uint16_t*>(x), groups * L, N, nullptr, (int)groups, L, amax, q_t, s_t, gscale, 0);
  return launch_status();
}
