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
// Work: one workgroup per 256 padded rows x 64 columns, as four 64-row
// quarters that each resolve their own expert (or weight group).  The tile is
// read with 16-byte loads, 128 contiguous bytes per row, into LDS (bf16).
// Then each wave takes one quarter and each thread one column of it: 4 blocks
// of 16 rows, 32 bytes of codes and a 4-byte scale word.  The four quarters
// of a column fill 128 consecutive bytes of that column's output row (and 16
// scale bytes).  The results are staged by output row in LDS and stored by
// consecutive lanes, eight per 128-byte line.  Stored straight from the
// column threads, each lane's piece was a request of its own, which tripled
// the L2 requests of the row quantizer's bytes.  Padded rows read as zeros.
#include "nvfp4_codec.hpp"

namespace nvfp4moe {
namespace {

typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

constexpr int kColTileRows = 256;  // padded rows per workgroup: 4 quarters of 64
constexpr int kColTileCols = 64;

// Expert offsets (and per-group global scales) kept in LDS up to this many.
constexpr int kColLds = 1025;

// The expert whose padded segment holds padded row pr (grouped layout): the
// last e with poff_e <= pr, offsets clamped to [0, M].  `off` is the LDS
// copy of the offsets or, past kColLds - 1 experts, global memory.
template <typename P>
__device__ int find_padded_segment(P off, int E, int64_t M, int64_t pr) {
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

// Grouped layout: M source rows, padded extent Kp, E experts (UNIFORM:
// false).  Uniform layout: E groups of L rows each (UNIFORM: true).  Work
// tiles T = y * tiles_x + x (x: 256-row tile, y: 64-column tile) are taken
// in a grid-stride loop over XCD-contiguous ranges of T (below); each
// workgroup loads its next tile into registers while it encodes the
// current one from LDS.  Four workgroups per CU (the
// register budget, 128 VGPRs, that holds the prefetched tile without spills;
// the encode loop over a column's four blocks stays rolled to fit it).
template <bool UNIFORM, bool IN_LDS>
__global__ __launch_bounds__(256, 4) void colwise_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                      const int32_t* __restrict__ off, int E, int64_t L,
                                                      const float* __restrict__ amax, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s, float* __restrict__ gscale, int64_t Kp,
                                                      int64_t tiles_x, int64_t tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kColTileRows][kColTileCols];
  // per work tile (two in flight) and quarter: expert (-1: nothing to
  // write), first source row, rows in the segment, segment-relative first row
  __shared__ int64_t seg[2][4][4];
  __shared__ float segg[2][4];  // and its global scale
  // The offsets (grouped) and the groups' global scales, copied once: the
  // per-tile lookups then read no global memory.  A global load there would
  // also wait for the prefetched tile (a wave's memory counter retires in
  // order), so the encode of a tile could not overlap the next one's loads.
  // (IN_LDS: they fit; a template parameter, so that the two kinds of
  // lookup are never merged into one flat access)
  __shared__ int32_t s_off[IN_LDS ? kColLds : 1];
  __shared__ float s_g[IN_LDS ? kColLds : 1];
  const int tid = threadIdx.x;
  const int64_t extent = UNIFORM ? (int64_t)E * L : Kp;
  // outputs: [N][extent / 2] codes, [N][extent / 16] scales (each under 2 GiB)
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, N * (extent / 2)), rs = make_rsrc(s, N * (extent / 16));
  const int ng = UNIFORM ? E : 1;
  if constexpr (IN_LDS) {
    if (!UNIFORM)
      for (int i = tid; i <= E; i += 256) s_off[i] = off[i];
    for (int i = tid; i < ng; i += 256) s_g[i] = global_scale(amax[i]);
  }
  __syncthreads();

  // threads 0..3: the quarters of work tile T
  auto resolve = [&](int64_t T, int buf) {
    const int64_t tx = T % tiles_x;
    const int64_t pr = tx * kColTileRows + 64 * tid;   // the quarter's first padded row
    int64_t e = -1, src0 = 0, cnt = 0, j0 = 0;
    float g = 1.0f;
    if (pr < extent) {
      if (UNIFORM) {
        e = pr / L;
        src0 = e * L;
        cnt = L;
        j0 = pr - src0;
      } else {
        int64_t lo, hi;
        if constexpr (IN_LDS) {
          e = find_padded_segment(s_off, E, M, pr);
          lo = s_off[e];
          hi = s_off[e + 1];
        } else {
          e = find_padded_segment(off, E, M, pr);
          lo = off[e];
          hi = off[e + 1];
        }
        lo = lo < 0 ? 0 : lo > M ? M : lo;
        hi = hi < lo ? lo : hi > M ? M : hi;
        src0 = lo;
        cnt = hi - lo;
        j0 = pr - 64 * (lo / 64 + e);
      }
      if constexpr (IN_LDS)
        g = s_g[UNIFORM ? e : 0];
      else
        g = global_scale(amax[UNIFORM ? e : 0]);
      // the segment's global scale, once (where its first block lies)
      if (T < tiles_x && j0 == 0) gscale[UNIFORM ? e : 0] = g;
      // a gap between padded segments (or before the first): nothing to
      // write (uniform: never)
      if (j0 < 0 || j0 >= (cnt + 63) / 64 * 64) e = -1;
    }
    seg[buf][tid][0] = e;
    seg[buf][tid][1] = src0;
    seg[buf][tid][2] = cnt;
    seg[buf][tid][3] = j0;
    segg[buf][tid] = g;
  };
  // 256 rows x 8 chunks of 16 bytes, 8 per thread; rows past their segment,
  // quarters with nothing to write and columns past N read as zeros
  auto fetch = [&](int64_t T, int buf, uint4 (&r)[8]) {
    const int64_t n0 = (T / tiles_x) * kColTileCols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int rr = c >> 3, ch = c & 7, qt = rr >> 6;
      const int64_t row = seg[buf][qt][3] + (rr & 63), col = n0 + ch * 8;
      r[i] = make_uint4(0u, 0u, 0u, 0u);
      if (seg[buf][qt][0] >= 0 && row < seg[buf][qt][2] && col < N)
        r[i] = *reinterpret_cast<const uint4*>(x + (seg[buf][qt][1] + row) * N + col);
    }
  };

  // Visit number Li -> work tile: Li = 8 j + x is the j-th tile of the x-th
  // of eight contiguous ranges of tiles (a bijection on [0, tiles)).  With a
  // grid that is a multiple of 8, workgroup b stays on XCD b % 8 and all its
  // tiles are in that XCD's range, so the workgroups of one XCD take
  // neighbouring row tiles together: the 16-byte scale pieces that eight
  // neighbouring row tiles write into one 128-byte line of an output row then
  // meet in that XCD's L2 instead of leaving as eight partial lines.
  const int64_t tq = tiles / 8, tr = tiles % 8;
  auto tile_of = [&](int64_t Lx) -> int64_t {
    const int64_t x = Lx % 8, j = Lx / 8;
    return x * tq + (x < tr ? x : tr) + j;
  };
  int64_t Li = blockIdx.x;  // gridDim.x <= tiles: every workgroup has a first tile
  int64_t T = tile_of(Li);
  int buf = 0;
  if (tid < 4) resolve(T, 0);
  __syncthreads();
  uint4 reg[8];
  fetch(T, 0, reg);
  // Three stores that write nothing (past the buffer, dropped): the loop's
  // first wait then finds the same three stores after the loads as on every
  // later iteration, so its count can leave them outstanding.
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_v{0u, 0u, 0u, 0u}, rq, kOOB, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_v{0u, 0u, 0u, 0u}, rq, kOOB + 16, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(0u, rs, kOOB, 0, 0);
  for (; Li < tiles; Li += gridDim.x) {
    const int64_t Ln = Li + gridDim.x;
    T = tile_of(Li);
    const int64_t Tn = Ln < tiles ? tile_of(Ln) : tiles;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(&tile[c >> 3][(c & 7) * 8]) = reg[i];
    }
    if (tid < 4 && Tn < tiles) resolve(Tn, buf ^ 1);
    __syncthreads();  // the tile is in LDS; the next tile's quarters are known
    if (Tn < tiles) fetch(Tn, buf ^ 1, reg);  // in flight while this tile is encoded

    const int64_t tx = T % tiles_x, n0 = (T / tiles_x) * kColTileCols;
    const int qt = tid >> 6, col = tid & 63;   // one wave per quarter
    const int64_t e = seg[buf][qt][0];
    const int64_t n = n0 + col;
    uint32_t codes[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t sw = 0;
    if (e >= 0 && n < N) {
      const float g = segg[buf][qt];
#pragma unroll 1
      for (int b = 0; b < 4; ++b) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __uint_as_float((uint32_t)tile[64 * qt + 16 * b + i][col] << 16);
        uint2 c2;
        uint32_t S;
        quantize_block(v, g, c2, S);
        codes[2 * b] = c2.x;
        codes[2 * b + 1] = c2.y;
        sw |= S << (8 * b);
      }
    }
    // Stage the results by output row (column n) in the tile's LDS: 128 code
    // bytes (quarter qt at byte 32 qt) and 16 scale bytes per column, so that
    // the stores below write whole rows of consecutive bytes -- eight lanes
    // per 128-byte line -- instead of one 16-byte piece per lane per line.
    __syncthreads();  // every thread is done reading the tile
    uint8_t* cst = reinterpret_cast<uint8_t*>(&tile[0][0]);  // [64][128] code bytes
    uint8_t* sst = cst + 64 * 128;                           // [64][16] scale bytes
    reinterpret_cast<uint4*>(cst + col * 128 + 32 * qt)[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    reinterpret_cast<uint4*>(cst + col * 128 + 32 * qt)[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
    *reinterpret_cast<uint32_t*>(sst + col * 16 + 4 * qt) = sw;
    __syncthreads();
    // element (segment e, column n, segment row j) sits at base + n * ld + j;
    // grouped: quarter u's padded rows start at tx * 256 + 64 * u
    auto at = [&](int u, int64_t nn) -> int64_t {
      return UNIFORM ? seg[buf][u][0] * N * L + nn * L + seg[buf][u][3] : nn * Kp + tx * kColTileRows + 64 * u;
    };
    // Every thread issues its three stores; one with nothing to write gets an
    // offset past the buffer and is dropped.  The count is then the same on
    // every path, so the wait for the next tile's loads at the top of the
    // loop leaves these stores outstanding (a conditional store made the
    // compiler wait for everything there).
    // codes: 64 rows x 8 chunks of 16 bytes (chunk c holds half c % 2 of quarter c / 2)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = tid + 256 * p;
      const int r = idx >> 3, c = idx & 7, u = c >> 1;
      const int64_t nn = n0 + r;
      const uint32_t voff = seg[buf][u][0] >= 0 && nn < N ? (uint32_t)(at(u, nn) / 2 + 16 * (c & 1)) : kOOB;
      const uint4 w = *reinterpret_cast<const uint4*>(cst + r * 128 + 16 * c);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4_v{w.x, w.y, w.z, w.w}, rq, voff, 0, 0);
    }
    // scales: 64 rows x 4 words
    {
      const int r = tid >> 2, u = tid & 3;
      const int64_t nn = n0 + r;
      const uint32_t voff = seg[buf][u][0] >= 0 && nn < N ? (uint32_t)(at(u, nn) / 16) : kOOB;
      __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(sst + r * 16 + 4 * u), rs, voff, 0, 0);
    }
    __syncthreads();  // the staging area is read before the next tile lands in LDS
    buf ^= 1;
  }
}

// Workgroups of the column-wise kernel: as many as are resident at once
// (four per CU: 40 KB of LDS and up to 128 VGPRs each), at most one per
// work tile, so that no workgroup starts its share late.
template <bool UNIFORM, bool IN_LDS>
int64_t colwise_grid(int64_t tiles) {
  static int per_cu = 0;
  if (per_cu < 1) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, colwise_kernel<UNIFORM, IN_LDS>, 256, 0) != hipSuccess ||
        occ < 1)
      occ = 1;
    per_cu = occ;
  }
  const int64_t g = (int64_t)device_cu_count() * per_cu;
  return tiles < g ? tiles : g;
}

template <bool UNIFORM, bool IN_LDS>
void colwise_launch(const uint16_t* x, int64_t M, int64_t N, const int32_t* off, int E, int64_t L, const float* amax,
                    uint8_t* q, uint8_t* s, float* gscale, int64_t Kp, int64_t tiles_x, int64_t tiles,
                    hipStream_t st) {
  colwise_kernel<UNIFORM, IN_LDS><<<(unsigned)colwise_grid<UNIFORM, IN_LDS>(tiles), 256, 0, st>>>(
      x, M, N, off, E, L, amax, q, s, gscale, Kp, tiles_x, tiles);
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
  if (N * (Kp / 2) > 0x7FFFFFF0LL) return NVFP4MOE_ESHAPE;  // codes under 2 GiB (32-bit store offsets)
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  const int64_t tiles_x = cdiv(Kp > 0 ? Kp : 1, kColTileRows);
  // Every row tile is visited (also with N == 0: row tile 0 writes the global scale).
  const int64_t tiles = tiles_x * cdiv(N > 0 ? N : 1, kColTileCols);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  if (E + 1 <= kColLds)
    colwise_launch<false, true>(xb, M_total, N, expert_offsets, E, 0, amax_in, q_t, s_t, gscale, Kp, tiles_x, tiles, st);
  else
    colwise_launch<false, false>(xb, M_total, N, expert_offsets, E, 0, amax_in, q_t, s_t, gscale, Kp, tiles_x, tiles,
                                 st);
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
  if (groups * L * (N / 2) > 0x7FFFFFF0LL) return NVFP4MOE_ESHAPE;  // codes under 2 GiB (32-bit store offsets)
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
  const int64_t tiles_x = cdiv(groups * L, kColTileRows);
  const int64_t tiles = tiles_x * cdiv(N, kColTileCols);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  if (groups <= kColLds)
    colwise_launch<true, true>(xb, groups * L, N, nullptr, (int)groups, L, amax, q_t, s_t, gscale, 0, tiles_x, tiles,
                               st);
  else
    colwise_launch<true, false>(xb, groups * L, N, nullptr, (int)groups, L, amax, q_t, s_t, gscale, 0, tiles_x, tiles,
                                st);
  return launch_status();
}
