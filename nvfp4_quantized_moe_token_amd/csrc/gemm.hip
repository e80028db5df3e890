// Grouped GEMMs over the contiguous per-expert layout: the W4A4 (NVFP4 x
// NVFP4) forward GEMM and the BF16 GEMMs of the backward pass.
//
// Grouped GEMM for MoE experts: "miniTE ускоряет RL в NVFP4 на B300",
// section "Диагностика, выравнивание и быстрые ядра"; on the token-wise NVFP4
// path with device-side metadata: "miniTE報告、NVFP4強化学習の安定性を検証",
// fourth paragraph; BF16 backward: same page, first paragraph.
//
// Design (gfx950).  NVFP4's per-16 E4M3 scales cannot be expressed in the
// gfx950 scaled-MFMA format (one power-of-two E8M0 scale per 32 values), and
// an E2M1 x E4M3 product has up to 6 significant bits, so it is exact in
// fp16 (range 2^-10 .. 2688) but not in fp8.  The W4A4 kernel therefore
// moves only packed codes and scale bytes (0.5625 B per element) from HBM
// into LDS; each wave expands the fragments it feeds to the MFMA exactly to
// fp16 in registers (hardware E2M1 decode with a unit scale, then one packed
// fp16 multiply by the block scale) and runs fp16 MFMA 32x32x16 with fp32
// accumulation.  The two global scales are applied in the fp32 epilogue.
//
// Data movement.  Every operand tile goes HBM -> LDS by buffer loads that
// write LDS directly (16 bytes per lane), so no registers stage the tiles
// and out-of-range rows/columns read as zeros (buffer range checks).  A ring
// of S LDS stages keeps S-1 K-steps in flight; each step waits for its own
// loads (s_waitcnt vmcnt) and one workgroup barrier.  Tile layouts in LDS:
//  * K-major bf16 tiles (rows x 64 k): 128-byte rows, 16-byte chunks
//    XOR-swizzled by row; fragments are ds_read_b128.
//  * MN-major bf16 tiles (64 k x columns, as stored in HBM): rows of the
//    reduction index, chunks XOR-swizzled by (row mod 4); fragments are
//    read transposed with ds_read_b64_tr_b16 (two per fragment).
//  * NVFP4 tiles (rows x 256 k): 128 bytes of codes per row, swizzled like
//    the K-major bf16 rows, and the row's 16 scale bytes.  In each 64-k
//    group, lane half h of an MFMA takes the 32 codes k in [32h, 32h+32),
//    8 per MFMA, for A and B alike (a fixed permutation of the reduction
//    order), so one ds_read_b128 feeds 4 MFMAs.
//
// Scheduling.  The host knows only the total row count, so the kernel is
// persistent: the grid is (CUs x resident workgroups), rounded to a multiple
// of the 8 XCDs.  Each workgroup counts the real tiles from the device
// offsets (a wave-wide prefix sum over experts), and the tiles are dealt to
// XCDs in 8 contiguous equal ranges (workgroup b runs on XCD b % 8), so
// consecutive tiles -- the n-tiles of one row block, the row blocks of one
// expert -- share that XCD's L2.  Row-grouped layouts (NT, NN, W4A4) order
// tiles by (expert row block, n-tile); TN tiles are (expert, k-tile, n-tile)
// and reduce over the expert's rows.  The expert offsets are copied to LDS
// at kernel start (up to 1024 experts) for the per-tile lookups.  The plain
// W4A4 GEMM with bf16 output also loads the next tile's first stage during
// the current tile's last step (see the kernel).
#include "mx_codec.hpp"
#include "nvfp4_codec.hpp"

namespace nvfp4moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int BK = 64;                       // reduction elements per MFMA group / bf16 stage
#ifndef NVFP4MOE_GEMM_NMAJOR
#define NVFP4MOE_GEMM_NMAJOR 1
#endif
constexpr bool kNMajor = NVFP4MOE_GEMM_NMAJOR;  // tile order within an expert (find_tile)
constexpr int NV_KS = 256;                   // reduction elements per NVFP4 stage
constexpr int MX_KS = 128;                   // reduction elements per MX (W4A8) stage

// W4A4_SILU: the W4A4 gate+up GEMM with the SiLU-gate epilogue.  W4A8:
// MXFP8 activations x MXFP4 weights on the scaled MFMA (W4A8_SILU: with the
// SiLU-gate epilogue).
// W4A4_SILU_Q: W4A4_SILU that also requantizes H to NVFP4 in the epilogue
// (its own instantiation, so that the plain SiLU-gate kernel keeps its
// registers).  W4A8_SILU_Q: W4A8_SILU that quantizes H to MXFP8 in the
// epilogue (no global scale, so no amax is needed first).
// W4A4_TN: the NVFP4 weight gradient, C_e = A_e^T . B_e reduced over the
// rows of expert e, both operands quantized column-wise (stored transposed:
// K-major rows whose reduction index runs over the expert's padded segment).
// W4A4_B: the same NVFP4 product by scale factoring onto the fp4 scaled MFMA
// (one 16-element block per MFMA, unit E8M0 scales, the E4M3 block-scale
// products applied to each partial sum in fp32) -- the alternative to the
// exact fp16 expansion, kept to measure the two against each other.
enum Mode {
  NT_BF16 = 0, NN_BF16 = 1, TN_BF16 = 2, W4A4 = 3, W4A4_SILU = 4, W4A8 = 5, W4A8_SILU = 6, W4A4_SILU_Q = 7,
  W4A4_TN = 8, W4A4_B = 9, W4A8_SILU_Q = 10
};
constexpr bool is_nv(int mode) {
  return mode == W4A4 || mode == W4A4_SILU || mode == W4A4_SILU_Q || mode == W4A4_TN || mode == W4A4_B;
}
constexpr bool is_tn(int mode) { return mode == TN_BF16 || mode == W4A4_TN; }
constexpr bool is_mx(int mode) { return mode == W4A8 || mode == W4A8_SILU || mode == W4A8_SILU_Q; }
constexpr bool is_q(int mode) { return is_nv(mode) || is_mx(mode); }
constexpr bool is_silu(int mode) {
  return mode == W4A4_SILU || mode == W4A8_SILU || mode == W4A4_SILU_Q || mode == W4A8_SILU_Q;
}

struct Params {
  const void* a;       // NT/NN/TN: bf16 A; W4A4: packed codes of A
  const void* b;       // bf16 B or packed codes of B
  const uint8_t* as;   // W4A4: scales of A
  const uint8_t* bs;   // W4A4: scales of B
  const float* ag;     // W4A4: global scale of A [1]
  const float* bg;     // W4A4: global scales of B [E]
  const int32_t* offsets;
  void* c;
  int64_t M, N, K;     // TN: K = columns of A (rows of C_e); W4A4_TN: K = rows of the transposed A
  int64_t kp;          // W4A4_TN: row length (padded reduction extent) of both transposed operands
  int E;
  int c_f32;
  int accumulate;
  int n_tiles;         // tiles along N
  int k_tiles_tn;      // TN: tiles along K (rows of C_e)
  void* h;             // SiLU-gate modes: H [M][N/2] bf16 (c = Y1 or NULL)
  float* amax;         // SiLU-gate modes: max |H| (cleared before the launch), or NULL
  const int32_t* bsrc; // TN with gathered B: B row of reduction row r is bsrc[r] / bk (none if < 0)
  int bk;
  int bk_shift;        // log2(bk) when bk is a power of two, else -1
  int64_t b_rows;      // TN with gathered B: rows of B
  // W4A4_SILU with H requantized in the epilogue (hq != NULL): NVFP4 codes,
  // scales and global scale of H with the handed-in amax h_amax_in[0].
  // W4A8_SILU_Q: MXFP8 codes (hq, one byte each) and E8M0 scales (hs).
  uint8_t* hq;
  uint8_t* hs;
  float* hg;
  const float* h_amax_in;
};

// ---- small device helpers ----

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wait until at most min(n, MAX) vector memory operations are outstanding
// (n wave-uniform).
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (MAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAX)
      wait_vmcnt<MAX>();
    else
      wait_vmcnt_upto<MAX - 1>(n);
  }
}
constexpr int kMaxEpilogueStores = 32;

// Wait until at most `ahead` steps of NDMA loads each are outstanding
// (ahead in [0, MAX], wave-uniform).
template <int MAX, int NDMA>
__device__ __forceinline__ void wait_steps_ahead(int ahead) {
  if constexpr (MAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAX)
      wait_vmcnt<MAX * NDMA>();
    else
      wait_steps_ahead<MAX - 1, NDMA>(ahead);
  }
}

// One wave-wide LDS-direct load: lane l's `size` bytes land at LDS byte
// address lds + size*l (lds wave-uniform).  Issued as inline assembly so the
// compiler does not make every later LDS read wait for it: the kernel keeps
// the count of its own loads (s_waitcnt vmcnt) and orders LDS with barriers.
// `lds` goes through readfirstlane: under register pressure the compiler may
// hold a uniform value in a vector register, which the scalar operand cannot
// take (a no-op when it is already scalar).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(r)
               : "memory", "m0");
}
// The same with 4 bytes per lane: lane l's word lands at lds + 4*l (probed).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(r)
               : "memory", "m0");
}
// K-major bf16 tile: chunk c (8 elements) of row r at byte r*128 + 16*(c ^ kswz(r)).
__device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 3)) & 7; }
// Swizzle of a K-major tile with ROWB-byte rows (128: kswz; 64: (r / 2) % 4),
// conflict-free for 16-byte reads of the same chunk in 8 consecutive rows.
template <int ROWB>
__device__ __forceinline__ int rswz(int r) {
  if constexpr (ROWB == 128) return kswz(r);
  else return (r >> 1) & 3;
}
// MN-major bf16 tile: chunk c of reduction row k at byte k*rowbytes + 16*(c ^ mswz(k)).
// Any 4 consecutive rows k = 4i..4i+3 then put a transposed read's 32- and
// 64-byte row segments on disjoint banks.
__device__ __forceinline__ int mswz(int k) { return (0xCA60 >> ((k & 3) * 4)) & 15; }  // {0, 6, 10, 12}
// Clamped [lo, hi) row range of expert e.  `off` is the global offsets array
// or its copy in LDS.
typedef __attribute__((address_space(3))) const int32_t lds_i32_t;
template <class OffPtr>
__device__ __forceinline__ void expert_range(OffPtr off, int e, int64_t M, int& lo, int& hi) {
  lo = off[e];
  hi = off[e + 1];
  lo = lo < 0 ? 0 : lo > M ? (int)M : lo;
  hi = hi < lo ? lo : hi > M ? (int)M : hi;
}

// Number of BM-row blocks over all experts.  Runs on one whole wave.
template <int BM>
__device__ int count_row_blocks(const int32_t* __restrict__ off, int E, int64_t M) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int cnt = 0;
    if (e < E) {
      int lo, hi;
      expert_range(off, e, M, lo, hi);
      cnt = (hi - lo + BM - 1) / BM;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    total += cnt;
  }
  return total;
}

// Map row block `slot` to (expert, first row, end row) by a prefix sum of
// per-expert block counts.  Runs on one whole wave; false past the last block.
// Tile L of the row-grouped layouts: its expert, row range and n-tile.  The
// tiles of one expert are numbered n-tile-major when NMAJOR (the expert's
// row blocks that share a weight panel are neighbours, so they run side by
// side on one XCD), row-block-major otherwise.  Tile numbers stay below 2^31
// (checked at launch), so the divisions are 32-bit ones.
template <int BM, bool NMAJOR, class OffPtr>
__device__ bool find_tile(OffPtr off, int E, int64_t M, int64_t L64, int n_tiles, int& e_out,
                          int64_t& r0, int64_t& r1, int& n_out) {
  const int lane = threadIdx.x & 63;
  const uint32_t L = (uint32_t)L64, nt = (uint32_t)n_tiles;
  const uint32_t slot = L / nt;  // the expert's tiles span its row blocks x n_tiles
  uint32_t running = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int lo = 0, hi = 0, cnt = 0;
    if (e < E) {
      expert_range(off, e, M, lo, hi);
      cnt = (hi - lo + BM - 1) / BM;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const uint32_t total = (uint32_t)__shfl(incl, 63, 64);
    if (slot < running + total) {
      const bool mine = slot >= running + incl - cnt && slot < running + incl;
      const uint64_t mask = __ballot(mine);
      const int srcl = __ffsll((unsigned long long)mask) - 1;
      e_out = __shfl(e, srcl, 64);
      const int lo_s = __shfl(lo, srcl, 64), hi_s = __shfl(hi, srcl, 64), ex = __shfl(incl - cnt, srcl, 64);
      const uint32_t cnt_s = (uint32_t)__shfl(cnt, srcl, 64);
      const uint32_t rb0 = running + (uint32_t)ex;  // the expert's first row block
      uint32_t rb;
      if (NMAJOR) {
        const uint32_t t = L - rb0 * nt;
        n_out = (int)(t / cnt_s);
        rb = t % cnt_s;
      } else {
        n_out = (int)(L % nt);
        rb = slot - rb0;
      }
      r0 = lo_s + (int64_t)rb * BM;
      r1 = r0 + BM < hi_s ? r0 + BM : hi_s;
      return true;
    }
    running += total;
  }
  return false;
}

// ---- HBM -> LDS loaders (one pipeline step, this wave's share) ----
//
// Each wave-wide load moves 1 KiB (64 lanes x 16 B) to a contiguous LDS
// range; a lane's 16 bytes are chosen so that the range holds the swizzled
// layout.  Offsets are relative to a range-checked operand region: offsets
// at or past its end, or marked kOOB, read as zeros.

// Gate+up tiles of the SiLU-gate epilogue: tile row r (of 256) is expert row
// gate_f * ((r / 32) % 2) + j0 + 32 * (r / 64) + r % 32, so 32-row granules
// alternate gate and up rows of the same 32 features; each wave's pair of
// adjacent 32-column MFMA blocks then holds matching gate and up columns.
__device__ __forceinline__ int64_t gate_up_row(int r, int64_t gate_f, int64_t j0) {
  return ((r >> 5) & 1) * gate_f + j0 + ((r >> 6) << 5) + (r & 31);
}

// K-major bf16 tile of ROWS rows x ROWB/2 k; row r of the tile is row r of
// the region (or gate_up_row(r) when gate_f > 0), element k0 + k.  `ld` is
// the row pitch in elements.
template <int ROWS, int NW, int ROWB = 128>
struct KMajorLoader {
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
  static constexpr int RPL = 64 / CPR;   // rows per 1 KiB load
  static_assert(ROWS % (RPL * NW) == 0, "K-major tile: rows per wave");
  static constexpr int N_INSTR = ROWS / (RPL * NW);
  __device__ __forceinline__ static void load(uint32_t lds, int wid, __amdgpu_buffer_rsrc_t r, int64_t ld,
                                              int64_t k0, int64_t K, int64_t gate_f = 0, int64_t j0 = 0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N_INSTR; ++i) {
      const int idx = wid + NW * i;
      const int row = idx * RPL + lane / CPR;
      const int c = (lane % CPR) ^ rswz<ROWB>(row);
      const int64_t k = k0 + c * 8;
      const int64_t grow = gate_f > 0 ? gate_up_row(row, gate_f, j0) : row;
      const uint32_t voff = k < K ? (uint32_t)((grow * ld + k) * 2) : kOOB;
      dma16(r, lds + idx * 1024, voff);
    }
  }
};

// MN-major bf16 tile of KR reduction rows x COLS columns; reduction row kr
// is region row (row0 + kr), column n0 + n; `ld` is the row pitch.
template <int COLS, int NW, int KR = 64>
struct MNMajorLoader {
  static_assert(COLS == 128 || COLS == 256, "MN-major tile width");
  static constexpr int CPR = COLS / 8;  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per 1 KiB load
  static_assert((KR / RPI) % NW == 0, "MN-major tile: loads per wave");
  static constexpr int N_INSTR = KR / RPI / NW;
  __device__ __forceinline__ static void load(uint32_t lds, int wid, __amdgpu_buffer_rsrc_t r, int64_t ld,
                                              int64_t row0, int64_t n0, int64_t ncols) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N_INSTR; ++i) {
      const int idx = wid + NW * i;
      const int kr = idx * RPI + lane / CPR;
      const int c = (lane % CPR) ^ mswz(kr);
      const int64_t n = n0 + c * 8;
      const uint32_t voff = n < ncols ? (uint32_t)(((row0 + kr) * ld + n) * 2) : kOOB;
      dma16(r, lds + idx * 1024, voff);
    }
  }
  // The same tile with each reduction row taken from its own row of the
  // region: load i's two rows (lanes 0..31 and 32..63) are src_rows[i][0..1],
  // a negative row reading as zeros.
  __device__ __forceinline__ static void load_rows(uint32_t lds, int wid, __amdgpu_buffer_rsrc_t r, int64_t ld,
                                                   const int32_t (&src_rows)[N_INSTR][2], int64_t n0,
                                                   int64_t ncols) {
    static_assert(RPI == 2, "gathered MN-major rows: two reduction rows per load");
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N_INSTR; ++i) {
      const int idx = wid + NW * i;
      const int kr = idx * RPI + lane / CPR;
      const int c = (lane % CPR) ^ mswz(kr);
      const int64_t n = n0 + c * 8;
      const int32_t row = lane < CPR ? src_rows[i][0] : src_rows[i][1];
      const uint32_t voff = n < ncols && row >= 0 ? (uint32_t)(((int64_t)row * ld + n) * 2) : kOOB;
      dma16(r, lds + idx * 1024, voff);
    }
  }
};

// ---- fragment readers (LDS -> MFMA operands) ----

// K-major bf16 fragment (ROWB-byte rows): rows base + (lane % 32),
// k = 16*kk + 8*(lane/32) + 0..7.
template <int ROWB>
__device__ __forceinline__ bf16x8_t frag_kmajor(const uint8_t* tile, int base, int kk, int lane) {
  const int row = base + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(tile + row * ROWB + ((c ^ rswz<ROWB>(row)) << 4));
}

// MN-major bf16 fragment through two transposed reads: column base +
// (lane % 32), k = 16*kk + 8*(lane/32) + 4*j + 0..3 for read j.  Within a
// 16-lane group, lane 4t+s addresses reduction row (k0 + t), columns
// 4s..4s+3 of the group's 16; the hardware returns to lane i the column i
// of that 4 x 16 block (probed on the device).
template <int COLS>
__device__ __forceinline__ bf16x8_t frag_mnmajor(const uint8_t* tile, int base, int kk, int lane) {
  const int col = base + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  bf16x8_t out;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = 16 * kk + 8 * (lane >> 5) + 4 * j + ((lane & 15) >> 2);
    const int off = kr * (COLS * 2) + (((col >> 3) ^ mswz(kr)) << 4) + ((col & 7) << 1);
    const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off));
    out[4 * j + 0] = v[0];
    out[4 * j + 1] = v[1];
    out[4 * j + 2] = v[2];
    out[4 * j + 3] = v[3];
  }
  return out;
}

// NVFP4 fragment of 64-element chunk c of a stage: the lane's 32 codes (row
// base + lane % 32, k in [64c + 32h, 64c + 32h + 32), h = lane / 32) and its
// two block scales, decoded E4M3 -> fp16 (exact) by one packed conversion.
// Code rows are 128 bytes (16-byte units swizzled like the K-major bf16
// tile), scale rows 16 bytes.
struct NVFrag {
  uint4 q;
  f16x2_t sc;  // scales of blocks 4c+2h (x) and 4c+2h+1 (y)
};
__device__ __forceinline__ NVFrag frag_nv(const uint8_t* codes, const uint8_t* scales, int base, int c, int lane) {
  const int row = base + (lane & 31), h = lane >> 5;
  NVFrag f;
  f.q = *reinterpret_cast<const uint4*>(codes + row * 128 + (((2 * c + h) ^ kswz(row)) << 4));
  const uint32_t s2 = *reinterpret_cast<const uint16_t*>(scales + row * 16 + 4 * c + 2 * h);
  f.sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s2, 1.0f, false);
  return f;
}
__device__ __forceinline__ uint32_t nv_pair(uint32_t w, f16x2_t sc, int sel) {
  f16x2_t v;
  switch (sel) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3); break;
  }
  v = v * sc;  // exact: <= 6 significant bits, inside the fp16 normal range
  return __builtin_bit_cast(uint32_t, v);
}
// MFMA operand kk (k = 32h + 8kk + 0..7): 8 codes expanded exactly to fp16.
__device__ __forceinline__ f16x8_t nv_expand(const NVFrag& f, int kk) {
  const uint32_t w = kk == 0 ? f.q.x : kk == 1 ? f.q.y : kk == 2 ? f.q.z : f.q.w;
  const _Float16 s = kk < 2 ? f.sc.x : f.sc.y;
  const f16x2_t sc = {s, s};
  uint4 o;
  o.x = nv_pair(w, sc, 0);
  o.y = nv_pair(w, sc, 1);
  o.z = nv_pair(w, sc, 2);
  o.w = nv_pair(w, sc, 3);
  return __builtin_bit_cast(f16x8_t, o);
}

// MX (W4A8) fragments of 64-element chunk c of a stage, in the operand
// layouts of the scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (probed on the
// device): for both operands lane l serves row l % 32 and its E8M0 scale
// covers the 32-element block l / 32 of the chunk; a 4-bit operand holds
// k = 32h .. 32h+31 (h = l / 32) in its 16 bytes, an 8-bit operand holds
// k = 16h .. 16h+15 in bytes 0..15 and k = 32+16h .. 32+16h+15 in bytes
// 16..31.
// fp8 A: the 16-byte units 4c + h and 4c + 2 + h of the row's 128 bytes.
__device__ __forceinline__ i32x8_t frag_mx_a(const uint8_t* codes, int base, int c, int lane) {
  const int row = base + (lane & 31), h = lane >> 5;
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(codes + row * 128 + (((4 * c + h) ^ kswz(row)) << 4));
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(codes + row * 128 + (((4 * c + 2 + h) ^ kswz(row)) << 4));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// fp4 B: the 16-byte unit 2c + h of the row's 64 bytes (the operand's upper
// four registers are not read for a 4-bit format).
__device__ __forceinline__ i32x8_t frag_mx_b(const uint8_t* codes, int base, int c, int lane) {
  const int row = base + (lane & 31), h = lane >> 5;
  const i32x4_t v = *reinterpret_cast<const i32x4_t*>(codes + row * 64 + (((2 * c + h) ^ rswz<64>(row)) << 4));
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}
// E8M0 scale of the lane's row and block 2c + h, in byte 0 (the MFMA reads
// byte 0 of the scale register with opsel 0); rows hold 4 bytes per stage.
__device__ __forceinline__ int scale_mx(const uint8_t* sc, int base, int c, int lane) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(sc + (base + (lane & 31)) * 4);
  return (int)(w >> (8 * (2 * c + (lane >> 5))));
}

// Scheduling hint: N_MFMA MFMAs with N_DS LDS reads interleaved one after
// each MFMA (the reads feed the next sub-step), then any reads left over.
template <int N_MFMA, int N_DS>
__device__ __forceinline__ void interleave_mfma_ds() {
  if constexpr (N_MFMA > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (N_DS > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
    interleave_mfma_ds<N_MFMA - 1, (N_DS > 0 ? N_DS - 1 : 0)>();
  } else if constexpr (N_DS > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, N_DS, 0);
  }
}

// Scheduling hint: N_MFMA MFMAs, each followed by up to PER VALU
// instructions (the operand expansion of the next sub-step).
template <int N_MFMA, int PER>
__device__ __forceinline__ void interleave_mfma_valu() {
  if constexpr (N_MFMA > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);  // VALU
    interleave_mfma_valu<N_MFMA - 1, PER>();
  }
}

// Wave-wide loads per pipeline step of one operand tile (A side or B side).
template <int MODE, bool A_SIDE, int ROWS, int NW, int BKB>
constexpr int loads_per_wave() {
  if constexpr (is_nv(MODE))
    return KMajorLoader<ROWS, NW>::N_INSTR;
  else if constexpr (is_mx(MODE))
    return A_SIDE ? KMajorLoader<ROWS, NW>::N_INSTR : KMajorLoader<ROWS, NW, 64>::N_INSTR;
  else if constexpr ((A_SIDE && MODE == TN_BF16) || (!A_SIDE && MODE != NT_BF16))
    return MNMajorLoader<ROWS, NW, BKB>::N_INSTR;
  else
    return KMajorLoader<ROWS, NW, BKB * 2>::N_INSTR;
}

template <int N>
struct IntConst {
  static constexpr int value = N;
};
// Quantized operand regions of a row-grouped tile: A rows [m0, m_end) (codes
// and scales); B the n-tile's rows of the expert (SiLU-gate tiles gather gate
// and up rows: the region runs from the tile's first gate row to the end of
// the expert, so a row's offset in it does not depend on the tile).  Bytes per row: NVFP4 codes
// K/2 and scales K/16 for both operands; MX (W4A8) A codes K (fp8), B codes
// K/2 (fp4), scales K/32 for both.
template <bool MX>
__device__ __forceinline__ void nv_a_regions(const Params& p, int64_t m0, int64_t m_end, __amdgpu_buffer_rsrc_t& ra,
                                             __amdgpu_buffer_rsrc_t& rsa) {
  const int64_t cb = MX ? p.K : p.K / 2, sb = MX ? p.K / 32 : p.K / 16;
  ra = make_rsrc(reinterpret_cast<const uint8_t*>(p.a) + m0 * cb, (m_end - m0) * cb);
  rsa = make_rsrc(p.as + m0 * sb, (m_end - m0) * sb);
}
template <int BN, bool SILU, bool MX>
__device__ __forceinline__ void nv_b_regions(const Params& p, int expert, int64_t n0, __amdgpu_buffer_rsrc_t& rb,
                                             __amdgpu_buffer_rsrc_t& rsb) {
  const int64_t nv = SILU ? p.N - n0 / 2 : p.N - n0 < BN ? p.N - n0 : BN;
  const int64_t brow = (int64_t)expert * p.N + (SILU ? n0 / 2 : n0);
  const int64_t sb = MX ? p.K / 32 : p.K / 16;
  rb = make_rsrc(reinterpret_cast<const uint8_t*>(p.b) + brow * (p.K / 2), nv * (p.K / 2));
  rsb = make_rsrc(p.bs + brow * sb, nv * sb);
}

// ---- the kernel ----

// Two waves per SIMD (at most 256 VGPRs each): one 8-wave workgroup, or two
// 4-wave workgroups per CU (then stated, so the compiler keeps to 256).
template <int MODE, int BM, int BN, int WM, int WN, int S, int BKB, bool OUT32>
__global__ __launch_bounds__(WM* WN * 64, WM* WN == 4 && (BM / WM) * (BN / WN) <= 64 * 128 ? 2 : 1) void gemm_kernel(Params p) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "bad wave tiling");
  constexpr bool NV = is_nv(MODE);
  constexpr bool MX = is_mx(MODE);
  constexpr bool QM = NV || MX;  // quantized operands, row-grouped
  constexpr bool SILU = is_silu(MODE);
  // Reduction elements per pipeline stage: 64 for bf16 (128-byte rows);
  // 256 for NVFP4, so that each row brings a whole 128-byte line of codes
  // and 16 bytes of scales per stage; 128 for MX (W4A8): 128 bytes of fp8
  // codes per A row, 64 bytes of fp4 codes per B row, 4 scale bytes each.
  // bf16 stages hold BKB reduction elements (64: 128-byte K-major rows; 32:
  // 64-byte rows, for deeper rings in the same LDS).
  static_assert(!QM || BKB == 64, "quantized stages use 128-byte A code rows");
  constexpr int KS = NV ? NV_KS : MX ? MX_KS : BKB;
  constexpr int A_BYTES = BM * BKB * 2;
  constexpr int B_BYTES = MX ? BN * 64 : BN * BKB * 2;
  constexpr int SC_ROW = NV ? 16 : MX ? 4 : 0;             // scale bytes per row and stage
  constexpr int SC_BYTES = (BM + BN) * SC_ROW;             // A scales then B scales
  constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  static_assert(!QM || (BM + BN) % (64 * NW) == 0, "quantized scales: rows per wave");
  constexpr int SC_INSTR = QM ? (BM + BN) / (64 * NW) : 0;
  // Per-wave loads per step, for the vmcnt waits.
  constexpr int A_INSTR = loads_per_wave<MODE, true, BM, NW, BKB>();
  constexpr int B_INSTR = loads_per_wave<MODE, false, BN, NW, BKB>();
  // TN: one 4-byte load per step of the gathered-B row indices (out of
  // range, i.e. nothing, when B is not gathered), so the count is fixed.
  constexpr int NIDX = MODE == TN_BF16 ? 1 : 0;
  constexpr int NDMA = A_INSTR + B_INSTR + SC_INSTR + NIDX;
  static_assert(S >= 2 && S <= 8 && NDMA * (S - 2) <= 63, "pipeline depth");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];
  __shared__ int64_t s_tile[5];  // tile lookup: expert, rows, -, n-tile; [3]: row-block count
  // TN with gathered B: per wave and ring slot, the bsrc entries of the
  // wave's B rows of that step (4 used of each 256-byte landing area).
  __shared__ __attribute__((aligned(256))) int32_t gidx[MODE == TN_BF16 ? NW * S * 64 : 1];
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(const lds_void_t*)smem;  // LDS byte address

  // Real tile count, then this XCD's contiguous share of it.
  int64_t total;
  if (is_tn(MODE)) {
    total = (int64_t)p.E * p.k_tiles_tn * p.n_tiles;
  } else {
    if (wid == 0) {
      const int blocks = count_row_blocks<BM>(p.offsets, p.E, p.M);
      if (lane == 0) s_tile[3] = blocks;
    }
    lds_barrier();
    total = s_tile[3] * p.n_tiles;
  }
  const int xcd = blockIdx.x & 7;
  const int64_t t_end = total * (xcd + 1) / 8, t_step = gridDim.x >> 3;

  float silu_amax = 0.0f;  // W4A4_SILU: this lane's max |H| over its tiles

  // Quantized stages: a lane's byte offsets in the regions of a tile are the
  // same for every tile and step (A and B regions start at the tile's first
  // rows; a step adds a fixed number of bytes per row), so they are computed
  // once.  NVFP4 code bytes past the reduction's end are loaded unmasked:
  // they land in the chunks of the last stage that the MFMA loop skips
  // (MX stages are always whole), and every byte past a region still reads
  // as zero.
  constexpr int NVA = QM ? KMajorLoader<BM, NW>::N_INSTR : 1;
  constexpr int NVB = NV ? KMajorLoader<BN, NW>::N_INSTR : MX ? KMajorLoader<BN, NW, 64>::N_INSTR : 1;
  uint32_t nv_oa[NVA], nv_ob[NVB], nv_os[SC_INSTR > 0 ? SC_INSTR : 1];
  if constexpr (MX) {
    const int64_t gf = SILU ? p.N / 2 : 0;
    // fp8 A: K bytes per row (128-byte chunk rows); fp4 B: K/2 bytes per row
    // (64-byte chunk rows); E8M0 scales: K/32 bytes per row.
#pragma unroll
    for (int i = 0; i < NVA; ++i) {
      constexpr int RPL = KMajorLoader<BM, NW>::RPL, CPR = KMajorLoader<BM, NW>::CPR;
      const int row = (wid + NW * i) * RPL + lane / CPR;
      nv_oa[i] = (uint32_t)(row * p.K + (((lane % CPR) ^ kswz(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NVB; ++i) {
      constexpr int RPL = KMajorLoader<BN, NW, 64>::RPL, CPR = KMajorLoader<BN, NW, 64>::CPR;
      const int row = (wid + NW * i) * RPL + lane / CPR;
      const int64_t grow = gf > 0 ? gate_up_row(row, gf, 0) : row;
      nv_ob[i] = (uint32_t)(grow * (p.K / 2) + (((lane % CPR) ^ rswz<64>(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < SC_INSTR; ++i) {
      const int idx = wid + NW * i;
      const bool is_a = idx * 64 < BM;
      const int row = (is_a ? idx * 64 : idx * 64 - BM) + lane;
      nv_os[i] = (uint32_t)((!is_a && gf > 0 ? gate_up_row(row, gf, 0) : row) * (p.K / 32));
    }
  } else if constexpr (NV) {
    const int64_t rowb = MODE == W4A4_TN ? p.kp / 2 : p.K / 2;  // code bytes per row
    const int64_t sld = MODE == W4A4_TN ? p.kp / 16 : p.K / 16;  // scale bytes per row
    const int64_t gf = SILU ? p.N / 2 : 0;
    constexpr int RPL = KMajorLoader<BM, NW>::RPL, CPR = KMajorLoader<BM, NW>::CPR;
#pragma unroll
    for (int i = 0; i < NVA; ++i) {
      const int row = (wid + NW * i) * RPL + lane / CPR;
      nv_oa[i] = (uint32_t)(row * rowb + (((lane % CPR) ^ kswz(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NVB; ++i) {
      const int row = (wid + NW * i) * RPL + lane / CPR;
      const int64_t grow = gf > 0 ? gate_up_row(row, gf, 0) : row;
      nv_ob[i] = (uint32_t)(grow * rowb + (((lane % CPR) ^ kswz(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < SC_INSTR; ++i) {
      const int idx = wid + NW * i;
      const bool is_a = idx * 64 < BM;
      const int row = (is_a ? idx * 64 : idx * 64 - BM) + lane;
      nv_os[i] = (uint32_t)((!is_a && gf > 0 ? gate_up_row(row, gf, 0) : row) * sld);
    }
  }

  // Plain W4A4 with bf16 output (PF): the next tile's first stage is loaded
  // during the current tile's last step, into the ring slot that step does
  // not read, and the epilogue stages its results through the other slot.
  // The next tile then starts on data already in flight, and its first wait
  // lets the previous epilogue's stores stay outstanding (they were issued
  // after those loads, and a wave's memory counter retires in order).  Each
  // wave finds the next tile itself from a copy of the offsets in LDS, so
  // no vector load (whose wait would also wait for the stores) runs in
  // between.  With the SiLU-gate epilogue and in the NN layout the same
  // scheme raised register spills and measured slower, so they keep the
  // plain loop.
  constexpr bool PF = MODE == W4A4 && !OUT32 && S == 2;
  // The SiLU-gate kernels prefetch the same way, right after the k-loop
  // instead of during the last step (which raised register spills), and
  // stage their epilogue through the slot of the tile's last stage.
  constexpr bool PF2 = (MODE == W4A4_SILU || MODE == W4A4_SILU_Q) && S == 2;
  constexpr bool PFX = PF || PF2;
  // Every layout keeps a copy of the expert offsets in LDS (up to 1024
  // experts), so the per-tile lookups read LDS rather than global memory.
  constexpr int kOffLds = 1025;
  __shared__ int32_t s_off[kOffLds];
  const bool off_in_lds = p.E < kOffLds;
  const bool pf_on = PFX && off_in_lds;
  if (off_in_lds) {
    for (int i = threadIdx.x; i <= p.E; i += NW * 64) s_off[i] = p.offsets[i];
    __syncthreads();
  }
  lds_i32_t* off_lds = (lds_i32_t*)s_off;
  int slot0 = 0;            // ring slot of this tile's stage 0
  bool pre = false;         // this tile's stage 0 is in flight (loaded during the previous tile)
  int nst = 0;              // global stores this wave issued after that prefetch
  int nx_e = -1, nx_nt = 0; // the next tile, found during the last step
  int64_t nx_r0 = 0, nx_r1 = 0;
  for (int64_t L = total * xcd / 8 + (blockIdx.x >> 3); L < t_end; L += t_step) {
    int expert;
    int64_t m0, m_end;  // output rows (row-grouped) or C_e rows (TN)
    int64_t n0;
    int64_t red;        // reduction length
    int lo = 0;         // TN: first row of the expert
    int64_t poff = 0;   // W4A4_TN: the expert's first column in the transposed operands
    lds_barrier();      // previous tile: every wave is done with LDS and s_tile
    if (is_tn(MODE)) {
      // 32-bit divisions: tile numbers stay below 2^31 (checked at launch)
      const uint32_t per_e = (uint32_t)(p.k_tiles_tn * p.n_tiles);
      expert = (int)((uint32_t)L / per_e);
      const int rem = (int)((uint32_t)L % per_e);
      m0 = (int64_t)(rem / p.n_tiles) * BM;
      m_end = p.K;
      n0 = (int64_t)(rem % p.n_tiles) * BN;
      int hi;
      if (off_in_lds)
        expert_range(off_lds, expert, p.M, lo, hi);
      else
        expert_range(p.offsets, expert, p.M, lo, hi);
      red = hi - lo;
      if (MODE == W4A4_TN) {
        // the segment is zero-padded to a multiple of 64 columns
        poff = 64 * ((int64_t)lo / 64 + expert);
        red = (red + 63) / 64 * 64;
      }
    } else if (PFX && pre) {
      // Found (and its first stage loaded) during the previous tile.
      expert = nx_e;
      m0 = nx_r0;
      m_end = nx_r1;
      n0 = (int64_t)nx_nt * BN;
      red = p.K;
    } else {
      if (wid == 0) {
        int e = -1, nt = 0;
        int64_t r0 = 0, r1 = 0;
        const bool ok = off_in_lds ? find_tile<BM, kNMajor>(off_lds, p.E, p.M, L, p.n_tiles, e, r0, r1, nt)
                                   : find_tile<BM, kNMajor>(p.offsets, p.E, p.M, L, p.n_tiles, e, r0, r1, nt);
        if (lane == 0) {
          s_tile[0] = ok ? e : -1;
          s_tile[1] = r0;
          s_tile[2] = r1;
          s_tile[4] = nt;
        }
      }
      lds_barrier();
      if (s_tile[0] < 0) break;  // uniform: only when offsets changed under the kernel
      expert = (int)s_tile[0];
      m0 = s_tile[1];
      m_end = s_tile[2];
      n0 = s_tile[4] * BN;
      red = p.K;
    }

    // Operand regions of this tile (range-checked buffers).
    __amdgpu_buffer_rsrc_t ra = make_rsrc(nullptr, 0), rb = ra, rsa = ra, rsb = ra;
    if constexpr (MODE == NT_BF16 || MODE == NN_BF16) {
      ra = make_rsrc(reinterpret_cast<const uint16_t*>(p.a) + m0 * p.K, (m_end - m0) * p.K * 2);
    } else if constexpr (MODE == TN_BF16) {
      ra = make_rsrc(reinterpret_cast<const uint16_t*>(p.a) + (int64_t)lo * p.K, red * p.K * 2);
    } else if constexpr (MODE == W4A4_TN) {
      // rows m0.. of the transposed A from column poff: codes kp/2 and
      // scales kp/16 bytes per row
      ra = make_rsrc(reinterpret_cast<const uint8_t*>(p.a) + m0 * (p.kp / 2) + poff / 2,
                     (p.K - m0) * (p.kp / 2) - poff / 2);
      rsa = make_rsrc(p.as + m0 * (p.kp / 16) + poff / 16, (p.K - m0) * (p.kp / 16) - poff / 16);
    } else {
      nv_a_regions<MX>(p, m0, m_end, ra, rsa);
    }
    if constexpr (MODE == NT_BF16) {
      const int64_t nv = p.N - n0 < BN ? p.N - n0 : BN;
      rb = make_rsrc(reinterpret_cast<const uint16_t*>(p.b) + ((int64_t)expert * p.N + n0) * p.K, nv * p.K * 2);
    } else if constexpr (MODE == NN_BF16) {
      rb = make_rsrc(reinterpret_cast<const uint16_t*>(p.b) + (int64_t)expert * p.K * p.N, p.K * p.N * 2);
    } else if constexpr (MODE == TN_BF16) {
      rb = p.bsrc ? make_rsrc(p.b, p.b_rows * p.N * 2)
                  : make_rsrc(reinterpret_cast<const uint16_t*>(p.b) + (int64_t)lo * p.N, red * p.N * 2);
    } else if constexpr (MODE == W4A4_TN) {
      rb = make_rsrc(reinterpret_cast<const uint8_t*>(p.b) + n0 * (p.kp / 2) + poff / 2,
                     (p.N - n0) * (p.kp / 2) - poff / 2);
      rsb = make_rsrc(p.bs + n0 * (p.kp / 16) + poff / 16, (p.N - n0) * (p.kp / 16) - poff / 16);
    } else {
      nv_b_regions<BN, SILU, MX>(p, expert, n0, rb, rsb);
    }
    const int64_t gate_f = SILU ? p.N / 2 : 0;
    const int64_t j0 = n0 / 2;

    // TN: bsrc entries of this wave's B rows of step s (rows (wid + NW i) * 2
    // + h, lane 2i + h) into ring slot s % S; out of range when B is not
    // gathered or past the expert's rows.
    using BLoad = MNMajorLoader<BN, NW, BKB>;
    const __amdgpu_buffer_rsrc_t rix = make_rsrc(p.bsrc, p.bsrc ? p.M * 4 : 0);
    auto index_load = [&](int64_t s) {
      const int i = lane >> 1, h = lane & 1;
      const int64_t rr = s * BKB + (wid + NW * i) * 2 + h;
      const uint32_t voff = lane < 2 * BLoad::N_INSTR && rr < red ? (uint32_t)((lo + rr) * 4) : kOOB;
      dma4(rix, (uint32_t)(uintptr_t)(const lds_void_t*)gidx + (wid * S + (int)(s % S)) * 256, voff);
    };
    // One quantized stage (codes and scales of A and B) of a tile with the
    // given regions into the LDS stage at byte address st.
    auto nv_load = [&](__amdgpu_buffer_rsrc_t ra_, __amdgpu_buffer_rsrc_t rb_, __amdgpu_buffer_rsrc_t rsa_,
                       __amdgpu_buffer_rsrc_t rsb_, int64_t k0, uint32_t st) {
      if constexpr (MX) {
        // fp8 A codes: 128 bytes (128 elements) per row, a K-major tile of
        // 64 16-bit units per row; fp4 B codes: 64 bytes per row; E8M0
        // scales: 4 bytes per row (one word), 64 rows per load, A rows first.
        // A step adds k0 A, k0/2 B and k0/32 scale bytes.
#pragma unroll
        for (int i = 0; i < NVA; ++i) dma16(ra_, st + (wid + NW * i) * 1024, nv_oa[i] + (uint32_t)k0);
#pragma unroll
        for (int i = 0; i < NVB; ++i) dma16(rb_, st + A_BYTES + (wid + NW * i) * 1024, nv_ob[i] + (uint32_t)(k0 / 2));
#pragma unroll
        for (int i = 0; i < SC_INSTR; ++i) {
          const int idx = wid + NW * i;
          dma4(idx * 64 < BM ? rsa_ : rsb_, st + A_BYTES + B_BYTES + idx * 256, nv_os[i] + (uint32_t)(k0 / 32));
        }
      } else {
        // Codes: 128 bytes (256 elements) per row, laid out like a K-major
        // bf16 tile of 64 16-bit units per row; scales: 16 bytes per row, 64
        // rows per load, A rows first.  The lanes' offsets are nv_oa, nv_ob
        // and nv_os; a step adds k0/2 code and k0/16 scale bytes.
        const uint32_t kc = (uint32_t)(k0 / 2), ksc = (uint32_t)(k0 / 16);
#pragma unroll
        for (int i = 0; i < NVA; ++i) dma16(ra_, st + (wid + NW * i) * 1024, nv_oa[i] + kc);
#pragma unroll
        for (int i = 0; i < NVB; ++i) dma16(rb_, st + A_BYTES + (wid + NW * i) * 1024, nv_ob[i] + kc);
#pragma unroll
        for (int i = 0; i < SC_INSTR; ++i) {
          const int idx = wid + NW * i;
          dma16(idx * 64 < BM ? rsa_ : rsb_, st + A_BYTES + B_BYTES + idx * 1024, nv_os[i] + ksc);
        }
      }
    };
    auto load_step = [&](int64_t kt, int stage) {
      const uint32_t st = smem_lds + stage * STAGE;
      // The step's first reduction element, kept opaque to induction-variable
      // rewriting: per-lane offsets carried across the k-loop started from
      // spill reloads before it, and the compiler then guarded every step
      // with a wait that also drained the LDS-direct loads in flight, which
      // it does not count.
      const int64_t k0 = (int64_t)__builtin_amdgcn_readfirstlane((int)(kt * KS));
      if constexpr (MODE == NT_BF16) {
        KMajorLoader<BM, NW, BKB * 2>::load(st, wid, ra, p.K, k0, p.K);
        KMajorLoader<BN, NW, BKB * 2>::load(st + A_BYTES, wid, rb, p.K, k0, p.K);
      } else if constexpr (MODE == NN_BF16) {
        KMajorLoader<BM, NW, BKB * 2>::load(st, wid, ra, p.K, k0, p.K);
        MNMajorLoader<BN, NW, BKB>::load(st + A_BYTES, wid, rb, p.N, k0, n0, p.N);
      } else if constexpr (MODE == TN_BF16) {
        MNMajorLoader<BM, NW, BKB>::load(st, wid, ra, p.K, k0, m0, p.K);
        if (p.bsrc) {
          const int32_t* ix = gidx + (wid * S + (int)(kt % S)) * 64;
          int32_t rows[BLoad::N_INSTR][2];
#pragma unroll
          for (int i = 0; i < BLoad::N_INSTR; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int32_t v = ix[2 * i + h];
              const int32_t t = p.bk_shift >= 0 ? v >> p.bk_shift : v / p.bk;
              rows[i][h] = k0 + (wid + NW * i) * 2 + h < red && v >= 0 ? t : -1;
            }
          BLoad::load_rows(st + A_BYTES, wid, rb, p.N, rows, n0, p.N);
        } else {
          BLoad::load(st + A_BYTES, wid, rb, p.N, k0, n0, p.N);
        }
        index_load(kt + S - 1);
      } else {
        nv_load(ra, rb, rsa, rsb, k0, st);
      }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (red + KS - 1) / KS;
    // A wave whose rows all lie past the expert's end (the last row block
    // of an expert is partly empty) skips its MFMAs; it still loads and
    // takes part in every barrier.
    int n_active = FM;
    if (!is_tn(MODE) && m_end - m0 <= wm * WTM) n_active = 0;
    if (MODE == TN_BF16 && p.bsrc) {
      // Row indices of the first S - 1 steps (the wave's own LDS area).
#pragma unroll
      for (int s = 0; s < S - 1; ++s) index_load(s);
      wait_vmcnt<0>();
    }
    // PF: the global scales are read with scalar loads (constant address
    // space), so that no vector-memory wait -- which would also wait for the
    // previous epilogue's stores or the prefetched stage -- comes from them.
    float alpha_t = 1.0f;
    if constexpr (PFX) {
      typedef __attribute__((address_space(4))) const float const_f32_t;
      const_f32_t* ag = (const_f32_t*)p.ag;
      const_f32_t* bg = (const_f32_t*)p.bg;
      alpha_t = ag[0] * bg[__builtin_amdgcn_readfirstlane(expert)];
    }
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk && !(PFX && pre && s == 0)) load_step(s, (slot0 + s) % S);
    bool pre_next = false;
    // Find the next tile (every wave, from the LDS offsets) and load its
    // first stage into ring slot (slot0 + nk) % S.
    auto prefetch_next = [&]() {
      int e = -1, nt = 0;
      int64_t r0 = 0, r1 = 0;
      const bool ok = find_tile<BM, kNMajor>(off_lds, p.E, p.M, L + t_step, p.n_tiles, e, r0, r1, nt);
      // The lookup is wave-uniform; say so, so that the regions stay scalar.
      if (__builtin_amdgcn_readfirstlane(ok ? 1 : 0) != 0) {
        nx_e = __builtin_amdgcn_readfirstlane(e);
        nx_nt = __builtin_amdgcn_readfirstlane(nt);
        nx_r0 = uniform64(r0);
        nx_r1 = uniform64(r1);
        __amdgpu_buffer_rsrc_t na, nb, nsa, nsb;
        nv_a_regions<MX>(p, nx_r0, nx_r1, na, nsa);
        nv_b_regions<BN, SILU, MX>(p, nx_e, (int64_t)nx_nt * BN, nb, nsb);
        nv_load(na, nb, nsa, nsb, 0, smem_lds + (uint32_t)((slot0 + nk) % S) * STAGE);
        pre_next = true;
      }
    };

    for (int64_t kt = 0; kt < nk; ++kt) {
      // This wave's loads for step kt are done once at most `ahead` later
      // steps' loads are outstanding; the barrier then makes every wave's
      // loads visible and frees the stage read in the previous step.  A
      // prefetched first stage is followed only by the previous epilogue's
      // nst stores, which may stay outstanding.
      const int64_t ahead = nk - 1 - kt < S - 2 ? nk - 1 - kt : S - 2;
      if (PFX && pre && kt == 0)
        wait_vmcnt_upto<kMaxEpilogueStores>(nst);
      else
        wait_steps_ahead<S - 2, NDMA>((int)ahead);
      lds_barrier();
      // TN issues the next stage's loads after its first MFMA sub-step rather
      // than here.  Right after the barrier all eight waves issue their loads
      // at once, and the waves queued behind the others start their MFMAs
      // late (2-3% on the TN GEMMs; no gain on NN and NT, and the NVFP4 loop
      // spills when the load state stays live into its chunks).
      constexpr bool kLateLoads = MODE == TN_BF16;
      bool loads_issued = false;
      if (!kLateLoads && kt + S - 1 < nk) load_step(kt + S - 1, (int)((slot0 + kt + S - 1) % S));
      if constexpr (PF) {
        // Last step: find the next tile (every wave, from the LDS offsets)
        // and load its first stage into the slot this step does not read.
        if (pf_on && kt == nk - 1 && L + t_step < t_end) prefetch_next();
      }

      const uint8_t* st = smem + (int)((slot0 + kt) % S) * STAGE;
      // One step of MFMAs over the first NA fragment rows of this wave.
      auto compute = [&](auto na_tag) {
        constexpr int NA = decltype(na_tag)::value;
        if constexpr (NA > 0) {
          if constexpr (MODE == W4A4_B) {
            // Per 64-element chunk c and 16-element block j of it: the lane
            // half h = j / 2 holds the block in half j % 2 of its 16 code
            // bytes (the NVFP4 stage layout is the fp4 MFMA's operand
            // layout); everything else is masked to zero, so the MFMA (unit
            // scales) returns the block's exact partial sums, which are
            // scaled by sA[m][b] * sB[n][b] and accumulated in fp32.
            const int64_t k_left = red - kt * KS;
            const int nchunk = k_left >= KS ? KS / BK : (int)(k_left / BK);
            const uint8_t* sca = st + A_BYTES + B_BYTES;
            const int h = lane >> 5;
#pragma unroll
            for (int c = 0; c < KS / BK; ++c) {
              if (c < nchunk) {
                uint4 qa[NA], qb[FN];
                float sa[NA][4];
#pragma unroll
                for (int i = 0; i < NA; ++i) {
                  const int row = wm * WTM + i * 32 + (lane & 31);
                  qa[i] = *reinterpret_cast<const uint4*>(st + row * 128 + (((2 * c + h) ^ kswz(row)) << 4));
                  const uint32_t w = *reinterpret_cast<const uint32_t*>(sca + row * 16 + 4 * c);
#pragma unroll
                  for (int j = 0; j < 4; ++j) sa[i][j] = e4m3_decode((w >> (8 * j)) & 0xFF);
                }
#pragma unroll
                for (int jf = 0; jf < FN; ++jf) {
                  const int row = wn * WTN + jf * 32 + (lane & 31);
                  qb[jf] = *reinterpret_cast<const uint4*>(st + A_BYTES + row * 128 + (((2 * c + h) ^ kswz(row)) << 4));
                }
#pragma unroll
                for (int jf = 0; jf < FN; ++jf) {
                  // B scale words of the 16 result rows n = 8g + 4(l/32) + r%4 this lane holds
                  uint32_t bw[16];
#pragma unroll
                  for (int r = 0; r < 16; ++r) {
                    const int n = wn * WTN + jf * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    bw[r] = *reinterpret_cast<const uint32_t*>(sca + BM * 16 + n * 16 + 4 * c);
                  }
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    const bool mine = h == (j >> 1);
                    const uint32_t lo = (j & 1) == 0;
                    i32x8_t ob;
                    ob[0] = mine && lo ? (int)qb[jf].x : 0;
                    ob[1] = mine && lo ? (int)qb[jf].y : 0;
                    ob[2] = mine && !lo ? (int)qb[jf].z : 0;
                    ob[3] = mine && !lo ? (int)qb[jf].w : 0;
                    ob[4] = ob[5] = ob[6] = ob[7] = 0;
                    float sb[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) sb[r] = e4m3_decode((bw[r] >> (8 * j)) & 0xFF);
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                      i32x8_t oa;
                      oa[0] = mine && lo ? (int)qa[i].x : 0;
                      oa[1] = mine && lo ? (int)qa[i].y : 0;
                      oa[2] = mine && !lo ? (int)qa[i].z : 0;
                      oa[3] = mine && !lo ? (int)qa[i].w : 0;
                      oa[4] = oa[5] = oa[6] = oa[7] = 0;
                      f32x16_t z;
#pragma unroll
                      for (int r = 0; r < 16; ++r) z[r] = 0.0f;
                      const f32x16_t part =
                          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ob, oa, z, 4, 4, 0, 127, 0, 127);
                      // the lane's result column is its A row m = l % 32: its scale is per lane
                      const float s_a = sa[i][j];
#pragma unroll
                      for (int r = 0; r < 16; ++r) acc[i][jf][r] = fmaf(part[r], s_a * sb[r], acc[i][jf][r]);
                    }
                  }
                }
              }
            }
          } else if constexpr (NV) {
            // 64-element chunks of this stage inside the reduction (a multiple of 64).
            const int64_t k_left = red - kt * KS;
            const int nchunk = k_left >= KS ? KS / BK : (int)(k_left / BK);
#pragma unroll
            for (int c = 0; c < KS / BK; ++c) {
              if (c < nchunk) {
                // Issue priority falls with the chunk index, so of the two
                // waves sharing a SIMD the one behind in the stage issues
                // first.  At equal priority the older wave always wins, runs
                // its stage ahead and then waits at the barrier while the
                // other finishes alone, and a lone wave keeps the MFMA pipe
                // only about two-thirds busy (W4A4 GEMMs 3-6% faster).
                switch (c) {
                  case 0: __builtin_amdgcn_s_setprio(3); break;
                  case 1: __builtin_amdgcn_s_setprio(2); break;
                  case 2: __builtin_amdgcn_s_setprio(1); break;
                  default: __builtin_amdgcn_s_setprio(0); break;
                }
                NVFrag fa[NA], fb[FN];
#pragma unroll
                for (int i = 0; i < NA; ++i) fa[i] = frag_nv(st, st + A_BYTES + B_BYTES, wm * WTM + i * 32, c, lane);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  fb[j] = frag_nv(st + A_BYTES, st + A_BYTES + B_BYTES + BM * 16, wn * WTN + j * 32, c, lane);
                // Operands of sub-step kk+1 are expanded while the MFMAs of kk run.
                f16x8_t av[2][NA], bv[2][FN];
                auto expand = [&](int kk, int buf) {
#pragma unroll
                  for (int i = 0; i < NA; ++i) av[buf][i] = nv_expand(fa[i], kk);
#pragma unroll
                  for (int j = 0; j < FN; ++j) bv[buf][j] = nv_expand(fb[j], kk);
                };
                expand(0, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * (NA + FN), 0);  // the fragment reads,
                __builtin_amdgcn_sched_group_barrier(0x002, 8 * (NA + FN), 0);  // then the first expansion
#pragma unroll
                for (int kk = 0; kk < BK / 16; ++kk) {
                  if (kk + 1 < BK / 16) expand(kk + 1, (kk + 1) & 1);
#pragma unroll
                  for (int i = 0; i < NA; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                      acc[i][j] =
                          __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[kk & 1][j], av[kk & 1][i], acc[i][j], 0, 0, 0);
                  // ~8 VALU per expanded fragment (4 converts, 4 multiplies)
                  if (kk + 1 < BK / 16) interleave_mfma_valu<NA * FN, (8 * (NA + FN) + NA * FN - 1) / (NA * FN)>();
                }
              }
            }
          } else if constexpr (MX) {
            // Two 64-element chunks per stage (K % 128 == 0); the fragments
            // and scales of chunk c+1 are read while the MFMAs of c run.
            // The B (fp4) fragment is the MFMA's first operand, as in the
            // other layouts, so the result is the transposed tile.
            i32x8_t fa[2][NA], fb[2][FN];
            int sa[2][NA], sb[2][FN];
            const uint8_t* sca = st + A_BYTES + B_BYTES;
            auto read_frags = [&](int c, int buf) {
#pragma unroll
              for (int i = 0; i < NA; ++i) {
                fa[buf][i] = frag_mx_a(st, wm * WTM + i * 32, c, lane);
                sa[buf][i] = scale_mx(sca, wm * WTM + i * 32, c, lane);
              }
#pragma unroll
              for (int j = 0; j < FN; ++j) {
                fb[buf][j] = frag_mx_b(st + A_BYTES, wn * WTN + j * 32, c, lane);
                sb[buf][j] = scale_mx(sca + BM * 4, wn * WTN + j * 32, c, lane);
              }
            };
            constexpr int NRD = 3 * NA + 2 * FN;  // LDS reads per chunk: 2 + 1 per A, 1 + 1 per B
            read_frags(0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
            for (int c = 0; c < KS / BK; ++c) {
              // the wave behind in the stage issues first (as in the NVFP4 loop)
              if (c == 0)
                __builtin_amdgcn_s_setprio(1);
              else
                __builtin_amdgcn_s_setprio(0);
              if (c + 1 < KS / BK) read_frags(c + 1, (c + 1) & 1);
#pragma unroll
              for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                      fb[c & 1][j], fa[c & 1][i], acc[i][j], 4 /* first operand: fp4 E2M1 */,
                      0 /* second operand: fp8 E4M3 */, 0, sb[c & 1][j], 0, sa[c & 1][i]);
              if (c + 1 < KS / BK)
                interleave_mfma_ds<NA * FN, NRD>();
              else
                interleave_mfma_ds<NA * FN, 0>();
            }
          } else {
            // Fragments of sub-step kk+1 are read while the MFMAs of kk run.
            bf16x8_t av[2][NA], bv[2][FN];
            auto read_frags = [&](int kk, int buf) {
#pragma unroll
              for (int i = 0; i < NA; ++i)
                av[buf][i] = MODE == TN_BF16 ? frag_mnmajor<BM>(st, wm * WTM + i * 32, kk, lane)
                                             : frag_kmajor<BKB * 2>(st, wm * WTM + i * 32, kk, lane);
#pragma unroll
              for (int j = 0; j < FN; ++j)
                bv[buf][j] = MODE == NT_BF16 ? frag_kmajor<BKB * 2>(st + A_BYTES, wn * WTN + j * 32, kk, lane)
                                             : frag_mnmajor<BN>(st + A_BYTES, wn * WTN + j * 32, kk, lane);
            };
            // LDS reads per sub-step: one per K-major fragment, two per MN-major one.
            constexpr int NRD = NA * (MODE == TN_BF16 ? 2 : 1) + FN * (MODE == NT_BF16 ? 1 : 2);
            read_frags(0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
            for (int kk = 0; kk < BKB / 16; ++kk) {
              if (kk + 1 < BKB / 16) read_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
              for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  acc[i][j] =
                      __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[kk & 1][j], av[kk & 1][i], acc[i][j], 0, 0, 0);
              if (kk + 1 < BKB / 16)
                interleave_mfma_ds<NA * FN, NRD>();
              else
                interleave_mfma_ds<NA * FN, 0>();
              if (kLateLoads && kk == 0 && kt + S - 1 < nk) {
                load_step(kt + S - 1, (int)((slot0 + kt + S - 1) % S));
                loads_issued = true;
              }
            }
          }
        }
      };
      if (n_active > 0) compute(IntConst<FM>{});
      if (kLateLoads && !loads_issued && kt + S - 1 < nk) load_step(kt + S - 1, (int)((slot0 + kt + S - 1) % S));
      if constexpr (NV || MX) __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (PF2) {
      if (pf_on && L + t_step < t_end) prefetch_next();
      nst = 0;
    }

    // Epilogue.  Register r of lane l of a 32x32 MFMA result holds result row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32 (probed on the device).  The
    // MFMAs take the B fragment as their first operand, so the result is the
    // transposed tile: lane l holds output row l%32 and, for g = 0..3, the
    // four consecutive output columns 8*g + 4*(l/32) + 0..3 in registers
    // 4g..4g+3 -- one 8-byte (bf16) or 16-byte (fp32) store each.
    float alpha = 1.0f;
    if (PFX) alpha = alpha_t;
    else if (MODE == W4A4_TN) alpha = p.ag[0] * p.bg[0];
    else if (NV) alpha = p.ag[0] * p.bg[expert];
    const int64_t ldc = p.N;
    float* C32 = reinterpret_cast<float*>(p.c);
    uint16_t* C16 = reinterpret_cast<uint16_t*>(p.c);
    const int64_t cbase = is_tn(MODE) ? (int64_t)expert * p.K * p.N : 0;
    if constexpr (SILU) {
      static_assert(BN == 256 && WTN % 64 == 0, "SiLU-gate tiles");
      // SiLU gate on the tile: block pair (2jj, 2jj+1) holds gate and up of
      // the same features.  Y1 is rounded to bf16 first, so H is the SiLU
      // gate of the stored Y1, as the standalone kernel computes it.
      uint16_t* Hp = reinterpret_cast<uint16_t*>(p.h);
      // global scale of H for the in-epilogue requantization
      const float h_g = MODE == W4A4_SILU_Q ? global_scale(p.h_amax_in[0]) : 1.0f;
      const int64_t F = p.N / 2;
      float m = 0.0f;
      // Gate and up of each 32-row block leave through a private LDS region
      // of the wave (two 32 x FW bf16 parts, 16-byte chunks XOR-swizzled by
      // row) and are read back by rows; H is computed from the read-back
      // rows (the same bf16 gate and up values), so every global store
      // writes 16 bytes per lane and whole 128-byte lines.
      constexpr int FW = WTN / 2;                // features per wave
      constexpr int CH = FW / 8;                 // 16-byte chunks per row and part
      constexpr int PART = 32 * FW * 2;
      static_assert(!PF && NW * 2 * PART <= (PF2 ? STAGE : S * STAGE) && (CH & (CH - 1)) == 0 && 64 % CH == 0,
                    "SiLU staging");
      lds_barrier();  // the stage ring is free: every wave is past its last step
      // PF2: in the slot of the tile's last stage (the other one holds the
      // next tile's first stage).
      uint8_t* reg = (PF2 ? smem + (int)((slot0 + nk - 1) % S) * STAGE : smem) + wid * 2 * PART;
      const int q = lane & 31, hh = lane >> 5;
      const int64_t f0 = j0 + wn * FW;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t row0 = m0 + wm * WTM + i * 32;
#pragma unroll
        for (int jj = 0; jj < FN / 2; ++jj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16_t& ga = acc[i][2 * jj];
            const f32x16_t& ua = acc[i][2 * jj + 1];
            const uint32_t g01 = pack_bf16x2(ga[4 * g] * alpha, ga[4 * g + 1] * alpha);
            const uint32_t g23 = pack_bf16x2(ga[4 * g + 2] * alpha, ga[4 * g + 3] * alpha);
            const uint32_t u01 = pack_bf16x2(ua[4 * g] * alpha, ua[4 * g + 1] * alpha);
            const uint32_t u23 = pack_bf16x2(ua[4 * g + 2] * alpha, ua[4 * g + 3] * alpha);
            // features jj*32 + 8g + 4hh .. +3: chunk jj*4 + g, half hh
            const int off = q * (FW * 2) + (((jj * 4 + g) ^ (q & (CH - 1))) << 4) + 8 * hh;
            *reinterpret_cast<uint2*>(reg + off) = make_uint2(g01, g23);
            *reinterpret_cast<uint2*>(reg + PART + off) = make_uint2(u01, u23);
          }
#pragma unroll
        for (int t = 0; t < 32 * CH / 64; ++t) {
          const int r = t * (64 / CH) + lane / CH, ch = lane % CH;
          const int off = r * (FW * 2) + ((ch ^ (r & (CH - 1))) << 4);
          const int64_t row = row0 + r, f = f0 + ch * 8;
          const uint4 vg = *reinterpret_cast<const uint4*>(reg + off);
          const uint4 vu = *reinterpret_cast<const uint4*>(reg + PART + off);
          const uint32_t gw[4] = {vg.x, vg.y, vg.z, vg.w}, uw[4] = {vu.x, vu.y, vu.z, vu.w};
          uint32_t hw[4];
#pragma unroll
          for (int w = 0; w < 4; ++w)
            hw[w] = pack_bf16x2(silu_gate(bf16_lo(gw[w]), bf16_lo(uw[w])), silu_gate(bf16_hi(gw[w]), bf16_hi(uw[w])));
          const bool valid = row < m_end;
          // PF2: count this wave's stores (a store with no active lane is
          // not counted, so the count never exceeds what is outstanding)
          if constexpr (PF2) nst += __ballot(valid) != 0 ? (C16 ? 2 : 0) + (Hp ? 1 : 0) : 0;
          if (valid) {
#pragma unroll
            for (int w = 0; w < 4; ++w) m = fmaxf(m, fmaxf(fabsf(bf16_lo(hw[w])), fabsf(bf16_hi(hw[w]))));
            if (C16) {
              *reinterpret_cast<uint4*>(C16 + row * ldc + f) = vg;
              *reinterpret_cast<uint4*>(C16 + row * ldc + F + f) = vu;
            }
            if (Hp) *reinterpret_cast<uint4*>(Hp + row * F + f) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          }
          if constexpr (MODE == W4A4_SILU_Q) {
            {
              // NVFP4 of H with the handed-in amax, from the stored bf16
              // values: lanes ch and ch ^ 1 (one row) hold the 16 features
              // of one block, 8 each; their amax is combined by a shuffle
              // (every lane of the pair takes it: same row, same validity).
              float hv[8];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                hv[2 * w] = bf16_lo(hw[w]);
                hv[2 * w + 1] = bf16_hi(hw[w]);
              }
              float a = 0.0f;
#pragma unroll
              for (int i2 = 0; i2 < 8; ++i2) a = fmaxf(a, fabsf(hv[i2]));
              a = fmaxf(a, __shfl_xor(a, 1, 64));
              uint32_t sbyte;
              float d;
              block_scale(a, h_g, sbyte, d);
              const uint32_t codes = encode8(hv, d);
              if constexpr (PF2) nst += (__ballot(valid) != 0 ? 1 : 0) + (__ballot(valid && (ch & 1) == 0) != 0 ? 1 : 0);
              if (valid) {
                *reinterpret_cast<uint32_t*>(p.hq + row * (F / 2) + f / 2) = codes;
                if ((ch & 1) == 0) p.hs[row * (F / 16) + f / 16] = (uint8_t)sbyte;
              }
            }
          }
          if constexpr (MODE == W4A8_SILU_Q) {
            // MXFP8 of H from the stored bf16 values: lanes ch .. ch ^ 3 (one
            // row, chunks 4b .. 4b+3) hold the 32 features of one block, 8
            // each; their amax is combined by two shuffles, every lane of the
            // group takes the shared exponent and encodes its 8 values, and
            // the group's first lane stores the scale byte.
            float hv[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              hv[2 * w] = bf16_lo(hw[w]);
              hv[2 * w + 1] = bf16_hi(hw[w]);
            }
            float a = 0.0f;
#pragma unroll
            for (int i2 = 0; i2 < 8; ++i2) a = fmaxf(a, fabsf(hv[i2]));
            a = fmaxf(a, __shfl_xor(a, 1, 64));
            a = fmaxf(a, __shfl_xor(a, 2, 64));
            const int se = shared_exp<8>(a);
            const uint2 codes = make_uint2(encode4_e4m3(hv, se), encode4_e4m3(hv + 4, se));
            if (valid) {
              *reinterpret_cast<uint2*>(p.hq + row * F + f) = codes;
              if ((ch & 3) == 0) p.hs[row * (F / 32) + f / 32] = (uint8_t)(se + 127);
            }
          }
        }
      }
      silu_amax = fmaxf(silu_amax, m);
      if constexpr (PF2) {
        slot0 = (int)((slot0 + nk) % S);
        pre = pre_next;
      }
      continue;
    }
    // The wave's results leave through a private LDS region (the stage ring
    // is free once every wave is past its last step): each 32-row block is
    // written in the register layout above and read back by rows, so that
    // every global store instruction writes whole 128-byte lines of
    // consecutive rows (16 bytes per lane) instead of 32 partial lines.
    constexpr int REGION = 32 * WTN * 4;  // one 32-row block in fp32
    // PF: bf16 blocks, in the ring slot of the tile's last stage (the other
    // slot holds the next tile's first stage).
    constexpr int REGION_PF = 32 * WTN * 2;
    static_assert(!PF || NW * REGION_PF <= STAGE, "PF epilogue staging");
    if constexpr (NW * REGION <= S * STAGE && WTN % 32 == 0) {
      lds_barrier();
      uint8_t* reg = PF ? smem + (int)((slot0 + nk - 1) % S) * STAGE + wid * REGION_PF : smem + wid * REGION;
      if constexpr (PF) nst = 0;
      const int q = lane & 31, h = lane >> 5;
      const int64_t col0 = n0 + wn * WTN;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t row0 = m0 + wm * WTM + i * 32;
        if constexpr (OUT32) {
          constexpr int CH = WTN / 4;  // 16-byte chunks per row
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x16_t& a = acc[i][j];
              const int ch = j * 8 + 2 * g + h;
              *reinterpret_cast<float4*>(reg + q * (WTN * 4) + ((ch ^ (q & (CH - 1))) << 4)) =
                  make_float4(a[4 * g] * alpha, a[4 * g + 1] * alpha, a[4 * g + 2] * alpha, a[4 * g + 3] * alpha);
            }
#pragma unroll 2
          for (int t = 0; t < 32 * CH / 64; ++t) {
            const int r = t * (64 / CH) + lane / CH, ch = lane % CH;
            float4 v = *reinterpret_cast<const float4*>(reg + r * (WTN * 4) + ((ch ^ (r & (CH - 1))) << 4));
            const int64_t row = row0 + r, col = col0 + ch * 4;
            if (row < m_end && col < p.N) {
              float4* dst = reinterpret_cast<float4*>(C32 + cbase + row * ldc + col);
              if (p.accumulate) {
                const float4 o = *dst;
                v.x += o.x;
                v.y += o.y;
                v.z += o.z;
                v.w += o.w;
              }
              *dst = v;
            }
          }
        } else {
          constexpr int CH = WTN / 8;  // 16-byte chunks (8 bf16) per row
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x16_t& a = acc[i][j];
              const int ch = j * 4 + g;
              *reinterpret_cast<uint2*>(reg + q * (WTN * 2) + ((ch ^ (q & (CH - 1))) << 4) + 8 * h) =
                  make_uint2(pack_bf16x2(a[4 * g] * alpha, a[4 * g + 1] * alpha),
                             pack_bf16x2(a[4 * g + 2] * alpha, a[4 * g + 3] * alpha));
            }
#pragma unroll 2
          for (int t = 0; t < 32 * CH / 64; ++t) {
            const int r = t * (64 / CH) + lane / CH, ch = lane % CH;
            const uint4 v = *reinterpret_cast<const uint4*>(reg + r * (WTN * 2) + ((ch ^ (r & (CH - 1))) << 4));
            const int64_t row = row0 + r, col = col0 + ch * 8;
            if constexpr (PF) nst += __ballot(row < m_end && col < p.N) != 0 ? 1 : 0;
            if (row < m_end && col < p.N) *reinterpret_cast<uint4*>(C16 + cbase + row * ldc + col) = v;
          }
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t row = m0 + wm * WTM + i * 32 + (lane & 31);
      if (row >= m_end) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (n0 + wn * WTN + j * 32 >= p.N) continue;  // N % 32 == 0: whole blocks
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t idx = cbase + row * ldc + n0 + wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
          const f32x16_t& a = acc[i][j];
          float4 v = make_float4(a[4 * g] * alpha, a[4 * g + 1] * alpha, a[4 * g + 2] * alpha, a[4 * g + 3] * alpha);
          if constexpr (OUT32) {
            float4* dst = reinterpret_cast<float4*>(C32 + idx);
            if (p.accumulate) {
              const float4 o = *dst;
              v.x += o.x;
              v.y += o.y;
              v.z += o.z;
              v.w += o.w;
            }
            *dst = v;
          } else {
            *reinterpret_cast<uint2*>(C16 + idx) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
          }
        }
      }
    }
    }
    if constexpr (PF) {
      slot0 = (int)((slot0 + nk) % S);
      pre = pre_next;
    }
  }
  // W4A4_SILU: one atomic per workgroup for the amax of H (every wave of the
  // workgroup leaves the tile loop together).
  if constexpr (SILU) {
    if (MODE == W4A4_SILU_Q && blockIdx.x == 0 && threadIdx.x == 0) p.hg[0] = global_scale(p.h_amax_in[0]);
    if (p.amax) {
      __shared__ float red[NW];
      const float m = wave_max(silu_amax);
      if (lane == 0) red[wid] = m;
      __syncthreads();
      if (threadIdx.x == 0) {
        float v = red[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) v = fmaxf(v, red[i]);
        atomicMax(reinterpret_cast<unsigned int*>(p.amax), __float_as_uint(v));
      }
    }
  }
}

// Global scale of the in-epilogue requantized H when the GEMM has no rows.
__global__ void h_gscale_kernel(const float* amax, float* g) { g[0] = global_scale(amax[0]); }

// Resident workgroups per CU of one kernel instantiation (cached; the same on
// every gfx950 device).
template <int MODE, int BM, int BN, int WM, int WN, int S, int BKB, bool OUT32>
int resident_per_cu() {
  static int cached = 0;
  if (cached > 0) return cached;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_kernel<MODE, BM, BN, WM, WN, S, BKB, OUT32>, WM * WN * 64,
                                                   0) !=
          hipSuccess ||
      occ < 1)
    occ = 1;
  cached = occ;
  return occ;
}

template <int MODE, int BM, int BN, int WM, int WN, int S, int BKB, bool OUT32>
int launch_cfg(const Params& p0, hipStream_t st) {
  Params p = p0;
  p.n_tiles = (int)cdiv(p.N, BN);
  int64_t upper;
  if (is_tn(MODE)) {
    p.k_tiles_tn = (int)cdiv(p.K, BM);
    upper = (int64_t)p.E * p.k_tiles_tn * p.n_tiles;
  } else {
    upper = (cdiv(p.M, BM) + p.E) * p.n_tiles;
  }
  if (upper <= 0) return NVFP4MOE_OK;
  if (upper > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  int64_t grid = (int64_t)device_cu_count() * resident_per_cu<MODE, BM, BN, WM, WN, S, BKB, OUT32>();
  if (grid > upper) grid = upper;
  grid = cdiv(grid, 8) * 8;  // whole XCD rounds
  gemm_kernel<MODE, BM, BN, WM, WN, S, BKB, OUT32><<<(unsigned)grid, WM * WN * 64, 0, st>>>(p);
  return launch_status();
}

// Tile configurations: (BM, BN, waves along M, waves along N, LDS stages,
// reduction elements per bf16 stage).
// Only the configuration pick_config chooses for each layout is compiled; a
// build for tuning sweeps may force one for all layouts with
// -DNVFP4MOE_GEMM_FORCE_CONFIG=<i>.
#define NVFP4MOE_GEMM_CONFIGS(X) \
  X(0, 256, 256, 2, 4, 2, 64)    \
  X(1, 256, 256, 4, 2, 2, 64)    \
  X(2, 256, 128, 2, 2, 3, 64)    \
  X(3, 128, 256, 2, 2, 3, 64)    \
  X(4, 128, 128, 2, 2, 4, 64)    \
  X(5, 256, 128, 4, 2, 2, 64)    \
  X(6, 128, 256, 2, 4, 2, 64)    \
  X(7, 256, 256, 2, 2, 2, 64)    \
  X(8, 128, 128, 2, 2, 2, 64)    \
  X(9, 256, 256, 4, 2, 4, 32)    \
  X(10, 256, 128, 4, 1, 3, 32)   \
  X(11, 128, 256, 2, 2, 3, 32)   \
  X(12, 256, 256, 4, 2, 3, 32)   \
  X(13, 256, 256, 2, 2, 4, 32)   \
  X(14, 256, 256, 4, 2, 3, 64)

// Measured on the MoE shapes (expert rows ~512, N 768..2048, K 768..2048):
// 256 x 256 tiles on 8 waves (4 x 2); two 64-k stages for the NT and W4A4
// GEMMs, four 32-k stages (a longer prefetch in the same LDS) for NN and TN,
// whose MN-major operands come through transposed LDS reads (NN -9..-12%,
// TN -2..-4% against two 64-k stages).  Two 4-wave workgroups per CU
// (config 10), to overlap one's epilogue with the other's loop, was slower.
constexpr int default_config(int mode) {
  return mode == NN_BF16 || mode == TN_BF16 ? 9 : is_mx(mode) ? 14 : 1;
}
#ifdef NVFP4MOE_GEMM_FORCE_CONFIG
constexpr int kForcedConfig = NVFP4MOE_GEMM_FORCE_CONFIG;
#else
constexpr int kForcedConfig = -1;
#endif
constexpr int built_config(int mode) { return kForcedConfig >= 0 ? kForcedConfig : default_config(mode); }

// Whether a configuration is valid for a layout: LDS within the 160 KiB of
// a gfx950 CU, whole loads per wave, NVFP4 stages of 64-element chunks, and
// for the SiLU-gate epilogue 256-column tiles whose wave halves are
// multiples of 64 columns.
constexpr bool cfg_ok(int mode, int bm, int bn, int wm, int wn, int s, int bkb) {
  const int nw = wm * wn;
  if (is_q(mode) && bkb != 64) return false;
  // MX: whole loads of 128-byte A rows (8 per load) and 64-byte B rows (16 per load) per wave
  if (is_mx(mode) && (bm % (8 * nw) != 0 || bn % (16 * nw) != 0)) return false;
  if (!is_q(mode)) {
    // whole K-major loads (512 / bkb rows each) and MN-major loads (512 / cols rows each) per wave
    const bool kmaj_a = mode != TN_BF16, kmaj_b = mode == NT_BF16;
    if (kmaj_a && bm % ((512 / bkb) * nw) != 0) return false;
    if (kmaj_b && bn % ((512 / bkb) * nw) != 0) return false;
    if (!kmaj_a && (bm != 128 && bm != 256 || (bkb / (512 / bm)) % nw != 0)) return false;
    if (!kmaj_b && (bn != 128 && bn != 256 || (bkb / (512 / bn)) % nw != 0)) return false;
    if ((bm / wm) % 32 != 0 || (bn / wn) % 32 != 0) return false;
  }
  const int stage = is_nv(mode) ? (bm + bn) * 144 : is_mx(mode) ? bm * 128 + bn * 64 + (bm + bn) * 4
                                                                : (bm + bn) * bkb * 2;
  return s * stage <= 152 * 1024 &&   // 160 KiB of LDS less the offsets copy and tile state
         (!is_q(mode) || (bm + bn) % (64 * wm * wn) == 0) &&
         (!is_silu(mode) || (bn == 256 && (bn / wn) % 64 == 0));
}

template <int MODE>
int launch_mode(int cfg, const Params& p, hipStream_t st) {
  switch (cfg) {
#define NVFP4MOE_CASE(I, BM_, BN_, WM_, WN_, S_, BK_)                                          \
  case I:                                                                                      \
    if constexpr (built_config(MODE) == I && cfg_ok(MODE, BM_, BN_, WM_, WN_, S_, BK_)) {       \
      if (p.c_f32) {                                                                           \
        if constexpr (!is_silu(MODE)) return launch_cfg<MODE, BM_, BN_, WM_, WN_, S_, BK_, true>(p, st); \
      } else {                                                                                 \
        return launch_cfg<MODE, BM_, BN_, WM_, WN_, S_, BK_, false>(p, st);                    \
      }                                                                                        \
    }                                                                                          \
    break;
    NVFP4MOE_GEMM_CONFIGS(NVFP4MOE_CASE)
#undef NVFP4MOE_CASE
    default: break;
  }
  return NVFP4MOE_ESHAPE;
}

// Tile configuration per layout (see default_config).
int pick_config(int mode, const Params& p) {
  (void)p;
  return built_config(mode);
}

int launch(int mode, const Params& p, hipStream_t st) {
  const int cfg = pick_config(mode, p);
  switch (mode) {
    case NT_BF16: return launch_mode<NT_BF16>(cfg, p, st);
    case NN_BF16: return launch_mode<NN_BF16>(cfg, p, st);
    case TN_BF16: return launch_mode<TN_BF16>(cfg, p, st);
    case W4A4_SILU: return launch_mode<W4A4_SILU>(cfg, p, st);
    case W4A8: return launch_mode<W4A8>(cfg, p, st);
    case W4A8_SILU: return launch_mode<W4A8_SILU>(cfg, p, st);
    case W4A8_SILU_Q: return launch_mode<W4A8_SILU_Q>(cfg, p, st);
    case W4A4_SILU_Q: return launch_mode<W4A4_SILU_Q>(cfg, p, st);
    case W4A4_TN: return launch_mode<W4A4_TN>(cfg, p, st);
    case W4A4_B: return launch_mode<W4A4_B>(cfg, p, st);
    default: return launch_mode<W4A4>(cfg, p, st);
  }
}

}  // namespace
}  // namespace nvfp4moe

using namespace nvfp4moe;

namespace {

// Shared by both W4A4 entry points.  silu: c = Y1 (NULL: not stored), h = H.
int w4a4_entry(const uint8_t* a_q, const uint8_t* a_s, const float* a_g, const uint8_t* b_q, const uint8_t* b_s,
               const float* b_g, const int32_t* expert_offsets, int E, int64_t M_total, int64_t N, int64_t K,
               void* c, int c_dtype, int silu, void* h, float* amax_out, hipStream_t st,
               const float* h_amax_in = nullptr, uint8_t* hq = nullptr, uint8_t* hs = nullptr, float* hg = nullptr,
               bool design_b = false) {
  const bool qh = hq != nullptr;
  if (E < 1 || M_total < 0 || N < 0 || K < 0) return NVFP4MOE_EINVAL;
  if (c_dtype != NVFP4MOE_F32 && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (silu && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!expert_offsets || !a_g || !b_g) return NVFP4MOE_EINVAL;
  if (M_total > 0 && N > 0 && (!a_q || !a_s || !b_q || !b_s || (silu ? !h && !qh : !c))) return NVFP4MOE_EINVAL;
  if (qh && (!h_amax_in || !hs || !hg || (amax_out && amax_out == h_amax_in))) return NVFP4MOE_EINVAL;
  if (K % 64 != 0 || N % 32 != 0) return NVFP4MOE_ESHAPE;
  if (silu && N % 256 != 0) return NVFP4MOE_ESHAPE;
  if (M_total > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x7FFFFFFFLL || !aligned(a_q, 16) || !aligned(b_q, 16) ||
      !aligned(a_s, 4) || !aligned(b_s, 4) ||
      !aligned(c, 16) || !aligned(h, 16) || !aligned(hq, 4) || !aligned(hg, 4) || !aligned(h_amax_in, 4))
    return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (silu && amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
  if (M_total == 0 || N == 0) {
    if (qh) h_gscale_kernel<<<1, 1, 0, st>>>(h_amax_in, hg);
    return launch_status();
  }
  Params p = {};
  p.a = a_q;
  p.b = b_q;
  p.as = a_s;
  p.bs = b_s;
  p.ag = a_g;
  p.bg = b_g;
  p.offsets = expert_offsets;
  p.c = c;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.E = E;
  p.c_f32 = c_dtype == NVFP4MOE_F32;
  p.h = h;
  p.amax = amax_out;
  p.hq = hq;
  p.hs = hs;
  p.hg = hg;
  p.h_amax_in = h_amax_in;
  return launch(silu ? (qh ? W4A4_SILU_Q : W4A4_SILU) : design_b ? W4A4_B : W4A4, p, st);
}

}  // namespace

extern "C" int grouped_gemm_w4a4(const uint8_t* a_q, const uint8_t* a_s, const float* a_g, const uint8_t* b_q,
                                 const uint8_t* b_s, const float* b_g, const int32_t* expert_offsets, int E,
                                 int64_t M_total, int64_t N, int64_t K, void* c, int c_dtype, int epilogue,
                                 float* amax_out, void* workspace, size_t ws_bytes, nvfp4moe_stream_t stream) {
  (void)workspace;
  (void)ws_bytes;
  if (epilogue == NVFP4MOE_EPI_NONE)
    return w4a4_entry(a_q, a_s, a_g, b_q, b_s, b_g, expert_offsets, E, M_total, N, K, c, c_dtype, 0, nullptr,
                      nullptr, as_stream(stream));
  if (epilogue == NVFP4MOE_EPI_SILU_GATE)
    return w4a4_entry(a_q, a_s, a_g, b_q, b_s, b_g, expert_offsets, E, M_total, N, K, nullptr, c_dtype, 1, c,
                      amax_out, as_stream(stream));
  return NVFP4MOE_EINVAL;
}

extern "C" int grouped_gemm_w4a4_silu_gate(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                                           const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                                           const int32_t* expert_offsets, int E, int64_t M_total, int64_t F,
                                           int64_t K, void* y1, void* h, float* amax_out, nvfp4moe_stream_t stream) {
  if (F < 0) return NVFP4MOE_EINVAL;
  return w4a4_entry(a_q, a_s, a_g, b_q, b_s, b_g, expert_offsets, E, M_total, 2 * F, K, y1, NVFP4MOE_BF16, 1, h,
                    amax_out, as_stream(stream));
}

namespace {

// Shared by both W4A8 entry points.  silu: c = Y1 (NULL: not stored), h = H.
int w4a8_entry(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
               const int32_t* expert_offsets, int E, int64_t M_total, int64_t N, int64_t K, void* c, int c_dtype,
               int silu, void* h, float* amax_out, hipStream_t st, uint8_t* hq = nullptr, uint8_t* hs = nullptr) {
  const bool qh = hq != nullptr;
  if (E < 1 || M_total < 0 || N < 0 || K < 0) return NVFP4MOE_EINVAL;
  if (c_dtype != NVFP4MOE_F32 && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (silu && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!expert_offsets || (qh && (!silu || !hs))) return NVFP4MOE_EINVAL;
  if (M_total > 0 && N > 0 && (!a_q || !a_s || !b_q || !b_s || (silu ? !h && !qh : !c))) return NVFP4MOE_EINVAL;
  if (K % 128 != 0 || N % 32 != 0) return NVFP4MOE_ESHAPE;
  if (silu && N % 256 != 0) return NVFP4MOE_ESHAPE;
  if (M_total > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x7FFFFFFFLL || !aligned(a_q, 16) || !aligned(b_q, 16) ||
      !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(c, 16) || !aligned(h, 16) || !aligned(hq, 8))
    return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (silu && amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
  if (M_total == 0 || N == 0) return launch_status();
  Params p = {};
  p.a = a_q;
  p.b = b_q;
  p.as = a_s;
  p.bs = b_s;
  p.offsets = expert_offsets;
  p.c = c;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.E = E;
  p.c_f32 = c_dtype == NVFP4MOE_F32;
  p.h = h;
  p.amax = amax_out;
  p.hq = hq;
  p.hs = hs;
  return launch(silu ? (qh ? W4A8_SILU_Q : W4A8_SILU) : W4A8, p, st);
}

}  // namespace

extern "C" int grouped_gemm_w4a8(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                                 const int32_t* expert_offsets, int E, int64_t M_total, int64_t N, int64_t K,
                                 void* c, int c_dtype, nvfp4moe_stream_t stream) {
  return w4a8_entry(a_q, a_s, b_q, b_s, expert_offsets, E, M_total, N, K, c, c_dtype, 0, nullptr, nullptr,
                    as_stream(stream));
}

extern "C" int grouped_gemm_w4a8_silu_gate(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                                           const uint8_t* b_s, const int32_t* expert_offsets, int E, int64_t M_total,
                                           int64_t F, int64_t K, void* y1, void* h, float* amax_out,
                                           nvfp4moe_stream_t stream) {
  if (F < 0) return NVFP4MOE_EINVAL;
  return w4a8_entry(a_q, a_s, b_q, b_s, expert_offsets, E, M_total, 2 * F, K, y1, NVFP4MOE_BF16, 1, h, amax_out,
                    as_stream(stream));
}

extern "C" int grouped_gemm_w4a8_silu_gate_mx(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                                              const uint8_t* b_s, const int32_t* expert_offsets, int E,
                                              int64_t M_total, int64_t F, int64_t K, void* y1, void* h,
                                              float* amax_out, uint8_t* q_h, uint8_t* s_h,
                                              nvfp4moe_stream_t stream) {
  if (F < 0) return NVFP4MOE_EINVAL;
  if (!q_h) return NVFP4MOE_EINVAL;
  return w4a8_entry(a_q, a_s, b_q, b_s, expert_offsets, E, M_total, 2 * F, K, y1, NVFP4MOE_BF16, 1, h, amax_out,
                    as_stream(stream), q_h, s_h);
}

extern "C" int grouped_gemm_w4a4_silu_gate_nvfp4(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                                                 const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                                                 const int32_t* expert_offsets, int E, int64_t M_total, int64_t F,
                                                 int64_t K, void* y1, void* h, float* amax_out,
                                                 const float* amax_h_in, uint8_t* q_h, uint8_t* s_h, float* g_h,
                                                 nvfp4moe_stream_t stream) {
  if (F < 0) return NVFP4MOE_EINVAL;
  if (!q_h) return NVFP4MOE_EINVAL;
  return w4a4_entry(a_q, a_s, a_g, b_q, b_s, b_g, expert_offsets, E, M_total, 2 * F, K, y1, NVFP4MOE_BF16, 1, h,
                    amax_out, as_stream(stream), amax_h_in, q_h, s_h, g_h);
}

extern "C" int grouped_gemm_w4a4_wgrad(const uint8_t* a_q, const uint8_t* a_s, const float* a_g, const uint8_t* b_q,
                                       const uint8_t* b_s, const float* b_g, const int32_t* expert_offsets, int E,
                                       int64_t M_total, int64_t Kp, int64_t N1, int64_t N2, void* c, int c_dtype,
                                       nvfp4moe_stream_t stream) {
  if (E < 1 || M_total < 0 || Kp < 0 || N1 < 0 || N2 < 0) return NVFP4MOE_EINVAL;
  if (c_dtype != NVFP4MOE_F32 && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (!expert_offsets || !a_g || !b_g) return NVFP4MOE_EINVAL;
  const bool has_out = N1 > 0 && N2 > 0;
  if (has_out && (!c || (M_total > 0 && (!a_q || !a_s || !b_q || !b_s)))) return NVFP4MOE_EINVAL;
  if (N1 % 32 != 0 || N2 % 32 != 0 || Kp % 64 != 0 || Kp < 64 * (M_total / 64 + (int64_t)E)) return NVFP4MOE_ESHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(c, 16))
    return NVFP4MOE_ESHAPE;
  // Operands are read through 32-bit buffer offsets.
  if (N1 * (Kp / 2) >= (1LL << 31) || N2 * (Kp / 2) >= (1LL << 31) || M_total > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (!has_out) return NVFP4MOE_OK;
  Params p = {};
  p.a = a_q;
  p.b = b_q;
  p.as = a_s;
  p.bs = b_s;
  p.ag = a_g;
  p.bg = b_g;
  p.offsets = expert_offsets;
  p.c = c;
  p.M = M_total;
  p.N = N2;
  p.K = N1;
  p.kp = Kp;
  p.E = E;
  p.c_f32 = c_dtype == NVFP4MOE_F32;
  return launch(W4A4_TN, p, as_stream(stream));
}

extern "C" int grouped_gemm_w4a4_scaled_mfma(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                                             const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                                             const int32_t* expert_offsets, int E, int64_t M_total, int64_t N,
                                             int64_t K, void* c, int c_dtype, nvfp4moe_stream_t stream) {
  return w4a4_entry(a_q, a_s, a_g, b_q, b_s, b_g, expert_offsets, E, M_total, N, K, c, c_dtype, 0, nullptr, nullptr,
                    as_stream(stream), nullptr, nullptr, nullptr, nullptr, true);
}

extern "C" int grouped_gemm_bf16_tn_gather(const void* a, const void* b, const int32_t* b_src, int k,
                                           int64_t b_rows, const int32_t* expert_offsets, int E, int64_t M_total,
                                           int64_t N, int64_t K, void* c, int c_dtype, int accumulate,
                                           nvfp4moe_stream_t stream) {
  if (E < 1 || M_total < 0 || N < 0 || K < 0 || k < 1 || b_rows < 0) return NVFP4MOE_EINVAL;
  if (c_dtype != NVFP4MOE_F32 && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (accumulate != 0 && accumulate != 1) return NVFP4MOE_EINVAL;
  if (accumulate && c_dtype != NVFP4MOE_F32) return NVFP4MOE_EINVAL;
  if (!expert_offsets) return NVFP4MOE_EINVAL;
  const bool has_out = K > 0 && N > 0;
  if (has_out && (!c || (M_total > 0 && (!a || !b_src || (b_rows > 0 && !b))))) return NVFP4MOE_EINVAL;
  if (K % 32 != 0 || N % 32 != 0) return NVFP4MOE_ESHAPE;
  if (M_total > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x7FFFFFFFLL || !aligned(a, 16) || !aligned(b, 16) ||
      !aligned(c, 16) || !aligned(b_src, 4))
    return NVFP4MOE_ESHAPE;
  // Buffer offsets are 32-bit: A and B must each stay below 2 GiB.
  if (M_total * K * 2 >= (1LL << 31) || b_rows * N * 2 >= (1LL << 31)) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (!has_out) return NVFP4MOE_OK;
  Params p = {};
  p.a = a;
  p.b = b;
  p.offsets = expert_offsets;
  p.c = c;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.E = E;
  p.c_f32 = c_dtype == NVFP4MOE_F32;
  p.accumulate = accumulate;
  // b_src is never read when no expert has rows; a NULL B with b_rows = 0
  // leaves every gathered row out of range (zeros).
  p.bsrc = b_src;
  p.bk = k;
  p.bk_shift = (k & (k - 1)) == 0 ? __builtin_ctz((unsigned)k) : -1;
  p.b_rows = b_rows;
  return launch(TN_BF16, p, as_stream(stream));
}

extern "C" int grouped_gemm_bf16(int layout, const void* a, const void* b, const int32_t* expert_offsets, int E,
                                 int64_t M_total, int64_t N, int64_t K, void* c, int c_dtype, int accumulate,
                                 void* workspace, size_t ws_bytes, nvfp4moe_stream_t stream) {
  (void)workspace;
  (void)ws_bytes;
  if (layout != NVFP4MOE_NT && layout != NVFP4MOE_NN && layout != NVFP4MOE_TN) return NVFP4MOE_EINVAL;
  if (E < 1 || M_total < 0 || N < 0 || K < 0) return NVFP4MOE_EINVAL;
  if (c_dtype != NVFP4MOE_F32 && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (accumulate != 0 && accumulate != 1) return NVFP4MOE_EINVAL;
  if (accumulate && c_dtype != NVFP4MOE_F32) return NVFP4MOE_EINVAL;
  if (!expert_offsets) return NVFP4MOE_EINVAL;
  const bool has_out = layout == NVFP4MOE_TN ? (K > 0 && N > 0) : (M_total > 0 && N > 0);
  if (has_out && (!c || (M_total > 0 && (!a || !b)))) return NVFP4MOE_EINVAL;
  if (K % 32 != 0 || N % 32 != 0) return NVFP4MOE_ESHAPE;
  if (M_total > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x7FFFFFFFLL || !aligned(a, 16) || !aligned(b, 16) ||
      !aligned(c, 16))
    return NVFP4MOE_ESHAPE;
  // Buffer offsets are 32-bit: one expert's operand must stay below 2 GiB.
  if (layout == NVFP4MOE_NN && K * N * 2 >= (1LL << 31)) return NVFP4MOE_ESHAPE;
  if (layout == NVFP4MOE_TN && (M_total * K * 2 >= (1LL << 31) || M_total * N * 2 >= (1LL << 31)))
    return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (!has_out) return NVFP4MOE_OK;
  Params p = {};
  p.a = a;
  p.b = b;
  p.offsets = expert_offsets;
  p.c = c;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.E = E;
  p.c_f32 = c_dtype == NVFP4MOE_F32;
  p.accumulate = accumulate;
  const int mode = layout == NVFP4MOE_NT ? NT_BF16 : layout == NVFP4MOE_NN ? NN_BF16 : TN_BF16;
  return launch(mode, p, as_stream(stream));
}
