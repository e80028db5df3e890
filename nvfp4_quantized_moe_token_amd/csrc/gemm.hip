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
// stages packed codes and scale bytes from HBM (0.5625 B per element),
// expands them exactly to fp16 while writing the LDS tile (hardware E2M1
// decode with a unit scale, then one packed fp16 multiply by the block
// scale), and runs fp16 MFMA with fp32 accumulation; the two global scales
// are applied in the fp32 epilogue.
//
// Tiling.  A workgroup of 256 threads (2 x 2 waves) computes a 128 x 128
// output tile; each wave owns 64 x 64 = 2 x 2 MFMA 32x32x16 tiles.  K moves
// in steps of 64 through two LDS stages (double buffer, one barrier per
// step); global loads of step k+1 are issued before the MFMAs of step k.
// LDS rows are 64 elements (128 B) with the 16-byte chunks XOR-swizzled by
// row, so fragment reads (ds_read_b128) and both writer patterns avoid bank
// conflicts.  Operands whose reduction dimension is not contiguous in memory
// (B of the NN layout, both operands of TN) are transposed in registers
// (4 x 8 blocks, v_perm) on their way to LDS.
//
// Scheduling.  The host knows only the total row count.  For row-grouped
// layouts (NT, NN, W4A4) the grid has one slot per possible (m-tile, n-tile)
// pair, ceil(M/128) + E m-tile slots; each workgroup maps its slot to an
// expert and row range by scanning the device offsets (wave-wide prefix
// sums), and surplus slots exit at once.  TN tiles are (expert, k-tile,
// n-tile) and reduce over the expert's rows.
#include "common.hpp"

namespace nvfp4moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int STAGE_ELEMS = (BM + BN) * BK;  // 16-bit elements per stage

enum Mode { NT_BF16 = 0, NN_BF16 = 1, TN_BF16 = 2, W4A4 = 3 };

struct Params {
  const void* a;       // NT/NN/TN: bf16 A; W4A4: packed codes of A
  const void* b;       // bf16 B or packed codes of B
  const uint8_t* as;   // W4A4: scales of A
  const uint8_t* bs;   // W4A4: scales of B
  const float* ag;     // W4A4: global scale of A [1]
  const float* bg;     // W4A4: global scales of B [E]
  const int32_t* offsets;
  void* c;
  int64_t M, N, K;     // TN: K = columns of A (rows of C_e)
  int E;
  int c_f32;
  int accumulate;
  int n_tiles;         // tiles along N
  int k_tiles_tn;      // TN: tiles along K (rows of C_e)
};

// Offset (in 16-bit elements) of chunk c (8 elements) of LDS row `row`.
__device__ __forceinline__ int lds_off(int row, int c) { return row * BK + ((c ^ ((row ^ (row >> 3)) & 7)) << 3); }

// Map m-tile slot `slot` to (expert, first row, end row) by a prefix sum of
// per-expert tile counts.  Runs on wave 0; returns false for surplus slots.
__device__ bool find_tile(const int32_t* __restrict__ off, int E, int64_t M, int slot, int& e_out, int64_t& r0,
                          int64_t& r1) {
  const int lane = threadIdx.x & 63;
  int running = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int lo = 0, hi = 0, cnt = 0;
    if (e < E) {
      lo = off[e];
      hi = off[e + 1];
      lo = lo < 0 ? 0 : lo > M ? (int)M : lo;
      hi = hi < lo ? lo : hi > M ? (int)M : hi;
      cnt = (hi - lo + BM - 1) / BM;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    if (slot < running + total) {
      const bool mine = slot >= running + incl - cnt && slot < running + incl;
      const uint64_t mask = __ballot(mine);
      const int srcl = __ffsll((unsigned long long)mask) - 1;
      e_out = __shfl(e, srcl, 64);
      const int lo_s = __shfl(lo, srcl, 64), hi_s = __shfl(hi, srcl, 64), ex = __shfl(incl - cnt, srcl, 64);
      r0 = lo_s + (int64_t)(slot - running - ex) * BM;
      r1 = r0 + BM < hi_s ? r0 + BM : hi_s;
      return true;
    }
    running += total;
  }
  return false;
}

// ---- loaders: global -> registers (issue) and registers -> LDS (commit) ----

// K-major bf16 tile: 128 rows x 64 k from a row-major [*, ld] matrix.
struct KMajorRegs {
  uint4 v[4];
};
__device__ __forceinline__ void kmajor_issue(KMajorRegs& r, const uint16_t* __restrict__ base, int64_t ld, int64_t row0,
                                             int64_t row_end, int64_t k0, int64_t K) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = threadIdx.x + NT * i, row = u >> 3, c = u & 7;
    const int64_t gr = row0 + row, gk = k0 + c * 8;
    r.v[i] = (gr < row_end && gk < K) ? *reinterpret_cast<const uint4*>(base + gr * ld + gk) : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void kmajor_commit(const KMajorRegs& r, uint16_t* lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = threadIdx.x + NT * i, row = u >> 3, c = u & 7;
    *reinterpret_cast<uint4*>(lds + lds_off(row, c)) = r.v[i];
  }
}

// MN-major bf16 tile: 64 reduction rows x 128 columns of a row-major
// [*, ld] matrix, stored transposed ([column][k]) in LDS.
struct MNMajorRegs {
  uint4 v[4];
};
__device__ __forceinline__ void mnmajor_issue(MNMajorRegs& r, const uint16_t* __restrict__ base, int64_t ld, int64_t k0,
                                              int64_t k_end, int64_t n0, int64_t ncols) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ng = lane & 15, kq = (lane >> 4) + 4 * wid;
  const int64_t gn = n0 + ng * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gk = k0 + kq * 4 + i;
    r.v[i] = (gk < k_end && gn < ncols) ? *reinterpret_cast<const uint4*>(base + gk * ld + gn) : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void mnmajor_commit(const MNMajorRegs& r, uint16_t* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ng = lane & 15, kq = (lane >> 4) + 4 * wid;
  const uint32_t w0[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
  const uint32_t w1[4] = {r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
  const uint32_t w2[4] = {r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w};
  const uint32_t w3[4] = {r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint2 d;
    d.x = __builtin_amdgcn_perm(w1[m], w0[m], sel);  // k = 4kq, 4kq+1
    d.y = __builtin_amdgcn_perm(w3[m], w2[m], sel);  // k = 4kq+2, 4kq+3
    const int row = ng * 8 + j;
    *reinterpret_cast<uint2*>(lds + lds_off(row, kq >> 1) + (kq & 1) * 4) = d;
  }
}

// NVFP4 K-major tile: 128 rows x 64 k (two 16-blocks of 32 per thread),
// expanded exactly to fp16.
struct NVRegs {
  uint4 q;
  uint32_t s;
};
__device__ __forceinline__ void nv_issue(NVRegs& r, const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                         int64_t K, int64_t row0, int64_t row_end, int64_t k0) {
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t gr = row0 + row, gk = k0 + half * 32;
  if (gr < row_end && gk < K) {
    r.q = *reinterpret_cast<const uint4*>(q + gr * (K / 2) + gk / 2);
    r.s = *reinterpret_cast<const uint16_t*>(s + gr * (K / 16) + gk / 16);
  } else {
    r.q = make_uint4(0, 0, 0, 0);
    r.s = 0;
  }
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
__device__ __forceinline__ void nv_commit(const NVRegs& r, uint16_t* lds) {
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.s, 0);
  const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.s, 1);
  const f16x2_t sc0 = {s0, s0}, sc1 = {s1, s1};
  const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const f16x2_t sc = wi < 2 ? sc0 : sc1;
    uint4 o;
    o.x = nv_pair(w[wi], sc, 0);
    o.y = nv_pair(w[wi], sc, 1);
    o.z = nv_pair(w[wi], sc, 2);
    o.w = nv_pair(w[wi], sc, 3);
    *reinterpret_cast<uint4*>(lds + lds_off(row, half * 4 + wi)) = o;
  }
}

// ---- the kernel ----

template <int MODE>
__global__ __launch_bounds__(NT) void gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE_ELEMS];
  __shared__ int64_t s_tile[3];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  int expert;
  int64_t m0, m_end;     // output rows (row-grouped) or C_e rows (TN)
  int64_t n0;
  int64_t k_begin, k_end;  // reduction range
  if (MODE == TN_BF16) {
    const int per_e = p.k_tiles_tn * p.n_tiles;
    expert = blockIdx.x / per_e;
    const int rem = blockIdx.x % per_e;
    m0 = (int64_t)(rem / p.n_tiles) * BM;
    m_end = p.K;
    n0 = (int64_t)(rem % p.n_tiles) * BN;
    int lo = p.offsets[expert], hi = p.offsets[expert + 1];
    lo = lo < 0 ? 0 : lo > p.M ? (int)p.M : lo;
    hi = hi < lo ? lo : hi > p.M ? (int)p.M : hi;
    k_begin = lo;
    k_end = hi;
  } else {
    const int slot = blockIdx.x / p.n_tiles;
    n0 = (int64_t)(blockIdx.x % p.n_tiles) * BN;
    if (wid == 0) {
      int e;
      int64_t r0, r1;
      const bool ok = find_tile(p.offsets, p.E, p.M, slot, e, r0, r1);
      if (lane == 0) {
        s_tile[0] = ok ? e : -1;
        s_tile[1] = r0;
        s_tile[2] = r1;
      }
    }
    __syncthreads();
    if (s_tile[0] < 0) return;
    expert = (int)s_tile[0];
    m0 = s_tile[1];
    m_end = s_tile[2];
    k_begin = 0;
    k_end = p.K;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Operand views.
  const uint16_t* A16 = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* B16 = reinterpret_cast<const uint16_t*>(p.b);
  const uint8_t* Aq = reinterpret_cast<const uint8_t*>(p.a);
  const uint8_t* Bq = reinterpret_cast<const uint8_t*>(p.b) + (MODE == W4A4 ? (int64_t)expert * p.N * (p.K / 2) : 0);
  const uint8_t* Bs = MODE == W4A4 ? p.bs + (int64_t)expert * p.N * (p.K / 16) : nullptr;
  const uint16_t* Be = MODE == NT_BF16 ? B16 + (int64_t)expert * p.N * p.K
                     : MODE == NN_BF16 ? B16 + (int64_t)expert * p.K * p.N
                                       : B16;

  KMajorRegs ra_k, rb_k;
  MNMajorRegs ra_mn, rb_mn;
  NVRegs ra_nv, rb_nv;

  auto issue = [&](int64_t kb) {
    if (MODE == NT_BF16) {
      kmajor_issue(ra_k, A16, p.K, m0, m_end, kb, p.K);
      kmajor_issue(rb_k, Be, p.K, n0, p.N, kb, p.K);
    } else if (MODE == NN_BF16) {
      kmajor_issue(ra_k, A16, p.K, m0, m_end, kb, p.K);
      mnmajor_issue(rb_mn, Be, p.N, kb, p.K, n0, p.N);
    } else if (MODE == TN_BF16) {
      mnmajor_issue(ra_mn, A16, p.K, kb, k_end, m0, p.K);
      mnmajor_issue(rb_mn, B16, p.N, kb, k_end, n0, p.N);
    } else {
      nv_issue(ra_nv, Aq, p.as, p.K, m0, m_end, kb);
      nv_issue(rb_nv, Bq, Bs, p.K, n0, p.N, kb);
    }
  };
  auto commit = [&](int stage) {
    uint16_t* As = smem + stage * STAGE_ELEMS;
    uint16_t* Bsm = As + BM * BK;
    if (MODE == NT_BF16) {
      kmajor_commit(ra_k, As);
      kmajor_commit(rb_k, Bsm);
    } else if (MODE == NN_BF16) {
      kmajor_commit(ra_k, As);
      mnmajor_commit(rb_mn, Bsm);
    } else if (MODE == TN_BF16) {
      mnmajor_commit(ra_mn, As);
      mnmajor_commit(rb_mn, Bsm);
    } else {
      nv_commit(ra_nv, As);
      nv_commit(rb_nv, Bsm);
    }
  };

  const int64_t nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  if (nk > 0) {
    issue(k_begin);
    commit(0);
    __syncthreads();
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int stage = (int)(kt & 1);
    if (kt + 1 < nk) issue(k_begin + (kt + 1) * BK);
    const uint16_t* As = smem + stage * STAGE_ELEMS;
    const uint16_t* Bsm = As + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      uint4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const uint4*>(As + lds_off(wm * 64 + i * 32 + (lane & 31), c));
        bf[i] = *reinterpret_cast<const uint4*>(Bsm + lds_off(wn * 64 + i * 32 + (lane & 31), c));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (MODE == W4A4)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, af[i]),
                                                                __builtin_bit_cast(f16x8_t, bf[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                                 __builtin_bit_cast(bf16x8_t, bf[j]), acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) commit(stage ^ 1);
    __syncthreads();
  }

  // Epilogue.
  float alpha = 1.0f;
  if (MODE == W4A4) alpha = p.ag[0] * p.bg[expert];
  const int64_t ldc = p.N;
  float* C32 = reinterpret_cast<float*>(p.c);
  uint16_t* C16 = reinterpret_cast<uint16_t*>(p.c);
  const int64_t cbase = MODE == TN_BF16 ? (int64_t)expert * p.K * p.N : 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= m_end) continue;
        const float v = acc[i][j][r] * alpha;
        const int64_t idx = cbase + row * ldc + col;
        if (p.c_f32) {
          C32[idx] = p.accumulate ? C32[idx] + v : v;
        } else {
          C16[idx] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
}

int launch(int mode, const Params& p0, hipStream_t st) {
  Params p = p0;
  p.n_tiles = (int)cdiv(p.N, BN);
  int64_t blocks;
  if (mode == TN_BF16) {
    p.k_tiles_tn = (int)cdiv(p.K, BM);
    blocks = (int64_t)p.E * p.k_tiles_tn * p.n_tiles;
  } else {
    blocks = (cdiv(p.M, BM) + p.E) * p.n_tiles;
  }
  if (blocks <= 0) return NVFP4MOE_OK;
  if (blocks > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  switch (mode) {
    case NT_BF16: gemm_kernel<NT_BF16><<<(unsigned)blocks, NT, 0, st>>>(p); break;
    case NN_BF16: gemm_kernel<NN_BF16><<<(unsigned)blocks, NT, 0, st>>>(p); break;
    case TN_BF16: gemm_kernel<TN_BF16><<<(unsigned)blocks, NT, 0, st>>>(p); break;
    default: gemm_kernel<W4A4><<<(unsigned)blocks, NT, 0, st>>>(p); break;
  }
  return launch_status();
}

}  // namespace
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" int grouped_gemm_w4a4(const uint8_t* a_q, const uint8_t* a_s, const float* a_g, const uint8_t* b_q,
                                 const uint8_t* b_s, const float* b_g, const int32_t* expert_offsets, int E,
                                 int64_t M_total, int64_t N, int64_t K, void* c, int c_dtype, int epilogue,
                                 float* amax_out, void* workspace, size_t ws_bytes, nvfp4moe_stream_t stream) {
  (void)amax_out;
  (void)workspace;
  (void)ws_bytes;
  if (E < 1 || M_total < 0 || N < 0 || K < 0) return NVFP4MOE_EINVAL;
  if (c_dtype != NVFP4MOE_F32 && c_dtype != NVFP4MOE_BF16) return NVFP4MOE_EINVAL;
  if (epilogue != NVFP4MOE_EPI_NONE) return NVFP4MOE_EINVAL;
  if (!expert_offsets || !a_g || !b_g) return NVFP4MOE_EINVAL;
  if (M_total > 0 && N > 0 && (!a_q || !a_s || !b_q || !b_s || !c)) return NVFP4MOE_EINVAL;
  if (K % 32 != 0 || N % 32 != 0) return NVFP4MOE_ESHAPE;
  if (M_total > 0x7FFFFFFFLL || !aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_s, 2) || !aligned(b_s, 2) ||
      !aligned(c, 16))
    return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (M_total == 0 || N == 0) return NVFP4MOE_OK;
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
  return launch(W4A4, p, as_stream(stream));
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
  if (M_total > 0x7FFFFFFFLL || !aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16)) return NVFP4MOE_ESHAPE;
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
