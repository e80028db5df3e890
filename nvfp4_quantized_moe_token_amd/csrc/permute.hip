// MoE token permutation: routing metadata, row gather, unpermute-combine.
//
// Contiguous per-expert data layout with the per-expert offsets produced and
// consumed on the device, and the activation amax fused into the gather
// ("miniTE報告、NVFP4強化学習の安定性を検証", fourth paragraph).
//
// Metadata is a deterministic stable counting sort of the flattened
// assignments i = t*k + j by expert id:
//   1. count_kernel  -- per chunk of kChunk assignments, a histogram over
//                       experts (LDS atomics; counts are order-free); for
//                       the fused permute-quantize also max |x| of X in parts.
//   2. scan_kernel   -- one workgroup: per-expert totals -> offsets, and
//                       the first row of every (chunk, expert) pair; src
//                       entries past the valid assignments become -1; the
//                       max of the amax parts.
//   3. rank_kernel   -- per chunk, four waves walk their 256 assignments in
//                       64-lane steps; equal ids inside a step are matched
//                       with ballots over the id bits, so the rank of an
//                       assignment is a popcount, never an atomic: the
//                       result does not depend on scheduling.
// For small histograms (E <= 1024, chunks * E <= 16384) steps 2 and 3 are
// one launch, rank_scan_kernel: each chunk's workgroup scans the histograms
// itself.
// Out-of-range ids are skipped (dest = -1) and flagged in the status word.
#include <mutex>

#include "nvfp4_codec.hpp"

namespace nvfp4moe {
namespace {

constexpr int kChunk = 1024;      // assignments per chunk (4 waves x 4 steps x 64)
constexpr int kMaxExperts = 4096;
constexpr int kAmaxParts = 256;   // workgroups that reduce the activation amax with the histograms
// Byte offset of the amax parts in the permutation workspace (after the
// per-chunk histograms, 256-byte aligned).
constexpr int64_t amax_parts_offset(int64_t chunks, int E) { return (chunks * E * 4 + 255) / 256 * 256; }

__device__ __forceinline__ float max_abs_bf16x8(const uint4 v) {
  const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[j])), fabsf(bf16_hi(ws[j]))));
  return m;
}

// Workgroups below `chunks` build one chunk's histogram.  With x given (the
// fused permute-quantize), every workgroup also takes the max |x| of its
// contiguous slice of the n16 16-byte words of X and stores it in
// amax_part[blockIdx.x] (no atomics; the scan kernel reduces the parts).
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ ids, int64_t R, int E, int64_t chunks,
                                                    int32_t* __restrict__ counts, float* __restrict__ amax_out,
                                                    const uint4* __restrict__ x, int64_t n16,
                                                    float* __restrict__ amax_part) {
  __shared__ int32_t hist[kMaxExperts];
  __shared__ float red[4];
  if (blockIdx.x < chunks) {
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0 && amax_out) *amax_out = 0.0f;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += 256) {
      const int64_t a = base + i;
      if (a < R) {
        const int32_t e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) counts[(int64_t)blockIdx.x * E + e] = hist[e];
  }
  if (x) {
    const int64_t w0 = n16 * blockIdx.x / gridDim.x, w1 = n16 * (blockIdx.x + 1) / gridDim.x;
    float m = 0.0f;
    int64_t i = w0 + threadIdx.x;
    for (; i + 3 * 256 < w1; i += 4 * 256) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = x[i + u * 256];
#pragma unroll
      for (int u = 0; u < 4; ++u) m = fmaxf(m, max_abs_bf16x8(v[u]));
    }
    for (; i < w1; i += 256) m = fmaxf(m, max_abs_bf16x8(x[i]));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) amax_part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

// counts[c][e] (in) -> first permuted row of (chunk c, expert e) (out);
// offsets[e] = exclusive prefix of the per-expert totals; src[p] = -1 for
// the rows p in [offsets[E], R) that no valid assignment fills.  1024
// threads are split into `slices` threads per expert, each owning a
// contiguous range of chunks, so every sequential walk is at most
// ceil(nchunks / slices) long; the walks read kScanBatch counts at a time so
// that their loads are in flight together.
constexpr int kScanBatch = 8;
//
// With amax_part given, it also reduces the nparts activation-amax parts of
// the histogram launch into amax_out[0].
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ counts, int64_t nchunks, int E,
                                                    int32_t* __restrict__ offsets, int64_t R,
                                                    int32_t* __restrict__ src, const float* __restrict__ amax_part,
                                                    int nparts, float* __restrict__ amax_out) {
  __shared__ int32_t ssum[kMaxExperts];   // per (expert, slice) partial sums
  __shared__ int32_t ebase[kMaxExperts];  // per expert first row
  __shared__ int32_t wsum[16];
  __shared__ int32_t s_valid;
  __shared__ float amax_red[16];
  if (amax_part) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += 1024) m = fmaxf(m, amax_part[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) amax_red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = amax_red[0];
      for (int w = 1; w < 16; ++w) v = fmaxf(v, amax_red[w]);
      *amax_out = v;
    }
  }
  const int slices = E >= 1024 ? 1 : 1024 / E;
  const int64_t cps = (nchunks + slices - 1) / slices;
  // Phase 1: slice sums.
  for (int e0 = 0; e0 < E; e0 += 1024 / slices) {
    const int e = e0 + (int)threadIdx.x / slices, sl = (int)threadIdx.x % slices;
    if (e < E) {
      int32_t sum = 0;
      const int64_t c1 = (sl + 1) * cps < nchunks ? (sl + 1) * cps : nchunks;
      for (int64_t c = sl * cps; c < c1; c += kScanBatch) {
        int32_t v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) v[u] = c + u < c1 ? counts[(c + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) sum += v[u];
      }
      ssum[e * slices + sl] = sum;
    }
  }
  __syncthreads();
  // Phase 2: exclusive scan of the expert totals (each thread owns `per`
  // consecutive experts).
  const int per = (E + 1023) / 1024;
  int32_t local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = threadIdx.x * per + i;
    if (e < E)
      for (int sl = 0; sl < slices; ++sl) local += ssum[e * slices + sl];
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int32_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int32_t run = incl - local;
  for (int w = 0; w < wid; ++w) run += wsum[w];
  for (int i = 0; i < per; ++i) {
    const int e = threadIdx.x * per + i;
    if (e < E) {
      offsets[e] = run;
      ebase[e] = run;
      for (int sl = 0; sl < slices; ++sl) run += ssum[e * slices + sl];
    }
  }
  if (threadIdx.x == 1023) {
    offsets[E] = run;
    s_valid = run;
  }
  __syncthreads();
  // Rows past the valid assignments (ids outside [0, E) were skipped).
  for (int64_t p = s_valid + (int64_t)threadIdx.x; p < R; p += 1024) src[p] = -1;
  // Phase 3: every slice walks its chunk range from its own start row.
  for (int e0 = 0; e0 < E; e0 += 1024 / slices) {
    const int e = e0 + (int)threadIdx.x / slices, sl = (int)threadIdx.x % slices;
    if (e < E) {
      int32_t r = ebase[e];
      for (int q = 0; q < sl; ++q) r += ssum[e * slices + q];
      const int64_t c1 = (sl + 1) * cps < nchunks ? (sl + 1) * cps : nchunks;
      for (int64_t c = sl * cps; c < c1; c += kScanBatch) {
        int32_t v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) v[u] = c + u < c1 ? counts[(c + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
          if (c + u < c1) counts[(c + u) * E + e] = r;
          r += v[u];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ ids, int64_t R, int E,
                                                   const int32_t* __restrict__ chunk_base, int32_t* __restrict__ dest,
                                                   int32_t* __restrict__ src, int32_t* __restrict__ status) {
  // E <= 1024: four waves, one cursor row each; otherwise wave 0 walks the
  // whole chunk with a single cursor row.
  __shared__ int32_t cursor[kMaxExperts];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const bool split = E <= 1024;
  const int64_t cbase = (int64_t)blockIdx.x * kChunk;
  const int64_t wbase = cbase + wid * (kChunk / 4);
  if (split) {
    for (int e = threadIdx.x; e < 4 * E; e += 256) cursor[e] = 0;
    __syncthreads();
    for (int s = 0; s < kChunk / 4; s += 64) {
      const int64_t a = wbase + s + lane;
      const int32_t e = a < R ? ids[a] : -1;
      if (e >= 0 && e < E) atomicAdd(&cursor[wid * E + e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
      int32_t r = chunk_base[(int64_t)blockIdx.x * E + e];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int32_t c = cursor[w * E + e];
        cursor[w * E + e] = r;
        r += c;
      }
    }
  } else {
    for (int e = threadIdx.x; e < E; e += 256) cursor[e] = chunk_base[(int64_t)blockIdx.x * E + e];
  }
  __syncthreads();
  if (!split && wid != 0) return;
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const int nsteps = split ? kChunk / 4 / 64 : kChunk / 64;
  const int64_t start = split ? wbase : cbase;
  int32_t* cur = split ? &cursor[wid * E] : cursor;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = 0; s < nsteps; ++s) {
    const int64_t a = start + (int64_t)s * 64 + lane;
    const int32_t raw = a < R ? ids[a] : -1;
    const bool valid = raw >= 0 && raw < E;
    if (a < R && !valid && status) atomicOr(status, NVFP4MOE_STATUS_BAD_EXPERT);
    const int32_t e = valid ? raw : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const uint64_t m = __ballot((e >> b) & 1);
      match &= ((e >> b) & 1) ? m : ~m;
    }
    if (valid) {
      const int32_t row = cur[e] + __popcll(match & lt);
      dest[a] = row;
      src[row] = (int32_t)a;
    } else if (a < R) {
      dest[a] = -1;
    }
    // The highest lane of each group advances its expert's cursor: one
    // writer per expert, after every lane of the wave has read it.
    __builtin_amdgcn_wave_barrier();
    if (valid && (match >> lane) == 1ull) cur[e] += __popcll(match);
    __builtin_amdgcn_wave_barrier();
  }
}

// The scan folded into the ranks, for small histograms (E <= 1024 and
// nchunks * E <= kFusedScanMax): one launch fewer.  Workgroup c reads every
// chunk's histogram (at most 64 KB, from L2) and forms, for each expert,
// the total over all chunks and the sum over the chunks before c; the
// exclusive scan of the totals gives offsets[e], and offsets[e] plus the
// earlier chunks' count is this chunk's first row of expert e -- what
// scan_kernel writes for every chunk.  The ranks inside the chunk then
// follow rank_kernel's split path.  Workgroup 0 writes the offsets and
// reduces the amax parts; every workgroup writes its share of the src tail.
constexpr int64_t kFusedScanMax = 16384;
__global__ __launch_bounds__(256) void rank_scan_kernel(const int32_t* __restrict__ ids, int64_t R, int E,
                                                        int64_t nchunks, const int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ dest,
                                                        int32_t* __restrict__ src, int32_t* __restrict__ status,
                                                        const float* __restrict__ amax_part, int nparts,
                                                        float* __restrict__ amax_out) {
  __shared__ int32_t cursor[4 * 1024];
  __shared__ int32_t base[1024];
  __shared__ int32_t wsum[4];
  __shared__ float amax_red[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t c = blockIdx.x;
  if (amax_part && c == 0) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += 256) m = fmaxf(m, amax_part[i]);
    m = wave_max(m);
    if (lane == 0) amax_red[wid] = m;
  }
  // Per expert (thread e, e + 256, ... of at most 4): total and the count
  // of the chunks before this one.
  int32_t tot[4] = {0, 0, 0, 0}, before[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x + 256 * i;
    if (e < E) {
      for (int64_t q = 0; q < nchunks; q += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = q + u < nchunks ? counts[(q + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tot[i] += v[u];
          if (q + u < c) before[i] += v[u];
        }
      }
    }
  }
  // Exclusive scan of the totals in expert order: thread t owns experts t,
  // t + 256, ...; the scan runs over (i, t) with i outer.
  int32_t run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int32_t incl = tot[i];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int32_t pre = incl - tot[i];
    for (int w = 0; w < wid; ++w) pre += wsum[w];
    const int32_t round_total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const int e = threadIdx.x + 256 * i;
    if (e < E) {
      const int32_t off = run + pre;
      base[e] = off + before[i];
      if (c == 0) offsets[e] = off;
    }
    run += round_total;
    __syncthreads();  // wsum is rewritten by the next round
  }
  const int32_t valid = run;
  if (c == 0 && threadIdx.x == 0) {
    offsets[E] = valid;
    if (amax_part) *amax_out = fmaxf(fmaxf(amax_red[0], amax_red[1]), fmaxf(amax_red[2], amax_red[3]));
  }
  // Rows past the valid assignments (ids outside [0, E) were skipped).
  for (int64_t p = valid + c * 256 + threadIdx.x; p < R; p += nchunks * 256) src[p] = -1;
  // Ranks inside the chunk: rank_kernel's split path from these bases.
  const int64_t cbase = c * kChunk;
  const int64_t wbase = cbase + wid * (kChunk / 4);
  for (int e = threadIdx.x; e < 4 * E; e += 256) cursor[e] = 0;
  __syncthreads();
  for (int st = 0; st < kChunk / 4; st += 64) {
    const int64_t a = wbase + st + lane;
    const int32_t e = a < R ? ids[a] : -1;
    if (e >= 0 && e < E) atomicAdd(&cursor[wid * E + e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int32_t r = base[e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int32_t n = cursor[w * E + e];
      cursor[w * E + e] = r;
      r += n;
    }
  }
  __syncthreads();
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  int32_t* cur = &cursor[wid * E];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int st = 0; st < kChunk / 4 / 64; ++st) {
    const int64_t a = wbase + (int64_t)st * 64 + lane;
    const int32_t raw = a < R ? ids[a] : -1;
    const bool ok = raw >= 0 && raw < E;
    if (a < R && !ok && status) atomicOr(status, NVFP4MOE_STATUS_BAD_EXPERT);
    const int32_t e = ok ? raw : 0;
    uint64_t match = __ballot(ok);
    for (int b = 0; b < bits; ++b) {
      const uint64_t m = __ballot((e >> b) & 1);
      match &= ((e >> b) & 1) ? m : ~m;
    }
    if (ok) {
      const int32_t row = cur[e] + __popcll(match & lt);
      dest[a] = row;
      src[row] = (int32_t)a;
    } else if (a < R) {
      dest[a] = -1;
    }
    __builtin_amdgcn_wave_barrier();
    if (ok && (match >> lane) == 1ull) cur[e] += __popcll(match);
    __builtin_amdgcn_wave_barrier();
  }
}

// Row gather (optionally weighted and dtype-converting) with fused amax.
// One workgroup walks rows p = blockIdx.x, blockIdx.x + gridDim.x, ...;
// every thread moves 16-byte pieces of the row.
template <int IN, int OUT, bool WEIGHTED>
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ x, int64_t row_elems,
                                                     const int32_t* __restrict__ src, const float* __restrict__ w,
                                                     int k, int64_t R, uint8_t* __restrict__ out,
                                                     float* __restrict__ amax_out) {
  constexpr int ib = IN == NVFP4MOE_F32 ? 4 : IN == NVFP4MOE_BF16 ? 2 : 1;
  constexpr int ob = OUT == NVFP4MOE_F32 ? 4 : OUT == NVFP4MOE_BF16 ? 2 : 1;
  float m = 0.0f;
  if (IN == OUT && !WEIGHTED) {
    const int64_t n16 = row_elems * ib / 16;
    for (int64_t p = blockIdx.x; p < R; p += gridDim.x) {
      const int32_t s = src[p];
      uint4* o = reinterpret_cast<uint4*>(out + p * row_elems * ob);
      if (s < 0) {
        for (int64_t c = threadIdx.x; c < n16; c += 256) o[c] = make_uint4(0, 0, 0, 0);
        continue;
      }
      const uint4* in = reinterpret_cast<const uint4*>(x + (int64_t)(s / k) * row_elems * ib);
      for (int64_t c = threadIdx.x; c < n16; c += 256) {
        const uint4 v = in[c];
        o[c] = v;
        if (amax_out) {
          const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (IN == NVFP4MOE_BF16) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[j])), fabsf(bf16_hi(ws[j]))));
            else if (IN == NVFP4MOE_F32) m = fmaxf(m, fabsf(__uint_as_float(ws[j])));
          }
        }
      }
    }
  } else {
    // Element path in groups of 8 (row_elems % 8 == 0).
    const int64_t n8 = row_elems / 8;
    for (int64_t p = blockIdx.x; p < R; p += gridDim.x) {
      const int32_t s = src[p];
      const float wt = (WEIGHTED && s >= 0) ? w[s] : 1.0f;
      for (int64_t c = threadIdx.x; c < n8; c += 256) {
        float v[8];
        if (s < 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = 0.0f;
        } else {
          const uint8_t* in = x + ((int64_t)(s / k) * row_elems + c * 8) * ib;
          if (IN == NVFP4MOE_BF16) {
            const uint4 u = *reinterpret_cast<const uint4*>(in);
            const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[2 * j] = bf16_lo(ws[j]);
              v[2 * j + 1] = bf16_hi(ws[j]);
            }
          } else {
            const uint4 u0 = reinterpret_cast<const uint4*>(in)[0], u1 = reinterpret_cast<const uint4*>(in)[1];
            v[0] = __uint_as_float(u0.x); v[1] = __uint_as_float(u0.y);
            v[2] = __uint_as_float(u0.z); v[3] = __uint_as_float(u0.w);
            v[4] = __uint_as_float(u1.x); v[5] = __uint_as_float(u1.y);
            v[6] = __uint_as_float(u1.z); v[7] = __uint_as_float(u1.w);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= wt;
        }
        uint8_t* o = out + (p * row_elems + c * 8) * ob;
        if (OUT == NVFP4MOE_BF16) {
          uint4 u;
          u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
          u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
          *reinterpret_cast<uint4*>(o) = u;
          if (amax_out) {
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(__uint_as_float(f32_to_bf16_rne(v[j]) << 16)));
          }
        } else {
          reinterpret_cast<uint4*>(o)[0] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                       __float_as_uint(v[2]), __float_as_uint(v[3]));
          reinterpret_cast<uint4*>(o)[1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                                                       __float_as_uint(v[6]), __float_as_uint(v[7]));
          if (amax_out) {
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
          }
        }
      }
    }
  }
  if (amax_out) block_atomic_max<256>(amax_out, m);
}

template <int IN, int OUT, bool WEIGHTED>
void launch_gather(const void* x, int64_t row_elems, const int32_t* src, const float* w, int k, int64_t R, void* out,
                   float* amax_out, hipStream_t st) {
  // One workgroup per row; with a fused amax every workgroup ends in one
  // same-address atomic, which serializes, so that grid stays capped.
  const int64_t cap = amax_out ? 2048 : kMaxStreamGrid;
  int64_t grid = R < cap ? R : cap;
  if (grid < 1) grid = 1;
  gather_kernel<IN, OUT, WEIGHTED><<<(unsigned)grid, 256, 0, st>>>(
      reinterpret_cast<const uint8_t*>(x), row_elems, src, w, k, R, reinterpret_cast<uint8_t*>(out), amax_out);
}

int gather_dispatch(const void* x, int x_dtype, int64_t row_elems, const int32_t* src, const float* w, int k,
                    int64_t R, void* out, int out_dtype, float* amax_out, hipStream_t st) {
  if (!w && x_dtype == out_dtype) {
    if (x_dtype == NVFP4MOE_BF16)
      launch_gather<NVFP4MOE_BF16, NVFP4MOE_BF16, false>(x, row_elems, src, w, k, R, out, amax_out, st);
    else if (x_dtype == NVFP4MOE_F32)
      launch_gather<NVFP4MOE_F32, NVFP4MOE_F32, false>(x, row_elems, src, w, k, R, out, amax_out, st);
    else
      launch_gather<NVFP4MOE_U8, NVFP4MOE_U8, false>(x, row_elems, src, w, k, R, out, nullptr, st);
    return launch_status();
  }
#define NVG(I, O)                                                                                       \
  if (x_dtype == I && out_dtype == O) {                                                                \
    if (w) launch_gather<I, O, true>(x, row_elems, src, w, k, R, out, amax_out, st);                   \
    else launch_gather<I, O, false>(x, row_elems, src, w, k, R, out, amax_out, st);                    \
    return launch_status();                                                                            \
  }
  NVG(NVFP4MOE_BF16, NVFP4MOE_BF16)
  NVG(NVFP4MOE_BF16, NVFP4MOE_F32)
  NVG(NVFP4MOE_F32, NVFP4MOE_F32)
  NVG(NVFP4MOE_F32, NVFP4MOE_BF16)
#undef NVG
  return NVFP4MOE_EINVAL;
}

// Eight values of a row piece (bf16 or fp32) as fp32, and back (bf16: RNE).
template <int IN>
__device__ __forceinline__ void load8(const uint8_t* in, float (&v)[8]) {
  if (IN == NVFP4MOE_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(in);
    const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_lo(ws[q]);
      v[2 * q + 1] = bf16_hi(ws[q]);
    }
  } else {
    const uint4 u0 = reinterpret_cast<const uint4*>(in)[0], u1 = reinterpret_cast<const uint4*>(in)[1];
    v[0] = __uint_as_float(u0.x); v[1] = __uint_as_float(u0.y);
    v[2] = __uint_as_float(u0.z); v[3] = __uint_as_float(u0.w);
    v[4] = __uint_as_float(u1.x); v[5] = __uint_as_float(u1.y);
    v[6] = __uint_as_float(u1.z); v[7] = __uint_as_float(u1.w);
  }
}
template <int OUT>
__device__ __forceinline__ void store8(uint8_t* o, const float (&v)[8]) {
  if (OUT == NVFP4MOE_BF16) {
    *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  } else {
    reinterpret_cast<uint4*>(o)[0] =
        make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    reinterpret_cast<uint4*>(o)[1] =
        make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7]));
  }
}

// Permutation fused with NVFP4 quantization (token-wise path with op
// fusion: "miniTE報告、NVFP4強化学習の安定性を検証", fourth paragraph), by
// scatter: each 16-element block of X is read once (T rows, not the T*k
// permuted ones), quantized once, and its codes and scale (and its bf16 copy
// when x_perm is wanted) are written to the k permuted rows dest[t*k+j] of
// its token.  Rows past offsets[E] (skipped assignments) are written as
// zeros.  quantize(permute(X)) == permute(quantize(X)) row by row, so the
// result equals nvfp4_quantize on the gathered X_perm.  One thread per block
// of X; the amax is read after the block's loads are issued (the empty asm
// keeps the compiler from hoisting it), so the latencies overlap.
template <int NT>
__global__ __launch_bounds__(NT) void quantize_scatter_kernel(const uint4* __restrict__ x, int64_t T, int k,
                                                              int64_t bpr, const int32_t* __restrict__ dest,
                                                              const int32_t* __restrict__ offsets, int E, int64_t R,
                                                              uint4* __restrict__ x_perm,
                                                              const float* __restrict__ amax, uint2* __restrict__ q,
                                                              uint8_t* __restrict__ scales, float* __restrict__ gscale) {
  if (blockIdx.x == 0 && threadIdx.x == 0) gscale[0] = global_scale(amax[0]);
  const int64_t nblk = T * bpr;
  const int64_t tid = blockIdx.x * (int64_t)NT + threadIdx.x, stride = (int64_t)gridDim.x * NT;
  for (int64_t b = tid; b < nblk; b += stride) {
    const int64_t t = b / bpr, j = b - t * bpr;
    const uint4 w0 = x[2 * b], w1 = x[2 * b + 1];
    asm volatile("" ::: "memory");
    const float g = global_scale(amax[0]);
    const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(ws[i]);
      v[2 * i + 1] = bf16_hi(ws[i]);
    }
    uint2 codes;
    uint32_t S;
    quantize_block(v, g, codes, S);
    for (int jj = 0; jj < k; ++jj) {
      const int32_t r = dest[t * k + jj];
      if (r < 0) continue;
      const int64_t ob = (int64_t)r * bpr + j;
      if (x_perm) {
        x_perm[2 * ob] = w0;
        x_perm[2 * ob + 1] = w1;
      }
      q[ob] = codes;
      scales[ob] = (uint8_t)S;
    }
  }
  int64_t valid = offsets[E];
  valid = valid < 0 ? 0 : valid > R ? R : valid;
  for (int64_t b = valid * bpr + tid; b < R * bpr; b += stride) {
    if (x_perm) {
      x_perm[2 * b] = make_uint4(0, 0, 0, 0);
      x_perm[2 * b + 1] = make_uint4(0, 0, 0, 0);
    }
    q[b] = make_uint2(0, 0);
    scales[b] = 0;
  }
}

constexpr int kScatterPieces = 4, kScatterMaxK = 8;

// out[dest[t*k+j]] = w[t*k+j] * x[t] (w = 1 when NULL), fp32 product rounded
// to the output type: the scatter form of the weighted gather.  Each
// 8-element piece of a token row is read once and written to the token's k
// permuted rows: one piece per thread, or (PIECES: the amax variant on its
// capped grid, top-k up to kScatterMaxK) several per thread, loaded before
// any is stored.  Rows of out past offsets[E] are zeros.
// With amax_out, max |out| goes there with one atomic per workgroup: the max
// of the fp32 products is rounded once, which equals the max of the rounded
// values (rounding to bf16 is monotone).
template <int IN, int OUT, bool PIECES>
__global__ __launch_bounds__(256) void scatter_kernel(const uint8_t* __restrict__ x, int64_t T, int k, int64_t n8,
                                                      const int32_t* __restrict__ dest, const float* __restrict__ w,
                                                      const int32_t* __restrict__ offsets, int E, int64_t R,
                                                      uint8_t* __restrict__ out, float* __restrict__ amax_out) {
  constexpr int ib = IN == NVFP4MOE_F32 ? 4 : 2;
  constexpr int ob = OUT == NVFP4MOE_F32 ? 4 : 2;
  const int64_t tid = blockIdx.x * 256ll + threadIdx.x, stride = (int64_t)gridDim.x * 256;
  const int64_t n = T * n8;
  float m = 0.0f;
  if constexpr (PIECES) {
    // (k <= kScatterMaxK) kScatterPieces pieces per thread and step, 256 apart, with their
    // routing: every load of the step is issued before its first store.  A
    // wave's memory counter retires in order, so a load issued after a store
    // also waits for that store (in a load-store loop, every store of the
    // thread would wait for the previous one).  Pieces past the end and ids
    // past k load valid entries again and store nothing.
    for (int64_t base = blockIdx.x * (256ll * kScatterPieces) + threadIdx.x; base < n;
         base += (int64_t)gridDim.x * 256 * kScatterPieces) {
      float v[kScatterPieces][8], wt[kScatterPieces][kScatterMaxK];
      int32_t rw[kScatterPieces][kScatterMaxK];
      int64_t cc[kScatterPieces];
#pragma unroll
      for (int p = 0; p < kScatterPieces; ++p) {
        const int64_t i0 = base + 256 * p, i = i0 < n ? i0 : n - 1;
        const int64_t t = i / n8;
        cc[p] = i - t * n8;
        load8<IN>(x + i * 8 * ib, v[p]);
#pragma unroll
        for (int j = 0; j < kScatterMaxK; ++j) {
          const int64_t a = t * k + (j < k ? j : k - 1);
          rw[p][j] = dest[a];
          wt[p][j] = w ? w[a] : 1.0f;
        }
      }
#pragma unroll
      for (int p = 0; p < kScatterPieces; ++p) {
        if (base + 256 * p >= n) continue;
#pragma unroll
        for (int j = 0; j < kScatterMaxK; ++j) {
          const int32_t r = rw[p][j];
          if (j >= k || r < 0) continue;
          float o[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            o[q] = v[p][q] * wt[p][j];
            m = fmaxf(m, fabsf(o[q]));
          }
          store8<OUT>(out + ((int64_t)r * n8 + cc[p]) * 8 * ob, o);
        }
      }
    }
  } else {
    for (int64_t i = tid; i < n; i += stride) {
      const int64_t t = i / n8, c = i - t * n8;
      float v[8];
      load8<IN>(x + (t * n8 + c) * 8 * ib, v);
      for (int j = 0; j < k; ++j) {
        const int32_t r = dest[t * k + j];
        if (r < 0) continue;
        const float wt = w ? w[t * k + j] : 1.0f;
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          o[q] = v[q] * wt;
          m = fmaxf(m, fabsf(o[q]));
        }
        store8<OUT>(out + ((int64_t)r * n8 + c) * 8 * ob, o);
      }
    }
  }
  int64_t valid = offsets[E];
  valid = valid < 0 ? 0 : valid > R ? R : valid;
  for (int64_t i = valid * n8 + tid; i < R * n8; i += stride) {
    float z[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    store8<OUT>(out + i * 8 * ob, z);
  }
  if (amax_out) block_atomic_max<256>(amax_out, OUT == NVFP4MOE_BF16 ? bf16_lo(pack_bf16x2(m, m)) : m);
}

// out[t] = sum_j w[t][j] * y[dest[t*k+j]], fp32 fma in ascending j.
template <int IN, int OUT>
__global__ __launch_bounds__(256) void unpermute_kernel(const uint8_t* __restrict__ y, const int32_t* __restrict__ dest,
                                                        const float* __restrict__ w, int64_t T, int k, int64_t D,
                                                        uint8_t* __restrict__ out) {
  constexpr int ib = IN == NVFP4MOE_F32 ? 4 : 2;
  constexpr int ob = OUT == NVFP4MOE_F32 ? 4 : 2;
  const int64_t n8 = D / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    for (int64_t c = threadIdx.x; c < n8; c += 256) {
      float acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int32_t r = dest[t * k + j];
        if (r < 0) continue;
        const float wt = w ? w[t * k + j] : 1.0f;
        const uint8_t* in = y + ((int64_t)r * D + c * 8) * ib;
        float v[8];
        if (IN == NVFP4MOE_BF16) {
          const uint4 u = *reinterpret_cast<const uint4*>(in);
          const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] = bf16_lo(ws[q]);
            v[2 * q + 1] = bf16_hi(ws[q]);
          }
        } else {
          const uint4 u0 = reinterpret_cast<const uint4*>(in)[0], u1 = reinterpret_cast<const uint4*>(in)[1];
          v[0] = __uint_as_float(u0.x); v[1] = __uint_as_float(u0.y);
          v[2] = __uint_as_float(u0.z); v[3] = __uint_as_float(u0.w);
          v[4] = __uint_as_float(u1.x); v[5] = __uint_as_float(u1.y);
          v[6] = __uint_as_float(u1.z); v[7] = __uint_as_float(u1.w);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(wt, v[q], acc[q]);
      }
      uint8_t* o = out + (t * D + c * 8) * ob;
      if (OUT == NVFP4MOE_BF16) {
        uint4 u;
        u.x = pack_bf16x2(acc[0], acc[1]); u.y = pack_bf16x2(acc[2], acc[3]);
        u.z = pack_bf16x2(acc[4], acc[5]); u.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(o) = u;
      } else {
        reinterpret_cast<uint4*>(o)[0] = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                                     __float_as_uint(acc[2]), __float_as_uint(acc[3]));
        reinterpret_cast<uint4*>(o)[1] = make_uint4(__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                                                     __float_as_uint(acc[6]), __float_as_uint(acc[7]));
      }
    }
  }
}

}  // namespace
}  // namespace nvfp4moe

namespace nvfp4moe {
// Routing metadata for R assignments: histograms, scan (with the src tail),
// stable ranks.  amax_cleared (nullable) is zeroed by the first kernel.
// With amax_x given (n16 16-byte bf16 words), the histogram launch also
// reduces max |x| in parts (workspace after the counts) and the scan writes
// it to amax_dst: no separate amax launch.
static int launch_metadata(const int32_t* topk_ids, int64_t R, int E, float* amax_cleared, void* workspace,
                           int32_t* offsets, int32_t* dest, int32_t* src, int32_t* status, hipStream_t st,
                           const void* amax_x = nullptr, int64_t amax_n16 = 0, float* amax_dst = nullptr) {
  const int64_t chunks = cdiv(R, kChunk);
  int32_t* counts = reinterpret_cast<int32_t*>(workspace);
  float* parts = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + amax_parts_offset(chunks, E));
  const int64_t nblk = amax_x ? (chunks > kAmaxParts ? chunks : kAmaxParts) : chunks;
  count_kernel<<<(unsigned)nblk, 256, 0, st>>>(topk_ids, R, E, chunks, counts, amax_cleared,
                                               reinterpret_cast<const uint4*>(amax_x), amax_n16, parts);
  if (E <= 1024 && chunks * E <= kFusedScanMax) {
    rank_scan_kernel<<<(unsigned)chunks, 256, 0, st>>>(topk_ids, R, E, chunks, counts, offsets, dest, src, status,
                                                       amax_x ? parts : nullptr, (int)nblk, amax_dst);
    return launch_status();
  }
  scan_kernel<<<1, 1024, 0, st>>>(counts, chunks, E, offsets, R, src, amax_x ? parts : nullptr, (int)nblk,
                                  amax_dst);
  rank_kernel<<<(unsigned)chunks, 256, 0, st>>>(topk_ids, R, E, counts, dest, src, status);
  return launch_status();
}
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" size_t moe_permute_workspace_size(int64_t T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const int64_t chunks = cdiv(T * k, kChunk);
  // per-chunk histograms, then the amax parts of the fused permute-quantize
  const int64_t parts = chunks > kAmaxParts ? chunks : kAmaxParts;
  return (size_t)(amax_parts_offset(chunks > 0 ? chunks : 1, E) + parts * 4);
}

extern "C" int moe_permute(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int x_dtype,
                           int64_t row_elems, void* x_perm, int32_t* offsets, int32_t* dest, int32_t* src,
                           float* amax_out, void* workspace, size_t ws_bytes, int32_t* status,
                           nvfp4moe_stream_t stream) {
  if (T < 0 || k < 1 || E < 1 || row_elems < 0) return NVFP4MOE_EINVAL;
  if (E > kMaxExperts || k > 64) return NVFP4MOE_ESHAPE;
  if (!offsets || (T > 0 && (!topk_ids || !dest || !src))) return NVFP4MOE_EINVAL;
  if (x) {
    const int eb = dtype_bytes(x_dtype);
    if (!eb) return NVFP4MOE_EINVAL;
    if (T > 0 && !x_perm) return NVFP4MOE_EINVAL;
    if ((row_elems * eb) % 16 != 0 || !aligned(x, 16) || (x_perm && !aligned(x_perm, 16))) return NVFP4MOE_ESHAPE;
    if (amax_out && x_dtype == NVFP4MOE_U8) return NVFP4MOE_EINVAL;
  }
  const int64_t R = T * k;
  if (R > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  if (ws_bytes < moe_permute_workspace_size(T, k, E) || (R > 0 && !workspace)) return NVFP4MOE_EWORKSPACE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  if (R == 0) {
    fill_u32_kernel<<<1, 256, 0, st>>>(reinterpret_cast<uint32_t*>(offsets), 0u, E + 1);
    if (amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
    return launch_status();
  }
  int rc = launch_metadata(topk_ids, R, E, x ? amax_out : nullptr, workspace, offsets, dest, src, status, st);
  if (rc != NVFP4MOE_OK) return rc;
  if (!x) {
    if (amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
    return launch_status();
  }
  return gather_dispatch(x, x_dtype, row_elems, src, nullptr, k, R, x_perm, x_dtype, amax_out, st);
}

extern "C" int moe_gather(const void* x, int x_dtype, int64_t row_elems, const int32_t* src, const float* topk_w,
                          int k, int64_t R, void* out, int out_dtype, nvfp4moe_stream_t stream) {
  if (row_elems < 0 || R < 0 || k < 1) return NVFP4MOE_EINVAL;
  const int ib = dtype_bytes(x_dtype), ob = dtype_bytes(out_dtype);
  if (!ib || !ob) return NVFP4MOE_EINVAL;
  if (R > 0 && (!x || !src || !out)) return NVFP4MOE_EINVAL;
  if (topk_w || x_dtype != out_dtype) {
    if (x_dtype == NVFP4MOE_U8 || out_dtype == NVFP4MOE_U8) return NVFP4MOE_EINVAL;
    if (row_elems % 8 != 0) return NVFP4MOE_ESHAPE;
  }
  if ((row_elems * ib) % 16 != 0 || (row_elems * ob) % 16 != 0 || !aligned(x, 16) || !aligned(out, 16))
    return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (R == 0 || row_elems == 0) return NVFP4MOE_OK;
  return gather_dispatch(x, x_dtype, row_elems, src, topk_w, k, R, out, out_dtype, nullptr, as_stream(stream));
}

extern "C" int moe_scatter(const void* x, int x_dtype, int64_t row_elems, const int32_t* dest, const float* topk_w,
                           const int32_t* offsets, int E, int64_t T, int k, void* out, int out_dtype,
                           float* amax_out, nvfp4moe_stream_t stream) {
  if (T < 0 || k < 1 || E < 1 || row_elems < 0) return NVFP4MOE_EINVAL;
  if ((x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16) || (out_dtype != NVFP4MOE_F32 && out_dtype != NVFP4MOE_BF16))
    return NVFP4MOE_EINVAL;
  if (!offsets) return NVFP4MOE_EINVAL;
  if (T > 0 && row_elems > 0 && (!x || !dest || !out)) return NVFP4MOE_EINVAL;
  if (row_elems % 8 != 0 || !aligned(x, 16) || !aligned(out, 16) || (amax_out && !aligned(amax_out, 4)))
    return NVFP4MOE_ESHAPE;
  if (T * k > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  const int64_t R = T * k, n8 = row_elems / 8;
  hipStream_t st = as_stream(stream);
  if (amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
  if (R == 0 || n8 == 0) return launch_status();
  // The amax variant's capped grid gives each thread several pieces: then
  // the kernel that issues a step's loads before its stores (measured on the
  // 8k-token dY: 0.075 -> 0.060 ms).  Without the amax one piece per thread
  // and the plain loop are faster (0.055 against 0.058 ms).
  const bool pieces = amax_out && k <= kScatterMaxK;
  int64_t grid = cdiv(T * n8, 256 * (pieces ? kScatterPieces : 1));
  if (grid > kMaxStreamGrid) grid = kMaxStreamGrid;
  // one same-address atomic per workgroup for the amax: a capped grid (an
  // uncapped one, with the atomic skipped when the workgroup's max is not
  // larger than the value it last read, was slower still)
  if (amax_out && grid > kAmaxGrid) grid = kAmaxGrid;
  const uint8_t* xi = reinterpret_cast<const uint8_t*>(x);
  uint8_t* o = reinterpret_cast<uint8_t*>(out);
#define NVS(I, O)                                                                                                 \
  if (x_dtype == I && out_dtype == O) {                                                                          \
    if (pieces)                                                                                                  \
      scatter_kernel<I, O, true><<<(unsigned)grid, 256, 0, st>>>(xi, T, k, n8, dest, topk_w, offsets, E, R, o,     \
                                                                 amax_out);                                        \
    else                                                                                                         \
      scatter_kernel<I, O, false><<<(unsigned)grid, 256, 0, st>>>(xi, T, k, n8, dest, topk_w, offsets, E, R, o,    \
                                                                  amax_out);                                       \
    return launch_status();                                                                                      \
  }
  NVS(NVFP4MOE_BF16, NVFP4MOE_BF16)
  NVS(NVFP4MOE_BF16, NVFP4MOE_F32)
  NVS(NVFP4MOE_F32, NVFP4MOE_F32)
  NVS(NVFP4MOE_F32, NVFP4MOE_BF16)
#undef NVS
  return NVFP4MOE_EINVAL;
}

extern "C" int moe_unpermute(const void* y_perm, int y_dtype, const int32_t* dest, const float* topk_w, int64_t T,
                             int k, int64_t D, void* out, int out_dtype, nvfp4moe_stream_t stream) {
  if (T < 0 || k < 1 || D < 0) return NVFP4MOE_EINVAL;
  if ((y_dtype != NVFP4MOE_F32 && y_dtype != NVFP4MOE_BF16) || (out_dtype != NVFP4MOE_F32 && out_dtype != NVFP4MOE_BF16))
    return NVFP4MOE_EINVAL;
  if (T > 0 && D > 0 && (!y_perm || !dest || !out)) return NVFP4MOE_EINVAL;
  if (D % 8 != 0 || !aligned(y_perm, 16) || !aligned(out, 16)) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (T == 0 || D == 0) return NVFP4MOE_OK;
  hipStream_t st = as_stream(stream);
  const unsigned grid = (unsigned)(T < kMaxStreamGrid ? T : kMaxStreamGrid);
  const uint8_t* y = reinterpret_cast<const uint8_t*>(y_perm);
  uint8_t* o = reinterpret_cast<uint8_t*>(out);
  if (y_dtype == NVFP4MOE_BF16 && out_dtype == NVFP4MOE_BF16)
    unpermute_kernel<NVFP4MOE_BF16, NVFP4MOE_BF16><<<grid, 256, 0, st>>>(y, dest, topk_w, T, k, D, o);
  else if (y_dtype == NVFP4MOE_BF16)
    unpermute_kernel<NVFP4MOE_BF16, NVFP4MOE_F32><<<grid, 256, 0, st>>>(y, dest, topk_w, T, k, D, o);
  else if (out_dtype == NVFP4MOE_BF16)
    unpermute_kernel<NVFP4MOE_F32, NVFP4MOE_BF16><<<grid, 256, 0, st>>>(y, dest, topk_w, T, k, D, o);
  else
    unpermute_kernel<NVFP4MOE_F32, NVFP4MOE_F32><<<grid, 256, 0, st>>>(y, dest, topk_w, T, k, D, o);
  return launch_status();
}

namespace {

// Scratch memory of the allocation-free fused permute-quantize: the
// per-chunk histograms and the activation-amax parts that the caller's
// workspace holds otherwise.  Every GPU the library runs on keeps its own
// copy until the process ends.  Nothing in it must start at zero: each
// call writes every histogram entry and every amax part it reads.
constexpr size_t kScratchBytes = NVFP4MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each device, taken once per device (with
// that device current) by hipGetSymbolAddress.  The array's own name is a
// host-side stand-in and is never passed to a kernel.
constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices] = {};
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4MOE_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4MOE_ELAUNCH;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return NVFP4MOE_OK;
}

// The fused permute-quantize with the caller's workspace, or (workspace ==
// nullptr, use_scratch) with the library's scratch array of this device.
int permute_nvfp4_impl(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int64_t D, void* x_perm,
                       const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales, float* gscale,
                       int32_t* offsets, int32_t* dest, int32_t* src, void* workspace, size_t ws_bytes,
                       bool use_scratch, int32_t* status, nvfp4moe_stream_t stream);

}  // namespace

extern "C" int moe_permute_mx(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int x_dtype,
                              int64_t D, uint8_t* q, uint8_t* scales, int32_t* offsets, int32_t* dest, int32_t* src,
                              void* workspace, size_t ws_bytes, int32_t* status, nvfp4moe_stream_t stream) {
  if (T < 0 || k < 1 || E < 1 || D < 0) return NVFP4MOE_EINVAL;
  if (x_dtype != NVFP4MOE_BF16 && x_dtype != NVFP4MOE_F32) return NVFP4MOE_EINVAL;
  if (E > kMaxExperts || k > 64) return NVFP4MOE_ESHAPE;
  if (!offsets || (T > 0 && (!topk_ids || !dest || !src))) return NVFP4MOE_EINVAL;
  if (T > 0 && D > 0 && (!x || !q || !scales)) return NVFP4MOE_EINVAL;
  if (D % 32 != 0) return NVFP4MOE_ESHAPE;
  if (T > 0 && D > 0 && (!aligned(x, 16) || !aligned(q, 16))) return NVFP4MOE_ESHAPE;
  const int64_t R = T * k;
  if (R > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  if (ws_bytes < moe_permute_workspace_size(T, k, E) || (R > 0 && !workspace)) return NVFP4MOE_EWORKSPACE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  if (R == 0) {
    fill_u32_kernel<<<1, 256, 0, st>>>(reinterpret_cast<uint32_t*>(offsets), 0u, E + 1);
    return launch_status();
  }
  const int rc = launch_metadata(topk_ids, R, E, nullptr, workspace, offsets, dest, src, status, st);
  if (rc != NVFP4MOE_OK) return rc;
  if (D == 0) return NVFP4MOE_OK;
  return mx_quantize_scatter_launch(x, x_dtype, T, k, D, dest, offsets, E, q, scales, st);
}

extern "C" int moe_permute_nvfp4(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int64_t D,
                                 void* x_perm, const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales,
                                 float* gscale, int32_t* offsets, int32_t* dest, int32_t* src, void* workspace,
                                 size_t ws_bytes, int32_t* status, nvfp4moe_stream_t stream) {
  return permute_nvfp4_impl(topk_ids, T, k, E, x, D, x_perm, amax_in, amax_out, q, scales, gscale, offsets, dest,
                            src, workspace, ws_bytes, false, status, stream);
}

extern "C" int moe_permute_nvfp4_noalloc(const int32_t* topk_ids, int64_t T, int k, int E, const void* x,
                                         int64_t D, void* x_perm, const float* amax_in, float* amax_out,
                                         uint8_t* q, uint8_t* scales, float* gscale, int32_t* offsets,
                                         int32_t* dest, int32_t* src, int32_t* status, nvfp4moe_stream_t stream) {
  return permute_nvfp4_impl(topk_ids, T, k, E, x, D, x_perm, amax_in, amax_out, q, scales, gscale, offsets, dest,
                            src, nullptr, kScratchBytes, true, status, stream);
}

namespace {
int permute_nvfp4_impl(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int64_t D, void* x_perm,
                       const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales, float* gscale,
                       int32_t* offsets, int32_t* dest, int32_t* src, void* workspace, size_t ws_bytes,
                       bool use_scratch, int32_t* status, nvfp4moe_stream_t stream) {
  if (T < 0 || k < 1 || E < 1 || D < 0) return NVFP4MOE_EINVAL;
  if (E > kMaxExperts || k > 64) return NVFP4MOE_ESHAPE;
  if (!offsets || !gscale || (!amax_in && !amax_out)) return NVFP4MOE_EINVAL;
  if (T > 0 && (!topk_ids || !dest || !src)) return NVFP4MOE_EINVAL;
  if (T > 0 && D > 0 && (!x || !q || !scales)) return NVFP4MOE_EINVAL;
  if (D % 16 != 0) return NVFP4MOE_ESHAPE;
  if (T > 0 && D > 0 && (!aligned(x, 16) || !aligned(q, 8) || (x_perm && !aligned(x_perm, 16))))
    return NVFP4MOE_ESHAPE;
  if (!aligned(gscale, 4) || (amax_in && !aligned(amax_in, 4)) || (amax_out && !aligned(amax_out, 4)))
    return NVFP4MOE_ESHAPE;
  const int64_t R = T * k;
  if (R > 0x7FFFFFFFLL) return NVFP4MOE_ESHAPE;
  // With the scratch array, a size beyond it is rejected here (EWORKSPACE),
  // before any HIP call.
  if (ws_bytes < moe_permute_workspace_size(T, k, E) || (R > 0 && !workspace && !use_scratch))
    return NVFP4MOE_EWORKSPACE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  if (use_scratch && R > 0) {
    const int rc = scratch_address(&workspace);
    if (rc != NVFP4MOE_OK) return rc;
  }
  hipStream_t st = as_stream(stream);
  const float* amax = amax_in ? amax_in : amax_out;
  if (R == 0) {
    if (!amax_in) {
      const int rc = launch_amax(x, NVFP4MOE_BF16, T * D * 2 / 16, 1, amax_out, st);
      if (rc != NVFP4MOE_OK) return rc;
    }
    fill_u32_kernel<<<1, 256, 0, st>>>(reinterpret_cast<uint32_t*>(offsets), 0u, E + 1);
  } else {
    // The activation amax is taken once, over the T unpermuted rows of x
    // (tokens whose ids are all invalid included), by the histogram launch
    // (in parts) and the scan (their max).  Rows of no elements have no
    // parts to reduce: the amax is then 0, written here.
    const bool fused_amax = !amax_in && D > 0;
    if (!amax_in && D == 0) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
    const int rc = launch_metadata(topk_ids, R, E, nullptr, workspace, offsets, dest, src, status, st,
                                   fused_amax ? x : nullptr, T * D * 2 / 16, fused_amax ? amax_out : nullptr);
    if (rc != NVFP4MOE_OK) return rc;
  }
  // Launched even without rows: it also writes the global scale.
  const int64_t bpr = D / 16, nblk = T * bpr;
  int64_t grid = cdiv(nblk > 0 ? nblk : 1, 256);
  if (grid > kMaxStreamGrid) grid = kMaxStreamGrid;
  quantize_scatter_kernel<256><<<(unsigned)grid, 256, 0, st>>>(
      reinterpret_cast<const uint4*>(x), T, k, bpr, dest, offsets, E, R, reinterpret_cast<uint4*>(x_perm), amax,
      reinterpret_cast<uint2*>(q), scales, gscale);
  return launch_status();
}
}  // namespace
