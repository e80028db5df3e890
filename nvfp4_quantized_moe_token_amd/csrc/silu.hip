// SiLU-gated expert activation between the two grouped GEMMs, with the amax
// of its output folded in so the requantization reuses it ("miniTE報告、
// NVFP4強化学習の安定性を検証", fourth paragraph: op fusion, amax reuse).
// H = silu(G) * U with Y1 = [G | U] per row; fp32 math, bf16 storage.
#include "common.hpp"

namespace nvfp4moe {
namespace {

__global__ __launch_bounds__(256) void silu_fwd_kernel(const uint16_t* __restrict__ y1, int64_t R, int64_t F,
                                                       uint16_t* __restrict__ h, float* __restrict__ amax_out) {
  const int64_t n8 = F / 8;
  const int64_t total = R * n8;
  float m = 0.0f;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / n8, c = (i - r * n8) * 8;
    const uint4 gw = *reinterpret_cast<const uint4*>(y1 + r * 2 * F + c);
    const uint4 uw = *reinterpret_cast<const uint4*>(y1 + r * 2 * F + F + c);
    const uint32_t g[4] = {gw.x, gw.y, gw.z, gw.w}, u[4] = {uw.x, uw.y, uw.z, uw.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float g0 = bf16_lo(g[j]), g1 = bf16_hi(g[j]);
      const float h0 = silu_gate(g0, bf16_lo(u[j]));
      const float h1 = silu_gate(g1, bf16_hi(u[j]));
      o[j] = pack_bf16x2(h0, h1);
      m = fmaxf(m, fmaxf(fabsf(bf16_lo(o[j])), fabsf(bf16_hi(o[j]))));
    }
    *reinterpret_cast<uint4*>(h + r * F + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (amax_out) block_atomic_max<256>(amax_out, m);
}

// dY1 = [dG | dU] from dH and Y1; with amax_out, max |dY1| (the max of the
// fp32 results rounded once to bf16, equal to the max of the stored values)
// with one atomic per workgroup.
template <int P>
__global__ __launch_bounds__(256) void silu_bwd_kernel(const uint16_t* __restrict__ y1, const uint16_t* __restrict__ dh,
                                                       int64_t R, int64_t F, uint16_t* __restrict__ dy1,
                                                       float* __restrict__ amax_out) {
  const int64_t n8 = F / 8;
  const int64_t total = R * n8;
  float m = 0.0f;
  // P pieces of 8 per thread and step, 256 apart: every load of the step is
  // issued before its first store.  A wave's memory counter retires in
  // order, so a load issued after a store also waits for that store; with
  // the capped grid of the amax variant a thread takes many pieces, and a
  // load-store-load loop would wait on every store.  Pieces past the end
  // load the last piece again (valid memory, an element of the tensor, so
  // the max is unchanged) and store nothing.
  for (int64_t base = blockIdx.x * (256ll * P) + threadIdx.x; base < total;
       base += (int64_t)gridDim.x * 256 * P) {
    uint4 gw[P], uw[P], dw[P];
    int64_t at[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t i0 = base + 256 * p, i = i0 < total ? i0 : total - 1;
      const int64_t r = i / n8, c = (i - r * n8) * 8;
      at[p] = r * 2 * F + c;
      gw[p] = *reinterpret_cast<const uint4*>(y1 + r * 2 * F + c);
      uw[p] = *reinterpret_cast<const uint4*>(y1 + r * 2 * F + F + c);
      dw[p] = *reinterpret_cast<const uint4*>(dh + r * F + c);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t g[4] = {gw[p].x, gw[p].y, gw[p].z, gw[p].w}, u[4] = {uw[p].x, uw[p].y, uw[p].z, uw[p].w};
      const uint32_t d[4] = {dw[p].x, dw[p].y, dw[p].z, dw[p].w};
      uint32_t og[4], ou[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float gg[2] = {bf16_lo(g[j]), bf16_hi(g[j])}, uu[2] = {bf16_lo(u[j]), bf16_hi(u[j])};
        float dd[2] = {bf16_lo(d[j]), bf16_hi(d[j])};
        float rg[2], ru[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float sg = sigmoid_f32(gg[q]);
          const float dsilu = sg * (1.0f + gg[q] * (1.0f - sg));
          rg[q] = dd[q] * uu[q] * dsilu;
          ru[q] = dd[q] * gg[q] * sg;
          m = fmaxf(m, fmaxf(fabsf(rg[q]), fabsf(ru[q])));
        }
        og[j] = pack_bf16x2(rg[0], rg[1]);
        ou[j] = pack_bf16x2(ru[0], ru[1]);
      }
      if (base + 256 * p < total) {
        *reinterpret_cast<uint4*>(dy1 + at[p]) = make_uint4(og[0], og[1], og[2], og[3]);
        *reinterpret_cast<uint4*>(dy1 + at[p] + F) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
      }
    }
  }
  if (amax_out) block_atomic_max<256>(amax_out, bf16_lo(pack_bf16x2(m, m)));
}

// With an amax the grid is capped (one same-address atomic per workgroup).
inline unsigned grid_for(int64_t work) {
  const int64_t g = cdiv(work, 256);
  return (unsigned)(g < 1 ? 1 : g > kAmaxGrid ? kAmaxGrid : g);
}

}  // namespace
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" int silu_gate_fwd(const void* y1, int64_t R, int64_t F, void* h, float* amax_out,
                             nvfp4moe_stream_t stream) {
  if (R < 0 || F < 0) return NVFP4MOE_EINVAL;
  if (R * F > 0 && (!y1 || !h)) return NVFP4MOE_EINVAL;
  if (F % 8 != 0 || !aligned(y1, 16) || !aligned(h, 16)) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  if (amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
  if (R * F > 0)
    silu_fwd_kernel<<<grid_for(R * F / 8), 256, 0, st>>>(reinterpret_cast<const uint16_t*>(y1), R, F,
                                                          reinterpret_cast<uint16_t*>(h), amax_out);
  return launch_status();
}

extern "C" int silu_gate_bwd(const void* y1, const void* dh, int64_t R, int64_t F, void* dy1, float* amax_out,
                             nvfp4moe_stream_t stream) {
  if (R < 0 || F < 0) return NVFP4MOE_EINVAL;
  if (R * F > 0 && (!y1 || !dh || !dy1)) return NVFP4MOE_EINVAL;
  if (F % 8 != 0 || !aligned(y1, 16) || !aligned(dh, 16) || !aligned(dy1, 16)) return NVFP4MOE_ESHAPE;
  if (amax_out && !aligned(amax_out, 4)) return NVFP4MOE_ESHAPE;
  const int arch = check_arch();
  if (arch != NVFP4MOE_OK) return arch;
  hipStream_t st = as_stream(stream);
  if (amax_out) fill_u32_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t*>(amax_out), 0u, 1);
  if (R * F == 0) return launch_status();
  // The amax variant's capped grid gives each thread several pieces, four
  // per step (measured on the 8k-token dY1: 0.099 -> 0.095 ms); without the
  // amax one piece per thread is faster (0.088 against 0.090 ms).
  const uint16_t* y1b = reinterpret_cast<const uint16_t*>(y1);
  const uint16_t* dhb = reinterpret_cast<const uint16_t*>(dh);
  uint16_t* dy1b = reinterpret_cast<uint16_t*>(dy1);
  if (amax_out) {
    silu_bwd_kernel<4><<<grid_for(cdiv(R * F / 8, 4)), 256, 0, st>>>(y1b, dhb, R, F, dy1b, amax_out);
  } else {
    int64_t grid = cdiv(R * F / 8, 256);
    if (grid > kMaxStreamGrid) grid = kMaxStreamGrid;
    silu_bwd_kernel<1><<<(unsigned)grid, 256, 0, st>>>(y1b, dhb, R, F, dy1b, nullptr);
  }
  return launch_status();
}
