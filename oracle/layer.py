"""Oracle: one MoE layer, W4A4 forward and BF16 backward, composed from the
other oracle modules (test infrastructure).

Dataflow ("miniTE報告、NVFP4強化学習の安定性を検証", first and fourth
paragraphs: token-wise NVFP4 forward over a contiguous permuted layout with
amax reuse; BF16 backward):

  forward   X --permute--> X_perm --quantize(amax_X)--> A1
            Y1 = A1 . Wgu_e^T          (grouped W4A4, gate rows then up rows)
            H  = silu(G) * U           (amax_H taken from H as stored)
            A2 = quantize(H, amax_H);  Y2 = A2 . Wdn_e^T
            out[t] = sum_j w[t, j] * Y2[dest[t*k + j]]
  backward  dY2[p] = w[src[p]] * dY[src[p] // k]
            dH = dY2 . Wdn_e;  dWdn_e = dY2_e^T . H_e
            dY1 = silu-gate backward;  dX_perm = dY1 . Wgu_e;  dWgu_e = dY1_e^T . X_perm_e
            dX[t] = sum_j dX_perm[dest[t*k + j]]

Where the GPU path stores a tensor as bf16 the composition rounds it to
bf16 too (round to nearest even), so that quantization downstream sees the
same kind of values; every product itself is fp64.  Parity tests compare the
GPU stage by stage, feeding the GPU's own stored intermediates into the next
oracle stage, because a requantized tensor's codes may flip at rounding
boundaries.
"""

import numpy as np

from . import gemm, moe, nvfp4


def bf16_round(x):
    """Round float values to the nearest bf16 (ties to even), returned as
    float32.  Finite inputs only."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return rounded.astype(np.uint32).view(np.float32).reshape(f.shape)


def quantize_weights(w):
    """Quantize stacked expert weights [E, N, K]: one global scale per expert."""
    E, N, K = w.shape
    q, s, g, amax = nvfp4.quantize(np.asarray(w, np.float32).reshape(E * N, K), groups=E)
    return q.reshape(E, N, K // 2), s.reshape(E, N, K // 16), g, amax


def forward(x, topk_ids, topk_w, w_gu, w_dn, wq_gu=None, wq_dn=None):
    """MoE layer forward.  x [T, D] (bf16 values as float32), topk_ids /
    topk_w [T, k], w_gu [E, 2F, D], w_dn [E, D, F] (bf16 values).
    Returns a dict with every intermediate."""
    T, k = topk_ids.shape
    E = w_gu.shape[0]
    off, dest, src = moe.permute_metadata(topk_ids, E)
    x_perm = moe.gather_rows(x, src, k).astype(np.float32)
    amax_x = np.float32(np.abs(np.asarray(x, np.float32)).max()) if x.size else np.float32(0)
    a1 = nvfp4.quantize(x_perm, amax=[amax_x])
    b1 = wq_gu if wq_gu is not None else quantize_weights(w_gu)
    y1_64, _ = gemm.grouped_gemm_w4a4(a1[0], a1[1], a1[2], b1[0], b1[1], b1[2], off)
    y1 = bf16_round(y1_64)
    h = bf16_round(moe.silu_gate_fwd(y1))
    amax_h = np.float32(np.abs(h).max()) if h.size else np.float32(0)
    a2 = nvfp4.quantize(h, amax=[amax_h])
    b2 = wq_dn if wq_dn is not None else quantize_weights(w_dn)
    y2_64, _ = gemm.grouped_gemm_w4a4(a2[0], a2[1], a2[2], b2[0], b2[1], b2[2], off)
    y2 = bf16_round(y2_64)
    out = bf16_round(moe.unpermute(y2, dest, k, topk_w))
    return dict(offsets=off, dest=dest, src=src, x_perm=x_perm, amax_x=amax_x,
                a1=a1, y1=y1, h=h, amax_h=amax_h, a2=a2, y2=y2, out=out)


def backward(fwd, dy, topk_w, w_gu, w_dn):
    """BF16 backward of ``forward`` given the upstream gradient dy [T, D]."""
    k = topk_w.shape[1]
    off, dest, src = fwd["offsets"], fwd["dest"], fwd["src"]
    dy2 = bf16_round(moe.gather_rows(dy, src, k, topk_w))
    dh = bf16_round(gemm.grouped_gemm_bf16("NN", dy2, w_dn, off)[0])
    dw_dn = gemm.grouped_gemm_bf16("TN", dy2, fwd["h"], off)[0].astype(np.float32)
    dy1 = bf16_round(moe.silu_gate_bwd(fwd["y1"], dh))
    dx_perm = bf16_round(gemm.grouped_gemm_bf16("NN", dy1, w_gu, off)[0])
    dw_gu = gemm.grouped_gemm_bf16("TN", dy1, fwd["x_perm"], off)[0].astype(np.float32)
    dx = bf16_round(moe.unpermute(dx_perm, dest, k, None))
    return dict(dy2=dy2, dh=dh, dw_dn=dw_dn, dy1=dy1, dx_perm=dx_perm, dw_gu=dw_gu, dx=dx)
