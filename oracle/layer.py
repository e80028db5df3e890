"""Oracle: one MoE layer, W4A4 forward and BF16 backward, composed from the
other oracle modules (test infrastructure).

Dataflow ("miniTE報告、NVFP4強化学習の安定性を検証", first and fourth
paragraphs: token-wise NVFP4 forward over a contiguous permuted layout with
amax reuse; BF16 backward):

  forward   x_perm = X[src // k]                   (permute)
            a1 = quantize(x_perm, amax_x)          (amax_x = max|X|)
            y1 = a1 . Wgu_e^T                      (grouped W4A4, gate rows then up rows)
            h  = silu(G) * U                       (amax_h = max|h| as stored)
            a2 = quantize(h, amax_h)
            y2 = a2 . Wdn_e^T
            out[t] = sum_j w[t, j] * y2[dest[t*k + j]]
  backward  dy2[p] = w[src[p]] * dY[src[p] // k]
            dh = dy2 . Wdn_e                 dw_dn_e = dy2_e^T . h_e
            dy1 = silu-gate backward(y1, dh)
            dx_perm = dy1 . Wgu_e            dw_gu_e = dy1_e^T . x_perm_e
            dX[t] = sum_j dx_perm[dest[t*k + j]]

Each stage is one function of the stored tensors it reads
(``forward_stage`` / ``backward_stage``), and ``forward`` / ``backward`` run
the stages in order, each reading what the previous ones stored.  The GPU
parity tests call the same stage functions with the GPU's own stored
tensors, so the wiring -- which tensor feeds which product, where the
routing weight enters -- is written once, here, and is the wiring the pins
in ``tests/test_oracle_layer.py`` hold to an independent per-token loop and
to automatic differentiation.

Where the GPU path stores a tensor as bf16 the chain rounds it to bf16 too
(round to nearest even), so that quantization downstream sees the same kind
of values; every product itself is fp64.
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


FORWARD_STAGES = ("x_perm", "a1", "y1", "h", "a2", "y2", "out")
BACKWARD_STAGES = ("dy2", "dh", "dw_dn", "dy1", "dx_perm", "dw_gu", "dx")
# stages whose stored form is bf16 (the chain rounds them)
_BF16_STORED = {"y1", "h", "y2", "out", "dy2", "dh", "dy1", "dx_perm", "dx"}


def _row_experts(offsets, rows, n):
    off = np.asarray(offsets, dtype=np.int64)
    r = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    return np.searchsorted(off, r, side="right") - 1


def _rowwise_w4a4(a, b, offsets, rows):
    """Rows of a grouped W4A4 product; ``a`` holds only the listed rows
    when ``rows`` is given."""
    aq, as_, ag = a
    if rows is None:
        return gemm.grouped_gemm_w4a4(aq, as_, ag, b[0], b[1], b[2], offsets)
    ex = _row_experts(offsets, rows, len(rows))
    # each listed row is its own one-row group of its expert
    E = len(offsets) - 1
    N = b[0].shape[1]
    C = np.zeros((len(rows), N))
    AB = np.zeros((len(rows), N))
    for e in np.unique(ex):
        if e < 0 or e >= E:
            continue
        sel = np.nonzero(ex == e)[0]
        c, ab = gemm.grouped_gemm_w4a4(aq[sel], as_[sel], ag, b[0][e:e + 1], b[1][e:e + 1],
                                       np.asarray(b[2]).reshape(E)[e:e + 1], [0, sel.size])
        C[sel], AB[sel] = c, ab
    return C, AB


def _rowwise_bf16_nn(a, w, offsets, rows):
    """Rows of the grouped BF16 NN product a . W_e (``a`` restricted to
    ``rows`` when given)."""
    if rows is None:
        return gemm.grouped_gemm_bf16("NN", a, w, offsets)
    ex = _row_experts(offsets, rows, len(rows))
    C = np.zeros((len(rows), w.shape[2]))
    AB = np.zeros_like(C)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        c, ab = gemm.grouped_gemm_bf16("NN", a[sel], w[e:e + 1], [0, sel.size])
        C[sel], AB[sel] = c, ab
    return C, AB


def forward_stage(name, s, x, topk_w, wq_gu, wq_dn, offsets, dest, src, rows=None):
    """One forward stage computed from the stored tensors in ``s``.

    ``s`` maps stage names (and "amax_x", "amax_h") to stored values.  With
    ``rows`` (permuted-row indices) the row-wise stages read and return only
    those rows: every row-wise entry of ``s`` is then already restricted to
    ``rows``.  Returns (value, bound): bound is sum|a*b| per element for the
    GEMMs and the combine, None elsewhere; quantize stages return the
    (q, scales, g) triple.
    """
    k = np.asarray(topk_w).shape[1]
    if name == "x_perm":                       # contiguous per-expert layout
        sr = src if rows is None else np.asarray(src)[rows]
        return moe.gather_rows(x, sr, k), None
    if name == "a1":                           # amax reuse: max|X| of the unpermuted tokens
        q, sc, g, _ = nvfp4.quantize(s["x_perm"], amax=[s["amax_x"]])
        return (q, sc, g), None
    if name == "y1":
        return _rowwise_w4a4(s["a1"], wq_gu, offsets, rows)
    if name == "h":
        return moe.silu_gate_fwd(s["y1"]), None
    if name == "a2":
        q, sc, g, _ = nvfp4.quantize(s["h"], amax=[s["amax_h"]])
        return (q, sc, g), None
    if name == "y2":
        return _rowwise_w4a4(s["a2"], wq_dn, offsets, rows)
    if name == "out":                          # dest indexes the stored y2 rows
        return moe.unpermute(s["y2"], dest, k, topk_w), moe.unpermute_absbound(s["y2"], dest, k, topk_w)
    raise ValueError(name)


def backward_stage(name, s, dy, topk_w, w_gu, w_dn, offsets, dest, src, rows=None):
    """One stage of the BF16 backward computed from the stored tensors in
    ``s`` (the forward's x_perm, y1, h and the backward's own dy2, dh, dy1,
    dx_perm).  ``rows`` as in ``forward_stage`` (row-wise stages only; the
    weight gradients reduce over every row of ``s``, grouped by
    ``offsets``).  Returns (value, bound) like ``forward_stage``.
    """
    k = np.asarray(topk_w).shape[1]
    if name == "dy2":      # backward of the weighted combine: the weight enters here, once
        sr = src if rows is None else np.asarray(src)[rows]
        return moe.gather_rows(dy, sr, k, topk_w), None
    if name == "dh":       # backward of y2 = h . Wdn_e^T w.r.t. h
        return _rowwise_bf16_nn(s["dy2"], w_dn, offsets, rows)
    if name == "dw_dn":    # ... w.r.t. Wdn_e: reduction over the expert's rows
        return gemm.grouped_gemm_bf16("TN", s["dy2"], s["h"], offsets)
    if name == "dy1":
        return moe.silu_gate_bwd(s["y1"], s["dh"]), None
    if name == "dx_perm":  # backward of y1 = x_perm . Wgu_e^T w.r.t. x_perm
        return _rowwise_bf16_nn(s["dy1"], w_gu, offsets, rows)
    if name == "dw_gu":
        return gemm.grouped_gemm_bf16("TN", s["dy1"], s["x_perm"], offsets)
    if name == "dx":       # backward of the permutation: unweighted sum of a token's rows
        return moe.unpermute(s["dx_perm"], dest, k, None), moe.unpermute_absbound(s["dx_perm"], dest, k, None)
    raise ValueError(name)


def _store(name, value):
    """The stored (GPU-side) form of a stage's value."""
    if name in _BF16_STORED:
        return bf16_round(value)
    if name in ("dw_dn", "dw_gu"):
        return np.asarray(value, np.float32)
    if name == "x_perm":
        return np.asarray(value, np.float32)
    return value


def forward(x, topk_ids, topk_w, w_gu, w_dn, wq_gu=None, wq_dn=None):
    """MoE layer forward.  x [T, D] (bf16 values as float32), topk_ids /
    topk_w [T, k], w_gu [E, 2F, D], w_dn [E, D, F] (bf16 values).
    Returns a dict with every stored intermediate and the routing metadata."""
    E = w_gu.shape[0]
    off, dest, src = moe.permute_metadata(topk_ids, E)
    wq_gu = wq_gu if wq_gu is not None else quantize_weights(w_gu)
    wq_dn = wq_dn if wq_dn is not None else quantize_weights(w_dn)
    s = dict(offsets=off, dest=dest, src=src,
             amax_x=np.float32(np.abs(np.asarray(x, np.float32)).max()) if x.size else np.float32(0))
    for name in FORWARD_STAGES:
        v, _ = forward_stage(name, s, x, topk_w, wq_gu, wq_dn, off, dest, src)
        s[name] = _store(name, v)
        if name == "h":
            s["amax_h"] = np.float32(np.abs(s["h"]).max()) if s["h"].size else np.float32(0)
    return s


def backward(fwd, dy, topk_w, w_gu, w_dn):
    """BF16 backward of ``forward`` given the upstream gradient dy [T, D];
    weight gradients in fp32, activation gradients rounded to bf16."""
    off, dest, src = fwd["offsets"], fwd["dest"], fwd["src"]
    s = {n: fwd[n] for n in ("x_perm", "y1", "h")}
    for name in BACKWARD_STAGES:
        v, _ = backward_stage(name, s, dy, topk_w, w_gu, w_dn, off, dest, src)
        s[name] = _store(name, v)
    return {n: s[n] for n in BACKWARD_STAGES}


# ---- the NVFP4 backward variant ----
#
# The learner's backward of the pages runs in BF16 ("miniTE報告、NVFP4強化学
# 習の安定性を検証", first paragraph); the headline 1.39x of "miniTE ускоряет
# RL в NVFP4 на B300" is read as possibly including quantized backward GEMMs.
# This variant keeps the BF16 backward's wiring and replaces its four grouped
# GEMMs with W4A4 ones:
#   data gradients  dh = dy2 . Wdn_e, dx_perm = dy1 . Wgu_e: NT W4A4 with
#                   the gradient quantized row-wise (along the contraction
#                   over the projection's output features) and the weight
#                   quantized along its input dimension (Wdn_e^T, Wgu_e^T);
#   weight grads    dw_dn_e = dy2_e^T . h_e, dw_gu_e = dy1_e^T . x_perm_e:
#                   both operands quantized column-wise (16 consecutive rows
#                   of one column per block, inside the expert's segment).
# Amax reuse: each gradient's amax is taken once (at its row-wise
# quantization) and reused by its column-wise one; h and x_perm reuse the
# forward's amax_h and amax_x; the transposed weights reuse the per-expert
# amax of the forward's weights (the same values).

NVFP4_BACKWARD_STAGES = ("dy2", "a_dy2", "dh", "dw_dn", "dy1", "a_dy1", "dx_perm", "dw_gu", "dx")


def quantize_weights_t(w):
    """NVFP4 of stacked expert weights transposed per expert ([E, N, K] ->
    codes of [E, K, N], blocks along N), one global scale per expert from
    the expert's amax (the same as the untransposed weight's)."""
    return quantize_weights(np.ascontiguousarray(np.transpose(np.asarray(w, np.float32), (0, 2, 1))))


def backward_nvfp4_stage(name, s, dy, topk_w, wt_gu, wt_dn, offsets, dest, src, rows=None):
    """One stage of the NVFP4 backward from the stored tensors in ``s``
    (forward: x_perm, y1, h, amax_x, amax_h; backward: dy2, amax_dy2, a_dy2,
    dh, dy1, amax_dy1, a_dy1, dx_perm).  wt_gu / wt_dn: quantize_weights_t of
    the bf16 weights.  ``rows`` as in backward_stage.  Returns (value,
    bound) like backward_stage; the quantize stages return (q, scales, g)."""
    k = np.asarray(topk_w).shape[1]
    if name in ("dy2", "dy1", "dx"):
        return backward_stage(name, s, dy, topk_w, None, None, offsets, dest, src, rows=rows)
    if name == "a_dy2":
        q, sc, g, _ = nvfp4.quantize(s["dy2"], amax=[s["amax_dy2"]])
        return (q, sc, g), None
    if name == "a_dy1":
        q, sc, g, _ = nvfp4.quantize(s["dy1"], amax=[s["amax_dy1"]])
        return (q, sc, g), None
    if name == "dh":
        return _rowwise_w4a4(s["a_dy2"], wt_dn, offsets, rows)
    if name == "dx_perm":
        return _rowwise_w4a4(s["a_dy1"], wt_gu, offsets, rows)
    if name in ("dw_dn", "dw_gu"):
        ga, gb = ("dy2", "h") if name == "dw_dn" else ("dy1", "x_perm")
        amax_a = s["amax_" + ga]
        amax_b = s["amax_h"] if gb == "h" else s["amax_x"]
        ca, g_a = nvfp4.quantize_colwise(s[ga], offsets, amax_a)
        cb, g_b = nvfp4.quantize_colwise(s[gb], offsets, amax_b)
        return gemm.grouped_gemm_w4a4_wgrad(ca, g_a, cb, g_b)
    raise ValueError(name)


def backward_nvfp4(fwd, dy, topk_w, wt_gu, wt_dn):
    """NVFP4 backward of ``forward``: the stages above in order, each gradient's
    amax taken from its bf16 values once."""
    off, dest, src = fwd["offsets"], fwd["dest"], fwd["src"]
    s = {n: fwd[n] for n in ("x_perm", "y1", "h", "amax_x", "amax_h")}
    for name in NVFP4_BACKWARD_STAGES:
        v, _ = backward_nvfp4_stage(name, s, dy, topk_w, wt_gu, wt_dn, off, dest, src)
        s[name] = _store(name, v) if name not in ("a_dy2", "a_dy1") else v
        if name in ("dy2", "dy1"):
            s["amax_" + name] = np.float32(np.abs(s[name]).max()) if s[name].size else np.float32(0)
    return {n: s[n] for n in NVFP4_BACKWARD_STAGES + ("amax_dy2", "amax_dy1")}
