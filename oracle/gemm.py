"""Oracle: grouped GEMMs over the contiguous per-expert layout
(test infrastructure).

Grouped GEMM for MoE experts: "miniTE ускоряет RL в NVFP4 на B300", section
"Диагностика, выравнивание и быстрые ядра" (grouped GEMMs matter because MoE
work is split over many experts); "miniTE報告、NVFP4強化学習の安定性を検証",
fourth paragraph (grouped GEMM on the token-wise NVFP4 path).  BF16 backward:
the same Japanese page, first paragraph.

All products are taken in fp64 on operands that are exact in fp64 (NVFP4
dequantized values, bf16 values), so the only rounding is fp64's.  Each
function also returns the per-element scale sum_k |a*b| used by the
tolerance |C - C_ref| <= 1e-3 * sum_k |a*b|.
"""

import numpy as np

from . import mx, nvfp4


def _segments(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return [(e, int(off[e]), int(off[e + 1])) for e in range(off.size - 1)]


def grouped_gemm_w4a4(a_q, a_s, a_g, b_q, b_s, b_g, offsets, rows=None):
    """C[r, n] = sum_k deq(A)[r, k] * deq(B_e)[n, k] for r in expert e's rows.

    a_q [M, K/2], a_s [M, K/16], a_g [1]; b_q [E, N, K/2], b_s [E, N, K/16],
    b_g [E]; offsets [E+1].  ``rows`` (optional index array) restricts the
    result to those rows.  Returns (C fp64, absbound fp64), shaped
    [len(rows) or M, N].
    """
    off = np.asarray(offsets, dtype=np.int64)
    E = off.size - 1
    M = a_q.shape[0]
    N = b_q.shape[1]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    expert_of = np.searchsorted(off, rows, side="right") - 1
    A = nvfp4.dequantize(a_q[rows], a_s[rows], np.asarray(a_g).reshape(1)[:1])
    C = np.zeros((rows.size, N))
    AB = np.zeros((rows.size, N))
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if sel.size == 0:
            continue
        B = nvfp4.dequantize(b_q[e], b_s[e], np.asarray(b_g).reshape(E)[e:e + 1])
        C[sel] = A[sel] @ B.T
        AB[sel] = np.abs(A[sel]) @ np.abs(B).T
    return C, AB


def grouped_gemm_w4a8(a_q, a_s, b_q, b_s, offsets, rows=None, a_elem="e4m3", b_elem="e2m1"):
    """The W4A8 variant: C[r, n] = sum_k deq(A)[r, k] * deq(B_e)[n, k] for r in
    expert e's rows, A MXFP8 (E4M3 elements) and B MXFP4 (E2M1 elements),
    both with E8M0 scales per 32 along K and no global scale.

    a_q [M, K], a_s [M, K/32]; b_q [E, N, K/2], b_s [E, N, K/32]; offsets
    [E+1].  ``rows`` restricts the result to those rows (then a_q / a_s
    hold only those rows).  Returns (C fp64, absbound fp64).
    """
    off = np.asarray(offsets, dtype=np.int64)
    E = off.size - 1
    M = a_q.shape[0]
    N = b_q.shape[1]
    rows_idx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    expert_of = np.searchsorted(off, rows_idx, side="right") - 1
    A = mx.dequantize(a_q, a_s, a_elem)
    C = np.zeros((len(rows_idx), N))
    AB = np.zeros((len(rows_idx), N))
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if sel.size == 0:
            continue
        B = mx.dequantize(b_q[e], b_s[e], b_elem)
        C[sel] = A[sel] @ B.T
        AB[sel] = np.abs(A[sel]) @ np.abs(B).T
    return C, AB


def dense_gemm_w4a4(a_q, a_s, a_g, b_q, b_s, b_g):
    """The dense special case: one group holding all M rows."""
    M = a_q.shape[0]
    return grouped_gemm_w4a4(a_q, a_s, a_g, b_q[None], b_s[None],
                             np.asarray(b_g).reshape(1), [0, M])


def grouped_gemm_bf16(layout, a, b, offsets):
    """Grouped BF16 GEMM in fp64 on the (exact) bf16 operand values.

    layout "NT": a [M, K], b [E, N, K] -> C [M, N],  C_e = A_e B_e^T
    layout "NN": a [M, K], b [E, K, N] -> C [M, N],  C_e = A_e B_e
    layout "TN": a [M, P], b [M, N]    -> C [E, P, N], C_e = A_e^T B_e
                 (reduction over expert e's rows; an empty expert gives 0)
    Returns (C, absbound).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    segs = _segments(offsets)
    if layout in ("NT", "NN"):
        N = b.shape[1] if layout == "NT" else b.shape[2]
        C = np.zeros((a.shape[0], N))
        AB = np.zeros((a.shape[0], N))
        for e, lo, hi in segs:
            if hi == lo:
                continue
            Be = b[e].T if layout == "NT" else b[e]
            C[lo:hi] = a[lo:hi] @ Be
            AB[lo:hi] = np.abs(a[lo:hi]) @ np.abs(Be)
        return C, AB
    if layout == "TN":
        E = len(segs)
        C = np.zeros((E, a.shape[1], b.shape[1]))
        AB = np.zeros_like(C)
        for e, lo, hi in segs:
            if hi == lo:
                continue
            C[e] = a[lo:hi].T @ b[lo:hi]
            AB[e] = np.abs(a[lo:hi]).T @ np.abs(b[lo:hi])
        return C, AB
    raise ValueError("layout must be NT, NN or TN")


def brute_force_matmul_nt(A, B):
    """Triple loop, pure Python, fp64: C[i, j] = sum_k A[i, k] * B[j, k].
    Only for tiny shapes; an independent check of the matmul-based paths."""
    M, K = len(A), len(A[0]) if len(A) else 0
    N = len(B)
    C = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for kk in range(K):
                acc += float(A[i][kk]) * float(B[j][kk])
            C[i][j] = acc
    return np.array(C, dtype=np.float64).reshape(M, N)


def grouped_gemm_w4a4_wgrad(a_cols, a_g, b_cols, b_g):
    """The NVFP4 weight gradient: for each expert e,
    C_e[i, j] = a_g * b_g * sum_r deq(A_e^T)[i, r] * deq(B_e^T)[j, r],
    the reduction over the expert's rows r, both operands quantized column-
    wise (nvfp4.quantize_colwise: blocks of 16 rows of one column, a
    segment's padding encodes zeros).  a_cols / b_cols: per-expert lists of
    (q [N1 or N2, L_e/2], s [., L_e/16]).  An empty expert gives zeros.
    Returns (C fp64 [E, N1, N2], absbound)."""
    E = len(a_cols)
    N1, N2 = a_cols[0][0].shape[0], b_cols[0][0].shape[0]
    C = np.zeros((E, N1, N2))
    AB = np.zeros_like(C)
    for e in range(E):
        (aq, as_), (bq, bs) = a_cols[e], b_cols[e]
        if aq.shape[1] == 0:
            continue
        A = nvfp4.dequantize(aq, as_, np.asarray(a_g, np.float32).reshape(1))
        B = nvfp4.dequantize(bq, bs, np.asarray(b_g, np.float32).reshape(1))
        C[e] = A @ B.T
        AB[e] = np.abs(A) @ np.abs(B).T
    return C, AB
