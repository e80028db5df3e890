"""Oracle: MoE token permutation, unpermute-combine and the SiLU gate
(test infrastructure).

Contiguous per-expert layout and device-side per-expert offsets:
"miniTE報告、NVFP4強化学習の安定性を検証" (aib.vote), fourth paragraph.
The order of rows inside an expert's segment is not fixed by the pages; the
reading used here is a stable sort of the flattened assignments
i = t*k + j by expert id (token order, then slot order, is kept).

Floating point is fp64 here; the GPU path is checked against it with
tolerances derived from its fp32 arithmetic and bf16 storage.
"""

import numpy as np


def permute_metadata(topk_ids, num_experts):
    """Stable counting sort of the flattened routing assignments.

    Returns (offsets int32 [E+1], dest int32 [T*k], src int32 [T*k]):
    assignment i = t*k + j goes to permuted row dest[i]; src[dest[i]] = i;
    expert e owns rows [offsets[e], offsets[e+1]).
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    if ids.size and (ids.min() < 0 or ids.max() >= num_experts):
        raise ValueError("expert id out of range")
    counts = np.bincount(ids, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    src = np.argsort(ids, kind="stable")          # library sort as one step
    dest = np.empty_like(src)
    dest[src] = np.arange(ids.size)
    return offsets.astype(np.int32), dest.astype(np.int32), src.astype(np.int32)


def gather_rows(x, src, k, weights=None):
    """Permuted copy: row p of the result is x[src[p] // k] (times the routing
    weight w[src[p]] when ``weights`` [T, k] is given), in fp64."""
    x = np.asarray(x)
    src = np.asarray(src, dtype=np.int64)
    out = x[src // k].astype(np.float64)
    if weights is not None:
        w = np.asarray(weights, dtype=np.float64).reshape(-1)
        out = out * w[src][:, None]
    return out


def unpermute(y_perm, dest, k, weights=None):
    """out[t] = sum_j w[t, j] * y_perm[dest[t*k + j]]  (w = 1 when None), fp64."""
    y = np.asarray(y_perm, dtype=np.float64)
    dest = np.asarray(dest, dtype=np.int64)
    T = dest.size // k
    rows = y[dest].reshape(T, k, y.shape[1])
    if weights is None:
        return rows.sum(axis=1)
    w = np.asarray(weights, dtype=np.float64).reshape(T, k, 1)
    return (rows * w).sum(axis=1)


def unpermute_absbound(y_perm, dest, k, weights=None):
    """sum_j |w[t, j] * y_perm[dest[t*k + j]]|, the scale of rounding error."""
    y = np.abs(np.asarray(y_perm, dtype=np.float64))
    w = None if weights is None else np.abs(np.asarray(weights, dtype=np.float64))
    return unpermute(y, dest, k, w)


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def silu_gate_fwd(y1):
    """H = silu(G) * U where y1 = [G | U] along the last axis (gate first)."""
    y1 = np.asarray(y1, dtype=np.float64)
    F = y1.shape[1] // 2
    return silu(y1[:, :F]) * y1[:, F:]


def silu_gate_bwd(y1, dh):
    """Gradient of H = silu(G) * U: returns dY1 = [dG | dU]."""
    y1 = np.asarray(y1, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    F = y1.shape[1] // 2
    G, U = y1[:, :F], y1[:, F:]
    sig = 1.0 / (1.0 + np.exp(-G))
    dsilu = sig * (1.0 + G * (1.0 - sig))
    return np.concatenate([dh * U * dsilu, dh * G * sig], axis=1)
