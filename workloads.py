"""Seeded synthetic inputs for the NVFP4 MoE hot path.

This module only draws random inputs; it holds none of the method's
arithmetic (no quantization, permutation or GEMM).  Both the HIP path and the
CPU oracle are fed from it.  The router below (top-k of biased logits,
softmax of the chosen raw logits) belongs to the harness, not to the path:
the path starts from routing ids and weights.

Shapes are those of the models the pages study (Qwen3-30B-A3B: d_model 2048,
128 experts, top-8, expert FFN 768; Qwen3-4B: hidden 2560, MLP 9728); the
pages' own data (RL on DAPO math) is not used, only these shapes.

Recipe (numpy Generator, seed 0 unless stated, draws in the order listed,
fp32 draws rounded to bf16 with round-to-nearest-even where the tensor is
bf16):
  dense_small   X [128,256] N(0,1); 1% of entries x20; W [256,256] N(0,0.02); fp32
  qwen3_4b_up   X [4096,2560] N(0,1); 0.5% x16; W [9728,2560] N(0,0.02); bf16
  moe_4k        T=4096; logits N(0,1) [T,128]; expert bias -1.1*ln(rank),
                rank a random permutation of 1..128; X [T,2048] N(0,1);
                W_gu [128,1536,2048], W_dn [128,2048,768] N(0,0.02); bf16
  moe_16k_skew  as moe_4k with T=16384, bias -1.6*ln(rank), X with 1% x32
  moe_8k_update as moe_4k with T=8192, no bias, plus dY [T,2048] N(0,1e-3)
"""

import numpy as np

D_MODEL = 2048
N_EXPERTS = 128
TOP_K = 8
FFN = 768


def _bf16(a):
    """Round an fp32 array to bf16 values (kept as fp32), ties to even."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _outliers(rng, x, frac, factor):
    if frac > 0:
        mask = rng.random(x.shape, dtype=np.float32) < frac
        x[mask] *= np.float32(factor)
    return x


def route(rng, T, E=N_EXPERTS, k=TOP_K, zipf_s=0.0):
    """Router stand-in: top-k of (logits + bias), ties to the lower expert id;
    weights = softmax over the k chosen raw logits (fp32)."""
    logits = rng.standard_normal((T, E), dtype=np.float32)
    rank = rng.permutation(E) + 1
    bias = (-zipf_s * np.log(rank)).astype(np.float32)
    biased = logits + bias[None, :]
    order = np.argsort(-biased, axis=1, kind="stable")[:, :k]
    ids = order.astype(np.int32)
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    w = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def dense_small(seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((128, 256), dtype=np.float32)
    x = _outliers(rng, x, 0.01, 20.0)
    w = rng.standard_normal((256, 256), dtype=np.float32) * np.float32(0.02)
    return dict(name="dense_small", x=x, w=w)


def qwen3_4b_up(seed=0, M=4096, N=9728, K=2560):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x = _bf16(_outliers(rng, x, 0.005, 16.0))
    w = _bf16(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    return dict(name="qwen3_4b_up", x=x, w=w)


def moe(T, zipf_s, outlier_frac=0.0, outlier_factor=1.0, with_dy=False, seed=0,
        E=N_EXPERTS, k=TOP_K, D=D_MODEL, F=FFN, weights=True, name=None):
    rng = np.random.default_rng(seed)
    ids, w = route(rng, T, E, k, zipf_s)
    x = rng.standard_normal((T, D), dtype=np.float32)
    x = _bf16(_outliers(rng, x, outlier_frac, outlier_factor))
    out = dict(name=name or f"moe_T{T}", T=T, E=E, k=k, D=D, F=F,
               topk_ids=ids, topk_w=w, x=x)
    if weights:
        out["w_gu"] = _bf16(rng.standard_normal((E, 2 * F, D), dtype=np.float32) * np.float32(0.02))
        out["w_dn"] = _bf16(rng.standard_normal((E, D, F), dtype=np.float32) * np.float32(0.02))
    if with_dy:
        out["dy"] = _bf16(rng.standard_normal((T, D), dtype=np.float32) * np.float32(1e-3))
    return out


def moe_4k(seed=0, **kw):
    return moe(4096, 1.1, seed=seed, name="moe_4k", **kw)


def moe_16k_skew(seed=0, **kw):
    return moe(16384, 1.6, 0.01, 32.0, seed=seed, name="moe_16k_skew", **kw)


def moe_8k_update(seed=0, **kw):
    return moe(8192, 0.0, with_dy=True, seed=seed, name="moe_8k_update", **kw)


CONFIGS = {
    "dense_small": dense_small,
    "qwen3_4b_up": qwen3_4b_up,
    "moe_4k": moe_4k,
    "moe_16k_skew": moe_16k_skew,
    "moe_8k_update": moe_8k_update,
}
