"""Batch invariance of the forward path on the GPU.

With the two per-tensor amaxes held fixed (passed in, as a delayed or
externally agreed scale would be), a token's NVFP4 codes, its H rows and its
layer output must not depend on which other tokens share its batch: the
permutation only moves rows, every GEMM reduces each output element over K in
one fixed order wherever the row lands in a tile, and the combine sums a
token's k rows in ascending j.  The test routes the same tokens once in a
small unbiased batch and once scattered through a larger, strongly skewed one
(their rows land at other offsets, in other row blocks and tiles) and
compares bits.  This is the kernel-level part of aligning the training and
inference executions ("miniTE ускоряет RL в NVFP4 на B300", section
"Диагностика, выравнивание и быстрые ядра", and its key-facts list: the
strict-alignment mode)."""

import numpy as np
import torch

import workloads
from _helpers import gpu, require_gpu, to_gpu

pytestmark = gpu


def _forward(x, ids, tw, wq_gu, wq_dn, E, amax_x, amax_h):
    from nvfp4_quantized_moe_token_amd import ops
    T, k = ids.shape
    m = ops.moe_permute_nvfp4(ids, E, x, want_x_perm=False, amax_in=amax_x)
    _, h, _ = ops.grouped_gemm_w4a4_silu_gate(m["q"], m["scales"], m["gscale"], wq_gu["q"], wq_gu["s"], wq_gu["g"],
                                              m["offsets"], want_y1=False, want_amax=False)
    q2, s2, g2, _ = ops.nvfp4_quantize(h, amax_in=amax_h)
    y2 = ops.grouped_gemm_w4a4(q2, s2, g2, wq_dn["q"], wq_dn["s"], wq_dn["g"], m["offsets"], out_dtype=torch.bfloat16)
    out = ops.moe_unpermute(y2, m["dest"], T, k, topk_w=tw)
    torch.cuda.synchronize()
    return out, h, m


def test_token_outputs_do_not_depend_on_the_batch():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    E, k, D, F = 16, 4, 256, 128
    a = workloads.moe(300, 0.0, seed=1, E=E, k=k, D=D, F=F, name="batch_a")
    b = workloads.moe(1000, 1.6, 0.01, 16.0, seed=2, E=E, k=k, D=D, F=F, weights=False, name="batch_b")
    # 50 tokens of batch A, scattered through batch B
    rng = np.random.default_rng(3)
    pos = np.sort(rng.choice(1000, 50, replace=False))
    for name in ("x", "topk_ids", "topk_w"):
        b[name] = b[name].copy()
        b[name][pos] = a[name][:50]
    counts_b = np.bincount(b["topk_ids"].reshape(-1), minlength=E)
    assert counts_b.max() > 512, "batch B must spread experts over several row blocks"
    w_gu, w_dn = to_gpu(a["w_gu"], torch.bfloat16), to_gpu(a["w_dn"], torch.bfloat16)
    wq_gu = moe_layer.quantize_expert_weights(w_gu)
    wq_dn = moe_layer.quantize_expert_weights(w_dn)
    amax_x = torch.tensor([max(np.abs(a["x"]).max(), np.abs(b["x"]).max())], dtype=torch.float32, device="cuda")
    amax_h = torch.tensor([3.0], dtype=torch.float32, device="cuda")
    runs = []
    for d in (a, b):
        x = to_gpu(d["x"], torch.bfloat16)
        ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
        runs.append(_forward(x, ids, tw, wq_gu, wq_dn, E, amax_x, amax_h))
    (out_a, h_a, m_a), (out_b, h_b, m_b) = runs
    # layer outputs, bit for bit
    assert torch.equal(out_a[:50].view(torch.int16), out_b[torch.from_numpy(pos).cuda()].view(torch.int16))
    # and the intermediate rows of every (token, j) assignment
    dest_a = m_a["dest"].view(300, k)[:50].reshape(-1).long()
    dest_b = m_b["dest"].view(1000, k)[torch.from_numpy(pos).cuda()].reshape(-1).long()
    assert not torch.equal(dest_a, dest_b), "rows must land at other positions"
    assert torch.equal(m_a["q"][dest_a], m_b["q"][dest_b])
    assert torch.equal(m_a["scales"][dest_a], m_b["scales"][dest_b])
    assert torch.equal(h_a[dest_a].view(torch.int16), h_b[dest_b].view(torch.int16))
