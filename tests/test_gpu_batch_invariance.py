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


def test_probe_tokens_bit_identical_across_workload_routings():
    """64 probe tokens (their rows, routing and upstream gradient) embedded
    at seeded positions in the moe_4k, moe_16k_skew and moe_8k_update
    batches -- unbiased, Zipf 1.1 and Zipf 1.6 routings of 4096, 16384 and
    8192 tokens over the same 128 experts -- with amax_X and amax_H held
    fixed: the probes' NVFP4 codes and scales of X and H, their bf16 H rows,
    their layer outputs and their dX rows from the BF16 backward are
    identical bit for bit in the three runs, although their rows land at
    other offsets, in other row blocks and tiles.  The full layer step runs
    as the benchmark launches it (fused permute-quantize with amax_in, the
    gate+up GEMM with the SiLU gate and the NVFP4 of H in its epilogue, the
    BF16 backward)."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    P = 64
    base = workloads.moe_8k_update()
    E, k, D, F = base["E"], base["k"], base["D"], base["F"]
    rng = np.random.default_rng(11)
    probe = workloads.moe(P, 0.0, 0.02, 24.0, with_dy=True, seed=99, E=E, k=k, D=D, F=F, weights=False,
                          name="probe")
    batches = [workloads.moe_4k(weights=False), workloads.moe_16k_skew(weights=False), base]
    w_gu, w_dn = to_gpu(base["w_gu"], torch.bfloat16), to_gpu(base["w_dn"], torch.bfloat16)
    wq_gu = moe_layer.quantize_expert_weights(w_gu)
    wq_dn = moe_layer.quantize_expert_weights(w_dn)
    amax_x = torch.tensor([256.0], dtype=torch.float32, device="cuda")   # above every |x| of the batches
    amax_h = torch.tensor([2.0], dtype=torch.float32, device="cuda")
    dev = torch.device("cuda:0")
    seen = []
    for d in batches:
        T = d["T"]
        assert np.abs(d["x"]).max() <= 256.0
        pos = np.sort(rng.choice(T, P, replace=False))
        x, ids, tw = d["x"].copy(), d["topk_ids"].copy(), d["topk_w"].copy()
        dy = d["dy"].copy() if "dy" in d else np.zeros((T, D), np.float32)
        x[pos], ids[pos], tw[pos], dy[pos] = probe["x"], probe["topk_ids"], probe["topk_w"], probe["dy"]
        buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=True)
        xg, twg = to_gpu(x, torch.bfloat16), to_gpu(tw, torch.float32)
        meta = moe_layer.forward(xg, to_gpu(ids, torch.int32), twg, wq_gu, wq_dn, buf, amax_x_in=amax_x,
                                 amax_h_in=amax_h)
        moe_layer.backward(to_gpu(dy, torch.bfloat16), twg, w_gu, w_dn, meta, buf)
        torch.cuda.synchronize()
        p = torch.from_numpy(pos).cuda()
        rows = meta["dest"].view(T, k)[p].reshape(-1).long()
        seen.append(dict(rows=rows.cpu(), a1_q=buf.a1_q[rows].cpu(), a1_s=buf.a1_s[rows].cpu(),
                         h=buf.h[rows].view(torch.int16).cpu(), a2_q=buf.a2_q[rows].cpu(),
                         a2_s=buf.a2_s[rows].cpu(), out=buf.out[p].view(torch.int16).cpu(),
                         dx=buf.dx[p].view(torch.int16).cpu(), gs=(buf.a1_g.cpu(), buf.a2_g.cpu())))
        del buf
    ref = seen[0]
    for other in seen[1:]:
        assert not torch.equal(other["rows"], ref["rows"]), "probe rows must land elsewhere"
        for key in ("a1_q", "a1_s", "h", "a2_q", "a2_s", "out", "dx"):
            assert torch.equal(other[key], ref[key]), key
        assert torch.equal(other["gs"][0], ref["gs"][0]) and torch.equal(other["gs"][1], ref["gs"][1])
