"""One MoE layer step (W4A4 forward + BF16 backward) captured into a HIP graph
and replayed: every replay, with eager work and host synchronisation in
between, must reproduce the eager step's outputs bit for bit (the library
issues only kernel launches, no memsets or host synchronisation, so the
whole step can be captured)."""

import torch

import workloads
from _helpers import gpu, require_gpu, to_gpu

pytestmark = gpu

OUTPUTS = ("a1_q", "a1_s", "y1", "h", "a2_q", "a2_s", "y2", "out", "dy2", "dh", "dy1", "dx_perm", "dx", "dw_dn",
           "dw_gu", "amax")


def _bits(t):
    return t.view(torch.uint8) if t.dtype == torch.uint8 else t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_layer_step_graph_replays_match_eager():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    T, k, E, D, F = 512, 8, 32, 256, 256
    d = workloads.moe(T, 1.1, 0.01, 16.0, with_dy=True, seed=5, E=E, k=k, D=D, F=F, name="graph")
    dev = torch.device("cuda:0")
    x, w_gu, w_dn, dy = (to_gpu(d[n], torch.bfloat16) for n in ("x", "w_gu", "w_dn", "dy"))
    ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
    wq_gu = moe_layer.quantize_expert_weights(w_gu)
    wq_dn = moe_layer.quantize_expert_weights(w_dn)
    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=True)

    def step():
        meta = moe_layer.forward(x, ids, tw, wq_gu, wq_dn, buf)
        moe_layer.backward(dy, tw, w_gu, w_dn, meta, buf)
        return meta

    meta = step()
    torch.cuda.synchronize()
    ref = {n: getattr(buf, n).clone() for n in OUTPUTS}
    ref_meta = {n: meta[n].clone() for n in ("offsets", "dest", "src")}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gmeta = step()
    torch.cuda.synchronize()

    for rep in range(3):
        for n in OUTPUTS:  # eager work between replays: clobber every output
            getattr(buf, n).fill_(0x55 if getattr(buf, n).dtype == torch.uint8 else 3.0)
        for n in ("offsets", "dest", "src"):
            gmeta[n].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTPUTS:
            assert torch.equal(_bits(getattr(buf, n)), _bits(ref[n])), (rep, n)
        for n in ("offsets", "dest", "src"):
            assert torch.equal(gmeta[n], ref_meta[n]), (rep, n)
