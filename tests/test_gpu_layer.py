"""Stage-wise GPU parity of one MoE layer (W4A4 forward, BF16 backward): each
oracle stage is fed the GPU's own stored input of that stage, so integer
outputs stay bit-exact and float outputs are held to their rounding."""

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_bf16_close, assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from oracle import layer, moe
from oracle.layer import bf16_round, quantize_weights

pytestmark = gpu


def _run(T, k, E, D, F, s=1.1, seed=0):
    from nvfp4_quantized_moe_token_amd import moe_layer
    d = workloads.moe(T, s, 0.01, 32.0, with_dy=True, seed=seed, E=E, k=k, D=D, F=F, name="layer")
    dev = torch.device("cuda:0")
    x, w_gu, w_dn, dy = (to_gpu(d[n], torch.bfloat16) for n in ("x", "w_gu", "w_dn", "dy"))
    ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
    wq_gu = moe_layer.quantize_expert_weights(w_gu)
    wq_dn = moe_layer.quantize_expert_weights(w_dn)
    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=True)
    meta = moe_layer.forward(x, ids, tw, wq_gu, wq_dn, buf)
    moe_layer.backward(dy, tw, w_gu, w_dn, meta, buf)
    torch.cuda.synchronize()
    return d, meta, buf, wq_gu, wq_dn


@pytest.mark.parametrize("T,k,E,D,F", [(256, 8, 16, 256, 128), (100, 2, 5, 128, 192)])
def test_layer_stagewise(T, k, E, D, F):
    """Every stage against the oracle's own stage function (the wiring of
    oracle.layer, pinned on the CPU), fed the GPU's stored inputs."""
    require_gpu()
    d, meta, buf, wq_gu, wq_dn = _run(T, k, E, D, F)
    off, dest, src = moe.permute_metadata(d["topk_ids"], E)
    np.testing.assert_array_equal(to_np(meta["offsets"]), off)
    np.testing.assert_array_equal(to_np(meta["dest"]), dest)
    np.testing.assert_array_equal(to_np(meta["src"]), src)
    amax = to_np(buf.amax)
    assert amax[0] == np.abs(d["x"]).max()
    wg = quantize_weights(d["w_gu"])
    wd = quantize_weights(d["w_dn"])
    for gpu_w, ref_w in ((wq_gu, wg), (wq_dn, wd)):
        np.testing.assert_array_equal(to_np(gpu_w["q"]), ref_w[0])
        np.testing.assert_array_equal(to_np(gpu_w["s"]), ref_w[1])
        np.testing.assert_array_equal(to_np(gpu_w["g"]), ref_w[2])
    # the GPU's stored tensors, by stage name
    g = dict(x_perm=to_np(buf.x_perm), a1=(to_np(buf.a1_q), to_np(buf.a1_s), to_np(buf.a1_g)),
             y1=to_np(buf.y1), h=to_np(buf.h), a2=(to_np(buf.a2_q), to_np(buf.a2_s), to_np(buf.a2_g)),
             y2=to_np(buf.y2), out=to_np(buf.out), amax_x=amax[0], amax_h=amax[1],
             dy2=to_np(buf.dy2), dh=to_np(buf.dh), dw_dn=to_np(buf.dw_dn), dy1=to_np(buf.dy1),
             dx_perm=to_np(buf.dx_perm), dw_gu=to_np(buf.dw_gu), dx=to_np(buf.dx))
    assert g["amax_h"] == np.abs(g["h"]).max()
    fs = lambda n: layer.forward_stage(n, g, d["x"], d["topk_w"], wg, wd, off, dest, src)  # noqa: E731
    bs = lambda n: layer.backward_stage(n, g, d["dy"], d["topk_w"], d["w_gu"], d["w_dn"], off, dest, src)  # noqa: E731
    np.testing.assert_array_equal(g["x_perm"], fs("x_perm")[0])
    for name in ("a1", "a2"):      # quantize with the reused amax: bit-exact
        ref, _ = fs(name)
        for got, want in zip(g[name], ref):
            np.testing.assert_array_equal(got, want, err_msg=name)
    for name in ("y1", "y2"):
        ref, ab = fs(name)
        assert_gemm_close(g[name], ref, ab, bf16_out=True, what=name)
    assert_bf16_close(g["h"], fs("h")[0], what="silu gate")
    ref, bound = fs("out")
    assert_bf16_close(g["out"], ref, scale=bound, what="combine")
    # backward
    assert_bf16_close(g["dy2"], bs("dy2")[0], what="dY2")
    for name, bf in (("dh", True), ("dw_dn", False), ("dx_perm", True), ("dw_gu", False)):
        ref, ab = bs(name)
        assert_gemm_close(g[name], ref, ab, bf16_out=bf, what=name)
    dy1_ref, _ = bs("dy1")
    scale = np.abs(dy1_ref) + 1e-3 * np.abs(np.concatenate([g["dh"], g["dh"]], axis=1)) * (np.abs(g["y1"]) + 1)
    assert_bf16_close(g["dy1"], dy1_ref, scale=scale, what="dY1")
    ref, bound = bs("dx")
    assert_bf16_close(g["dx"], ref, scale=bound, what="dX")


def test_backward_with_wgrad_stream_matches_serial():
    # The weight-gradient GEMMs on a second stream give the same bits as the
    # serial backward (same kernels, only the order of independent launches).
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    d, meta, buf, wq_gu, wq_dn = _run(256, 8, 16, 256, 128)
    ref = {n: getattr(buf, n).clone() for n in ("dy2", "dh", "dy1", "dx_perm", "dx", "dw_dn", "dw_gu")}
    for n in ref:
        getattr(buf, n).fill_(7.0)
    dy, tw = to_gpu(d["dy"], torch.bfloat16), to_gpu(d["topk_w"], torch.float32)
    w_gu, w_dn = to_gpu(d["w_gu"], torch.bfloat16), to_gpu(d["w_dn"], torch.bfloat16)
    moe_layer.backward(dy, tw, w_gu, w_dn, meta, buf, wgrad_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for n, t in ref.items():
        got = getattr(buf, n)
        assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                           t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)), n


def test_backward_gathered_gate_up_matches_copy():
    # The gate+up weight gradient gathered from X through src gives the same
    # bits as the TN GEMM on the kept permuted copy.
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    d, meta, buf, wq_gu, wq_dn = _run(256, 8, 16, 256, 128)
    ref = buf.dw_gu.clone()
    buf.dw_gu.fill_(7.0)
    dy, tw = to_gpu(d["dy"], torch.bfloat16), to_gpu(d["topk_w"], torch.float32)
    w_gu, w_dn = to_gpu(d["w_gu"], torch.bfloat16), to_gpu(d["w_dn"], torch.bfloat16)
    moe_layer.backward(dy, tw, w_gu, w_dn, meta, buf, x=to_gpu(d["x"], torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(buf.dw_gu.view(torch.int32), ref.view(torch.int32))


def test_silu_extremes():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    g = np.array([-100, -20, -1, -0.0, 0, 1e-3, 1, 20, 100, 1e30, -1e30, 7, 0.5, -0.5, 3, -3] * 8, np.float32)
    u = np.linspace(-3, 3, g.size).astype(np.float32)
    y1 = np.concatenate([g.reshape(8, -1), u.reshape(8, -1)], axis=1)
    yg = to_gpu(y1, torch.bfloat16)
    h, amax = ops.silu_gate_fwd(yg)
    torch.cuda.synchronize()
    yv = to_np(yg)
    ref = moe.silu_gate_fwd(yv)
    hv = to_np(h)
    assert np.isfinite(hv).all()
    assert_bf16_close(hv, ref, what="silu extremes")
    assert to_np(amax)[0] == np.abs(hv).max()


@pytest.mark.parametrize("R,F", [(300, 96), (65536, 768)])
def test_silu_gate_bwd_amax(R, F):
    """silu_gate_bwd with its amax: dY1 bit-equal to the call without it, the
    amax equal to max |dY1| over the stored values (at the 8k update's size
    the grid is capped and each thread takes many rows), and dY1 against the
    oracle's SiLU backward."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(R + F)
    y1 = bf16_round((rng.standard_normal((R, 2 * F)) * 2).astype(np.float32))
    dh = bf16_round((rng.standard_normal((R, F)) * 0.1).astype(np.float32))
    y1[R // 2, 3] = 9.0                   # a large gate: dU = dH * silu(G) peaks
    dh[R // 2, 3] = -4.0
    yg, dg = to_gpu(y1, torch.bfloat16), to_gpu(dh, torch.bfloat16)
    d0 = ops.silu_gate_bwd(yg, dg)
    amax = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    d1 = ops.silu_gate_bwd(yg, dg, amax_out=amax)
    torch.cuda.synchronize()
    assert torch.equal(d0, d1)
    assert float(amax) == float(d1.float().abs().max())
    rows = np.arange(R) if R <= 1000 else np.unique(np.concatenate([[0, R // 2, R - 1], rng.integers(0, R, 64)]))
    ref = moe.silu_gate_bwd(y1[rows], dh[rows])
    assert_bf16_close(to_np(d1)[rows], ref, what="silu bwd")
