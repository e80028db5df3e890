"""Stage-wise GPU parity of one MoE layer (W4A4 forward, BF16 backward): each
oracle stage is fed the GPU's own stored input of that stage, so integer
outputs stay bit-exact and float outputs are held to their rounding."""

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_bf16_close, assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from oracle import gemm, moe, nvfp4
from oracle.layer import quantize_weights

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
    require_gpu()
    d, meta, buf, wq_gu, wq_dn = _run(T, k, E, D, F)
    off, dest, src = moe.permute_metadata(d["topk_ids"], E)
    np.testing.assert_array_equal(to_np(meta["offsets"]), off)
    np.testing.assert_array_equal(to_np(meta["dest"]), dest)
    # permute + amax + quantize (bit-exact)
    xp = to_np(buf.x_perm)
    np.testing.assert_array_equal(xp, d["x"][src // k])
    amax = to_np(buf.amax)
    assert amax[0] == np.abs(d["x"]).max()
    a1 = nvfp4.quantize(xp, amax=[amax[0]])
    np.testing.assert_array_equal(to_np(buf.a1_q), a1[0])
    np.testing.assert_array_equal(to_np(buf.a1_s), a1[1])
    wg = quantize_weights(d["w_gu"])
    wd = quantize_weights(d["w_dn"])
    for gpu_w, ref_w in ((wq_gu, wg), (wq_dn, wd)):
        np.testing.assert_array_equal(to_np(gpu_w["q"]), ref_w[0])
        np.testing.assert_array_equal(to_np(gpu_w["s"]), ref_w[1])
        np.testing.assert_array_equal(to_np(gpu_w["g"]), ref_w[2])
    # GEMM1
    y1_ref, ab1 = gemm.grouped_gemm_w4a4(a1[0], a1[1], a1[2], wg[0], wg[1], wg[2], off)
    y1 = to_np(buf.y1)
    assert_gemm_close(y1, y1_ref, ab1, bf16_out=True, what="gate+up")
    # SiLU gate + amax of H
    h = to_np(buf.h)
    assert_bf16_close(h, moe.silu_gate_fwd(y1), what="silu gate")
    assert amax[1] == np.abs(h).max()
    # requantize H with the reused amax (bit-exact), GEMM2
    a2 = nvfp4.quantize(h, amax=[amax[1]])
    np.testing.assert_array_equal(to_np(buf.a2_q), a2[0])
    np.testing.assert_array_equal(to_np(buf.a2_s), a2[1])
    y2_ref, ab2 = gemm.grouped_gemm_w4a4(a2[0], a2[1], a2[2], wd[0], wd[1], wd[2], off)
    y2 = to_np(buf.y2)
    assert_gemm_close(y2, y2_ref, ab2, bf16_out=True, what="down")
    # unpermute-combine
    out_ref = moe.unpermute(y2, dest, k, d["topk_w"])
    assert_bf16_close(to_np(buf.out), out_ref, scale=moe.unpermute_absbound(y2, dest, k, d["topk_w"]),
                      what="combine")
    # backward
    dy2 = to_np(buf.dy2)
    assert_bf16_close(dy2, moe.gather_rows(d["dy"], src, k, d["topk_w"]), what="dY2")
    dh_ref, abh = gemm.grouped_gemm_bf16("NN", dy2, d["w_dn"], off)
    dh = to_np(buf.dh)
    assert_gemm_close(dh, dh_ref, abh, bf16_out=True, what="dH")
    dwd_ref, abwd = gemm.grouped_gemm_bf16("TN", dy2, h, off)
    assert_gemm_close(to_np(buf.dw_dn), dwd_ref, abwd, what="dW_dn")
    dy1 = to_np(buf.dy1)
    dy1_ref = moe.silu_gate_bwd(y1, dh)
    scale = np.abs(dy1_ref) + 1e-3 * np.abs(np.concatenate([dh, dh], axis=1)) * (np.abs(y1) + 1)
    assert_bf16_close(dy1, dy1_ref, scale=scale, what="dY1")
    dxp_ref, abx = gemm.grouped_gemm_bf16("NN", dy1, d["w_gu"], off)
    dxp = to_np(buf.dx_perm)
    assert_gemm_close(dxp, dxp_ref, abx, bf16_out=True, what="dX_perm")
    dwg_ref, abwg = gemm.grouped_gemm_bf16("TN", dy1, xp, off)
    assert_gemm_close(to_np(buf.dw_gu), dwg_ref, abwg, what="dW_gu")
    dx_ref = moe.unpermute(dxp, dest, k, None)
    assert_bf16_close(to_np(buf.dx), dx_ref, scale=moe.unpermute_absbound(dxp, dest, k, None), what="dX")


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
