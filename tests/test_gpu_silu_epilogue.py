"""GPU parity of the W4A4 gate+up GEMM with the SiLU gate in its epilogue.

The fused entry points must give, bit for bit, what the unfused chain gives
(grouped_gemm_w4a4 with a bf16 output, then silu_gate_fwd): the same Y1, the
same H and the same amax.  Y1 itself is checked against the fp64 oracle GEMM
and H against the oracle's SiLU gate of that Y1, so the fused result is pinned
to the oracle through the unfused path."""

import numpy as np
import pytest
import torch

from _helpers import assert_bf16_close, assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from oracle import gemm, moe, nvfp4
from oracle.layer import quantize_weights

pytestmark = gpu


def _operands(seed, M, F, K, counts):
    rng = np.random.default_rng(seed)
    E = len(counts)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 20
    w = (rng.standard_normal((E, 2 * F, K)) * 0.05).astype(np.float32)
    a = nvfp4.quantize(x)
    b = quantize_weights(w)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t = dict(aq=to_gpu(a[0], torch.uint8), as_=to_gpu(a[1], torch.uint8), ag=to_gpu(a[2], torch.float32),
             bq=to_gpu(b[0], torch.uint8), bs=to_gpu(b[1], torch.uint8), bg=to_gpu(b[2], torch.float32),
             offs=to_gpu(offs, torch.int32))
    return a, b, offs, t


def _w(t):
    return (t["aq"], t["as_"], t["ag"], t["bq"], t["bs"], t["bg"], t["offs"])


def _many(seed, E, hi):
    counts = np.random.default_rng(seed).integers(0, hi, E)
    counts[::7] = 0
    return [int(c) for c in counts]


_MANY_1 = _many(5, 300, 120)   # ~510 tiles: every workgroup runs several in a row
_MANY_2 = _many(6, 160, 300)   # ~480 tiles of three steps, the last one partial

CASES = [
    (300, 128, 192, [0, 1, 200, 0, 99]),      # empty experts, a 1-row expert, ragged row tails
    (770, 256, 128, [256, 1, 257, 256]),      # 256-row tile boundaries, two gate/up tile pairs
    (257, 384, 256, [257]),                   # one expert, three tile pairs, one row past two tiles
    (512, 768, 2048, [100, 300, 0, 112]),     # the model's FFN width and d_model
    # more tiles than workgroups: the next tile's first stage is loaded after
    # each tile's last step (and its offsets are the tile-independent ones)
    (sum(_MANY_1), 256, 128, _MANY_1),
    (sum(_MANY_2), 384, 640, _MANY_2),
]


@pytest.mark.parametrize("M,F,K,counts", CASES)
def test_silu_epilogue_equals_unfused(M, F, K, counts):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    a, b, offs, t = _operands(M + F + K, M, F, K, counts)
    R = int(offs[-1])
    y1 = ops.grouped_gemm_w4a4(*_w(t), out_dtype=torch.bfloat16)
    h_ref, amax_ref = ops.silu_gate_fwd(y1[:R].contiguous())
    y1f, hf, amf = ops.grouped_gemm_w4a4_silu_gate(*_w(t))
    torch.cuda.synchronize()
    assert torch.equal(y1f[:R].view(torch.int16), y1[:R].view(torch.int16)), "Y1 bits differ"
    assert torch.equal(hf[:R].view(torch.int16), h_ref.view(torch.int16)), "H bits differ"
    assert to_np(amf)[0] == to_np(amax_ref)[0]
    # pinned to the oracle: Y1 against the fp64 GEMM, H against the oracle SiLU gate of Y1
    ref, ab = gemm.grouped_gemm_w4a4(a[0], a[1], a[2], b[0], b[1], b[2], offs)
    assert_gemm_close(to_np(y1f)[:R], ref[:R], ab[:R], bf16_out=True, what="fused Y1")
    assert_bf16_close(to_np(hf)[:R], moe.silu_gate_fwd(to_np(y1f)[:R]), what="fused H")
    assert to_np(amf)[0] == np.abs(to_np(hf)[:R]).max(initial=0.0)


def test_silu_epilogue_without_y1_and_through_epilogue_flag():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import _lib, ops
    M, F, K, counts = 300, 128, 192, [0, 1, 200, 0, 99]
    a, b, offs, t = _operands(11, M, F, K, counts)
    R = int(offs[-1])
    _, h_full, am_full = ops.grouped_gemm_w4a4_silu_gate(*_w(t))
    y_none, h_noy, am_noy = ops.grouped_gemm_w4a4_silu_gate(*_w(t), want_y1=False)
    assert y_none is None
    # grouped_gemm_w4a4 with the SiLU-gate epilogue: c receives H
    h_epi = torch.full((M, F), 3.0, dtype=torch.bfloat16, device="cuda")
    am_epi = torch.empty(1, dtype=torch.float32, device="cuda")
    E = len(counts)
    p = lambda x: x.data_ptr()  # noqa: E731
    rc = _lib.load().grouped_gemm_w4a4(p(t["aq"]), p(t["as_"]), p(t["ag"]), p(t["bq"]), p(t["bs"]), p(t["bg"]),
                                       p(t["offs"]), E, M, 2 * F, K, p(h_epi), _lib.BF16, _lib.EPI_SILU_GATE,
                                       p(am_epi), None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    for h, am in ((h_noy, am_noy), (h_epi, am_epi)):
        assert torch.equal(h[:R].view(torch.int16), h_full[:R].view(torch.int16))
        assert to_np(am)[0] == to_np(am_full)[0]
    assert (to_np(h_epi)[R:] == 3.0).all(), "rows past offsets[E] must stay untouched"


def test_silu_epilogue_no_rows():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    M, F, K = 64, 128, 64
    a, b, offs, t = _operands(3, M, F, K, [0, 0, 0])
    amax = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    h = torch.full((M, F), 3.0, dtype=torch.bfloat16, device="cuda")
    ops.grouped_gemm_w4a4_silu_gate(*_w(t), want_y1=False, h=h, amax_out=amax)
    torch.cuda.synchronize()
    assert to_np(amax)[0] == 0.0
    assert (to_np(h) == 3.0).all()


@pytest.mark.parametrize("M,F,K,counts", CASES)
def test_silu_epilogue_requantizes_h_with_handed_in_amax(M, F, K, counts):
    """H requantized inside the epilogue with a handed-in amax equals
    nvfp4_quantize(H, amax_in) of the unfused chain, bit for bit -- with the
    exact amax of H, a larger (stale) one, a smaller one that saturates, and
    with or without the bf16 Y1 and H stored -- and the oracle's quantize of
    that H.  amax_out receives max |H| of the call either way."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    a, b, offs, t = _operands(M * 3 + F + K, M, F, K, counts)
    R = int(offs[-1])
    y1, h_ref, amax_ref = ops.grouped_gemm_w4a4_silu_gate(*_w(t))
    torch.cuda.synchronize()
    amax_h = float(to_np(amax_ref)[0])
    h_np = to_np(h_ref)[:R]
    for factor, store in ((1.0, True), (1.5, False), (0.25, False), (1.0, False)):
        amax_in = torch.tensor([amax_h * factor], dtype=torch.float32, device="cuda")
        y1s = torch.full_like(y1, 3.0) if store else None
        hs = torch.full_like(h_ref, 3.0) if store else None
        q_ref, s_ref, g_ref, _ = ops.nvfp4_quantize(h_ref[:R].contiguous(), amax_in=amax_in)
        q, s, g, am = ops.grouped_gemm_w4a4_silu_gate_nvfp4(*_w(t), amax_in, y1=y1s, h=hs)
        torch.cuda.synchronize()
        assert torch.equal(q[:R], q_ref), (factor, "codes")
        assert torch.equal(s[:R], s_ref), (factor, "scales")
        assert to_np(g)[0] == to_np(g_ref)[0]
        assert to_np(am)[0] == amax_h
        rq, rs, rg, _ = nvfp4.quantize(h_np, amax=[np.float32(amax_h * factor)])
        np.testing.assert_array_equal(to_np(q)[:R], rq)
        np.testing.assert_array_equal(to_np(s)[:R], rs)
        if store:
            assert torch.equal(y1s[:R].view(torch.int16), y1[:R].view(torch.int16))
            assert torch.equal(hs[:R].view(torch.int16), h_ref[:R].view(torch.int16))


def test_layer_forward_with_delayed_amax():
    """moe_layer.forward with amax_h_in: the down GEMM's input is the
    epilogue's NVFP4 of H, equal to the two-launch path's with the same amax;
    the output equals that path's output bit for bit."""
    require_gpu()
    import workloads
    from nvfp4_quantized_moe_token_amd import moe_layer, ops
    T, k, E, D, F = 300, 4, 12, 256, 128
    d = workloads.moe(T, 1.1, 0.01, 16.0, E=E, k=k, D=D, F=F, name="delayed")
    x, ids = to_gpu(d["x"], torch.bfloat16), to_gpu(d["topk_ids"], torch.int32)
    tw = to_gpu(d["topk_w"], torch.float32)
    wq_gu = moe_layer.quantize_expert_weights(to_gpu(d["w_gu"], torch.bfloat16))
    wq_dn = moe_layer.quantize_expert_weights(to_gpu(d["w_dn"], torch.bfloat16))
    dev = torch.device("cuda:0")
    ref = moe_layer.Buffers(T, k, E, D, F, dev)
    moe_layer.forward(x, ids, tw, wq_gu, wq_dn, ref, keep_y1=True, keep_x_perm=False)
    stale = (ref.amax[1:2] * 1.25).contiguous()
    # the two-launch path with the stale amax
    q2, s2, g2, _ = ops.nvfp4_quantize(ref.h, amax_in=stale)
    fused = moe_layer.Buffers(T, k, E, D, F, dev)
    moe_layer.forward(x, ids, tw, wq_gu, wq_dn, fused, keep_y1=False, keep_x_perm=False, amax_h_in=stale)
    torch.cuda.synchronize()
    assert torch.equal(fused.a2_q, q2) and torch.equal(fused.a2_s, s2) and torch.equal(fused.a2_g, g2)
    assert to_np(fused.amax)[1] == to_np(ref.amax)[1]
    meta = ops.moe_permute(ids, E)
    y2 = ops.grouped_gemm_w4a4(q2, s2, g2, wq_dn["q"], wq_dn["s"], wq_dn["g"], meta["offsets"],
                               out_dtype=torch.bfloat16)
    out = ops.moe_unpermute(y2, meta["dest"], T, k, topk_w=tw)
    torch.cuda.synchronize()
    assert torch.equal(fused.out.view(torch.int16), out.view(torch.int16))
