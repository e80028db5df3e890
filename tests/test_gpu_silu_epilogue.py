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


CASES = [
    (300, 128, 192, [0, 1, 200, 0, 99]),      # empty experts, a 1-row expert, ragged row tails
    (770, 256, 128, [256, 1, 257, 256]),      # 256-row tile boundaries, two gate/up tile pairs
    (257, 384, 256, [257]),                   # one expert, three tile pairs, one row past two tiles
    (512, 768, 2048, [100, 300, 0, 112]),     # the model's FFN width and d_model
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
