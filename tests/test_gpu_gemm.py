"""GPU parity of the grouped GEMMs against the fp64 oracle:
|C - C_ref| <= 1e-3 * sum_k |a*b| per element (plus bf16 output rounding)."""

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from oracle import gemm, moe, nvfp4
from oracle.layer import bf16_round, quantize_weights

pytestmark = gpu


def _nv_operands(rng, M, N, K, E, a_scale=1.0, b_scale=0.02):
    x = (rng.standard_normal((M, K)) * a_scale).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 20
    w = (rng.standard_normal((E, N, K)) * b_scale).astype(np.float32)
    a = nvfp4.quantize(x)
    b = quantize_weights(w)
    return a, b


def _gpu_w4a4(a, b, offs, out_dtype):
    from nvfp4_quantized_moe_token_amd import ops
    out = ops.grouped_gemm_w4a4(to_gpu(a[0], torch.uint8), to_gpu(a[1], torch.uint8), to_gpu(a[2], torch.float32),
                                to_gpu(b[0], torch.uint8), to_gpu(b[1], torch.uint8), to_gpu(b[2], torch.float32),
                                to_gpu(np.asarray(offs, np.int32), torch.int32), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(out)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,N,K,counts", [
    (300, 160, 192, [0, 1, 200, 0, 99]),      # empty experts, a 1-row expert, M and N tails, K = 3 steps
    (257, 256, 256, [257]),                   # one expert, one row past two full tiles
    (640, 96, 64, [128, 128, 0, 384]),        # exact tiles, K = one step
    (770, 288, 128, [256, 1, 257, 256]),      # 256-row tile boundaries, N tail past 256
])
def test_w4a4_small(M, N, K, counts, out_dtype):
    require_gpu()
    rng = np.random.default_rng(M + N + K)
    E = len(counts)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a, b = _nv_operands(rng, M, N, K, E)
    c = _gpu_w4a4(a, b, offs, out_dtype)
    ref, ab = gemm.grouped_gemm_w4a4(a[0], a[1], a[2], b[0], b[1], b[2], offs)
    assert_gemm_close(c, ref, ab, bf16_out=out_dtype == torch.bfloat16)


@pytest.mark.parametrize("E,rows_per,N,K", [
    (300, 60, 512, 128),     # 600 tiles (several per workgroup), one step each: next-tile prefetch
    (160, 150, 512, 640),    # three steps per tile (the last one partial), ~480 tiles
    (1100, 16, 96, 64),      # more experts than the LDS offsets copy holds: global lookups, no prefetch
])
def test_w4a4_many_tiles_full(E, rows_per, N, K):
    """Every output element of launches where each workgroup runs several
    tiles in a row (the bf16-output path loads the next tile's first stage
    during the current tile's last step), with ragged expert sizes."""
    require_gpu()
    rng = np.random.default_rng(E + K)
    counts = rng.integers(0, 2 * rows_per, E)
    counts[rng.random(E) < 0.1] = 0
    M = int(counts.sum())
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a, b = _nv_operands(rng, M, N, K, E)
    c = _gpu_w4a4(a, b, offs, torch.bfloat16)
    ref, ab = gemm.grouped_gemm_w4a4(a[0], a[1], a[2], b[0], b[1], b[2], offs)
    assert_gemm_close(c, ref, ab, bf16_out=True)


def test_w4a4_rows_past_offsets_untouched():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(5)
    M, N, K = 200, 64, 64
    offs = np.array([0, 50, 120], np.int32)   # rows 120.. belong to no expert
    a, b = _nv_operands(rng, M, N, K, 2)
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    ops.grouped_gemm_w4a4(to_gpu(a[0], torch.uint8), to_gpu(a[1], torch.uint8), to_gpu(a[2], torch.float32),
                          to_gpu(b[0], torch.uint8), to_gpu(b[1], torch.uint8), to_gpu(b[2], torch.float32),
                          to_gpu(offs, torch.int32), out=out)
    c = to_np(out)
    assert (c[120:] == 7.0).all()
    ref, ab = gemm.grouped_gemm_w4a4(a[0], a[1], a[2], b[0], b[1], b[2], offs)
    assert_gemm_close(c[:120], ref[:120], ab[:120])


def test_dense_small_config():
    require_gpu()
    d = workloads.dense_small()
    a = nvfp4.quantize(d["x"])
    w = nvfp4.quantize(d["w"])
    b = (w[0][None], w[1][None], w[2])
    c = _gpu_w4a4(a, b, [0, 128], torch.float32)
    ref, ab = gemm.dense_gemm_w4a4(a[0], a[1], a[2], w[0], w[1], w[2])
    assert_gemm_close(c, ref, ab)


def test_qwen3_4b_up_sampled():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.qwen3_4b_up()
    x, w = to_gpu(d["x"], torch.bfloat16), to_gpu(d["w"], torch.bfloat16)
    aq, as_, ag, _ = ops.nvfp4_quantize(x)
    bq, bs, bg, _ = ops.nvfp4_quantize(w)
    M = x.shape[0]
    offs = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    c = ops.grouped_gemm_w4a4(aq, as_, ag, bq[None], bs[None], bg, offs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(0).choice(M, 48, replace=False))
    ref, ab = gemm.grouped_gemm_w4a4(to_np(aq), to_np(as_), to_np(ag), to_np(bq)[None], to_np(bs)[None],
                                     to_np(bg), [0, M], rows=rows)
    assert_gemm_close(to_np(c)[rows], ref, ab, bf16_out=True)


@pytest.mark.parametrize("cfg", ["moe_4k", "moe_16k_skew"])
def test_moe_gate_up_sampled(cfg):
    # Full-size grouped GEMM1 launch; the oracle checks, for a seeded subset
    # of experts (always including the largest), the first and last row of
    # every 128-row tile plus random rows.
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer, ops
    d = workloads.CONFIGS[cfg]()
    E, k = d["E"], d["k"]
    x = to_gpu(d["x"], torch.bfloat16)
    r = ops.moe_permute(to_gpu(d["topk_ids"], torch.int32), E, x=x, want_amax=True)
    aq, as_, ag, _ = ops.nvfp4_quantize(r["x_perm"], amax_in=r["amax"])
    wq = moe_layer.quantize_expert_weights(to_gpu(d["w_gu"], torch.bfloat16))
    c = ops.grouped_gemm_w4a4(aq, as_, ag, wq["q"], wq["s"], wq["g"], r["offsets"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    off = to_np(r["offsets"])
    counts = np.diff(off)
    rng = np.random.default_rng(1)
    experts = set(rng.choice(np.nonzero(counts)[0], 6, replace=False).tolist()) | {int(counts.argmax())}
    rows = []
    for e in sorted(experts):
        lo, hi = off[e], off[e + 1]
        for t0 in range(lo, hi, 128):
            rows += [t0, min(t0 + 127, hi - 1)]
        rows += rng.integers(lo, hi, 8).tolist()
    rows = np.unique(np.array(rows))
    wgq, wgs, wgg = to_np(wq["q"]), to_np(wq["s"]), to_np(wq["g"])
    ref, ab = gemm.grouped_gemm_w4a4(to_np(aq), to_np(as_), to_np(ag), wgq, wgs, wgg, off, rows=rows)
    assert_gemm_close(to_np(c)[rows], ref, ab, bf16_out=True, what=cfg)


def _bf(rng, shape, scale=1.0):
    return bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("counts,K,N", [
    ([0, 1, 200, 0, 70], 96, 160),     # empty and 1-row experts, K half a step past one
    ([300, 0, 257, 3], 320, 288),      # several 256-wide tiles with tails in M, N and K
])
def test_bf16_small(layout, out_dtype, counts, K, N):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(11 + K)
    E = len(counts)
    M = sum(counts)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = _bf(rng, (M, K))
    b = _bf(rng, (E, N, K) if layout == "NT" else (E, K, N) if layout == "NN" else (M, N), 0.05)
    lay = {"NT": ops.NT, "NN": ops.NN, "TN": ops.TN}[layout]
    c = ops.grouped_gemm_bf16(lay, to_gpu(a, torch.bfloat16), to_gpu(b, torch.bfloat16),
                              to_gpu(offs, torch.int32), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, ab = gemm.grouped_gemm_bf16(layout, a, b, offs)
    assert_gemm_close(to_np(c), ref, ab, bf16_out=out_dtype == torch.bfloat16, what=layout)
    if layout == "TN":
        for e in np.flatnonzero(np.asarray(counts) == 0):
            assert (to_np(c)[e] == 0).all(), "empty expert %d" % e


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_bf16_more_experts_than_lds_offsets(layout):
    """1100 experts (past the 1024 whose offsets the GEMMs copy to LDS): the
    per-tile lookups read the offsets from global memory."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(23)
    E, K, N = 1100, 64, 96
    counts = rng.integers(0, 12, E)
    M = int(counts.sum())
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = _bf(rng, (M, K))
    b = _bf(rng, (E, N, K) if layout == "NT" else (E, K, N) if layout == "NN" else (M, N), 0.05)
    lay = {"NT": ops.NT, "NN": ops.NN, "TN": ops.TN}[layout]
    c = ops.grouped_gemm_bf16(lay, to_gpu(a, torch.bfloat16), to_gpu(b, torch.bfloat16),
                              to_gpu(offs, torch.int32), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ab = gemm.grouped_gemm_bf16(layout, a, b, offs)
    assert_gemm_close(to_np(c), ref, ab, what=layout)



@pytest.mark.parametrize("E,hi,K,N,accumulate", [
    (600, 100, 64, 96, False),      # ~2-3 tiles per workgroup; 0-100 rows: 0 to 4 steps
    (200, 70, 320, 288, False),     # four tiles per expert with K and N tails
    (400, 140, 96, 160, True),      # accumulating into a non-zero dW
])
def test_bf16_tn_many_tiles_per_workgroup(E, hi, K, N, accumulate):
    """TN with more tiles than workgroups, so that each workgroup loads its
    next tile's first stages while its previous tile's results are still
    being stored: every expert's dW against the oracle, empty experts zero
    (or untouched when accumulating)."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(E + hi + K)
    counts = rng.integers(0, hi + 1, E)
    counts[rng.random(E) < 0.1] = 0
    counts[:3] = [1, 31, 33]        # one-row and one-step-boundary experts
    M = int(counts.sum())
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = _bf(rng, (M, K))
    b = _bf(rng, (M, N), 0.05)
    c0 = (rng.standard_normal((E, K, N)) * 0.1).astype(np.float32) if accumulate else None
    out = to_gpu(c0, torch.float32) if accumulate else None
    c = ops.grouped_gemm_bf16(ops.TN, to_gpu(a, torch.bfloat16), to_gpu(b, torch.bfloat16), to_gpu(offs, torch.int32),
                              out=out, out_dtype=torch.float32, accumulate=accumulate)
    torch.cuda.synchronize()
    ref, ab = gemm.grouped_gemm_bf16("TN", a, b, offs)
    if accumulate:
        assert_gemm_close(to_np(c), ref + c0, ab + np.abs(c0), what="TN accumulate, many tiles")
    else:
        assert_gemm_close(to_np(c), ref, ab, what="TN many tiles")
        for e in np.flatnonzero(counts == 0):
            assert (to_np(c)[e] == 0).all(), "empty expert %d" % e

def test_bf16_tn_accumulate():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(12)
    counts = [33, 0, 130]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M, K, N = sum(counts), 64, 96
    a, b = _bf(rng, (M, K)), _bf(rng, (M, N))
    c0 = rng.standard_normal((3, K, N)).astype(np.float32)
    out = to_gpu(c0, torch.float32)
    ops.grouped_gemm_bf16(ops.TN, to_gpu(a, torch.bfloat16), to_gpu(b, torch.bfloat16), to_gpu(offs, torch.int32),
                          out=out, accumulate=True)
    torch.cuda.synchronize()
    ref, ab = gemm.grouped_gemm_bf16("TN", a, b, offs)
    assert_gemm_close(to_np(out), ref + c0, ab + np.abs(c0), what="TN accumulate")
    np.testing.assert_array_equal(to_np(out)[1], c0[1])


def test_moe_8k_backward_shapes_sampled():
    # Full-size NN and TN launches of the down projection's backward; the
    # oracle checks sampled rows (NN) and two experts' weight gradients (TN).
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.moe_8k_update()
    E, k, F = d["E"], d["k"], d["F"]
    r = ops.moe_permute(to_gpu(d["topk_ids"], torch.int32), E)
    off = to_np(r["offsets"])
    R = int(off[-1])
    rng = np.random.default_rng(2)
    dy2 = _bf(rng, (R, 2048), 1e-3)
    h = _bf(rng, (R, F))
    w_dn = d["w_dn"]
    dy2_g, h_g = to_gpu(dy2, torch.bfloat16), to_gpu(h, torch.bfloat16)
    dh = ops.grouped_gemm_bf16(ops.NN, dy2_g, to_gpu(w_dn, torch.bfloat16), r["offsets"], out_dtype=torch.bfloat16)
    dw = ops.grouped_gemm_bf16(ops.TN, dy2_g, h_g, r["offsets"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(R, 64, replace=False))
    experts = np.searchsorted(off, rows, side="right") - 1
    dh_np = to_np(dh)
    for rr, e in zip(rows, experts):
        ref, ab = gemm.grouped_gemm_bf16("NN", dy2[rr:rr + 1], w_dn[e:e + 1], [0, 1])
        assert_gemm_close(dh_np[rr:rr + 1], ref, ab, bf16_out=True, what="NN row %d" % rr)
    dw_np = to_np(dw)
    for e in (0, 77):
        lo, hi = off[e], off[e + 1]
        ref, ab = gemm.grouped_gemm_bf16("TN", dy2[lo:hi], h[lo:hi], [0, hi - lo])
        assert_gemm_close(dw_np[e], ref[0], ab[0], what="TN expert %d" % e)


@pytest.mark.parametrize("counts,K,N,k", [
    ([0, 1, 200, 0, 70], 96, 160, 3),   # empty and 1-row experts, ragged tails
    ([300, 0, 257, 3], 320, 288, 2),
])
def test_bf16_tn_gather_small(counts, K, N, k):
    # The gathered weight gradient against the oracle's TN on the explicitly
    # gathered rows, and bit for bit against the library's TN on those rows.
    # A few rows carry b_src = -1 (no source row: zeros).
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(31 + K)
    E, M = len(counts), sum(counts)
    T = (M + k - 1) // k + 5
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src = rng.integers(0, T * k, M).astype(np.int32)
    src[rng.choice(M, min(M, 4), replace=False)] = -1
    a = _bf(rng, (M, K))
    x = _bf(rng, (T, N), 0.05)
    xg = np.where((src >= 0)[:, None], x[np.maximum(src, 0) // k], 0.0).astype(np.float32)
    a_g, offs_g = to_gpu(a, torch.bfloat16), to_gpu(offs, torch.int32)
    c = ops.grouped_gemm_bf16_tn_gather(a_g, to_gpu(x, torch.bfloat16), to_gpu(src, torch.int32), k, offs_g)
    c_ref = ops.grouped_gemm_bf16(ops.TN, a_g, to_gpu(xg, torch.bfloat16), offs_g)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32))
    ref, ab = gemm.grouped_gemm_bf16("TN", a, xg, offs)
    assert_gemm_close(to_np(c), ref, ab, what="TN gather")


def test_bf16_tn_gather_moe_8k_gate_up():
    # Full-size weight gradient of the gate+up projection as the backward
    # runs it: dY1 against the unpermuted tokens gathered through src, bit
    # for bit equal to the TN GEMM on the permuted copy of the tokens.
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.moe_8k_update()
    E, k = d["E"], d["k"]
    x = to_gpu(d["x"], torch.bfloat16)
    r = ops.moe_permute(to_gpu(d["topk_ids"], torch.int32), E, x=x)
    R = r["x_perm"].shape[0]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    dy1 = (torch.randn(R, 2 * d["F"], device="cuda", generator=gen) * 1e-3).to(torch.bfloat16)
    dw = ops.grouped_gemm_bf16_tn_gather(dy1, x, r["src"], k, r["offsets"])
    dw_ref = ops.grouped_gemm_bf16(ops.TN, dy1, r["x_perm"], r["offsets"])
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32))



@pytest.mark.parametrize("counts,N,K", [([0, 1, 300, 0, 37, 256, 511], 96, 256), ([700], 512, 320)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w4a4_scaled_mfma_design_matches_oracle(counts, N, K, out_dtype):
    """The scale-factoring design (fp4 scaled MFMA, one block per issue,
    fp32 rescale) computes the same product within the tolerance."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(sum(counts) + N + K)
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 20
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    a = nvfp4.quantize(x)
    b = quantize_weights(w)
    g = [to_gpu(a[0], torch.uint8), to_gpu(a[1], torch.uint8), to_gpu(a[2], torch.float32),
         to_gpu(b[0], torch.uint8), to_gpu(b[1], torch.uint8), to_gpu(b[2], torch.float32), to_gpu(off, torch.int32)]
    c = ops.grouped_gemm_w4a4_scaled_mfma(*g, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, ab = gemm.grouped_gemm_w4a4(a[0], a[1], a[2], b[0], b[1], b[2], off)
    assert_gemm_close(to_np(c), ref, ab, bf16_out=out_dtype == torch.bfloat16, what="scaled-mfma design")
