"""GPU parity of the NVFP4 backward variant: column-wise and transposed
quantization bit for bit against the oracle (including the zero padding of
each expert's segment), the W4A4 weight-gradient GEMM within
|C - C_ref| <= 1e-3 * sum|a*b| (empty experts, ragged segments, tails), and
the whole variant stage by stage against oracle.layer.backward_nvfp4_stage
fed the GPU's stored inputs -- at small shapes in full, at the 8k-update
shapes on sampled rows and two experts' full weight gradients."""

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_bf16_close, assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from oracle import gemm, layer, moe, nvfp4

pytestmark = gpu


def _check_colwise(q_t, s_t, g, x, off, amax, Kp):
    """GPU column-wise layout against the oracle, segment by segment."""
    cols, g_ref = nvfp4.quantize_colwise(x, off, amax)
    q_t, s_t = to_np(q_t), to_np(s_t)
    assert q_t.shape[1] == Kp // 2 and s_t.shape[1] == Kp // 16
    poff = nvfp4.segment_pad_offset(off)
    for e, (q, s) in enumerate(cols):
        L = q.shape[1] * 2
        p0 = int(poff[e])
        np.testing.assert_array_equal(q_t[:, p0 // 2:(p0 + L) // 2], q, err_msg="codes, expert %d" % e)
        np.testing.assert_array_equal(s_t[:, p0 // 16:(p0 + L) // 16], s, err_msg="scales, expert %d" % e)
        pad = -(-(off[e + 1] - off[e]) // 64) * 64
        assert (q_t[:, (p0 + L) // 2:(p0 + pad) // 2] == 0).all() and (s_t[:, (p0 + L) // 16:(p0 + pad) // 16] == 0).all()
    assert to_np(g)[0] == g_ref[0]


@pytest.mark.parametrize("counts,N", [([0, 1, 17, 64, 65, 0, 200, 3], 40), ([513], 264), ([5] * 30, 8)])
def test_colwise_quantize_matches_oracle(counts, N):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(sum(counts) + N)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1]) + 3                  # rows past offsets[E] belong to no expert
    x = (rng.standard_normal((M, N)) * np.exp2(rng.integers(-3, 3, (M, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 30
    x = workloads._bf16(x)               # the values the GPU sees
    amax = np.float32(np.abs(x).max())
    q_t, s_t, g = ops.nvfp4_quantize_colwise(to_gpu(x, torch.bfloat16), to_gpu(off, torch.int32),
                                             to_gpu(np.array([amax]), torch.float32))
    torch.cuda.synchronize()
    _check_colwise(q_t, s_t, g, x, off, amax, ops.padded_extent(M, len(counts)))
    # a stale amax (saturating) takes the same path
    q_t, s_t, g = ops.nvfp4_quantize_colwise(to_gpu(x, torch.bfloat16), to_gpu(off, torch.int32),
                                             to_gpu(np.array([amax / 4]), torch.float32))
    torch.cuda.synchronize()
    _check_colwise(q_t, s_t, g, x, off, amax / 4, ops.padded_extent(M, len(counts)))



def test_colwise_tiles_straddle_experts_and_gaps_stay_unwritten():
    """Expert segments of 10, 70, 1, 0, 130, 64 and 5 rows: padded segments at
    columns 0, 64, 192, (256: empty), 320, 512 and 640, so one 256-column
    work tile spans four experts, and columns 256..319 and 576..639 belong to
    no segment.  Those gap columns keep the sentinel the outputs held."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    counts = [10, 70, 1, 0, 130, 64, 5]
    rng = np.random.default_rng(21)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M, N = int(off[-1]), 136
    x = workloads._bf16((rng.standard_normal((M, N)) * np.exp2(rng.integers(-2, 3, (M, 1)))).astype(np.float32))
    amax = np.float32(np.abs(x).max())
    Kp = ops.padded_extent(M, len(counts))
    q_t = torch.full((N, Kp // 2), 0xAB, dtype=torch.uint8, device="cuda")
    s_t = torch.full((N, Kp // 16), 0xCD, dtype=torch.uint8, device="cuda")
    q_t, s_t, g = ops.nvfp4_quantize_colwise(to_gpu(x, torch.bfloat16), to_gpu(off, torch.int32),
                                             to_gpu(np.array([amax]), torch.float32), Kp=Kp, q_t=q_t, s_t=s_t)
    torch.cuda.synchronize()
    _check_colwise(q_t, s_t, g, x, off, amax, Kp)
    poff = nvfp4.segment_pad_offset(off)
    assert list(poff) == [0, 64, 192, 256, 320, 512, 640]
    qn, sn = to_np(q_t), to_np(s_t)
    covered = np.zeros(Kp, bool)
    for e in range(len(counts)):
        covered[poff[e]:poff[e] + -(-counts[e] // 64) * 64] = True
    gap = ~covered
    assert gap[256:320].all() and gap[576:640].all()
    assert (qn[:, gap[0::2]] == 0xAB).all() and (sn[:, gap[0::16]] == 0xCD).all()

def test_transposed_weights_match_oracle():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    rng = np.random.default_rng(3)
    E, N, K = 5, 192, 128
    w = workloads._bf16((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    wt = moe_layer.quantize_expert_weights_t(to_gpu(w, torch.bfloat16))
    wq = moe_layer.quantize_expert_weights(to_gpu(w, torch.bfloat16))
    wt2 = moe_layer.quantize_expert_weights_t(to_gpu(w, torch.bfloat16), amax=wq["amax"])
    torch.cuda.synchronize()
    ref = layer.quantize_weights_t(w)
    for got in (wt, wt2):
        np.testing.assert_array_equal(to_np(got["q"]), ref[0])
        np.testing.assert_array_equal(to_np(got["s"]), ref[1])
        np.testing.assert_array_equal(to_np(got["g"]), ref[2])


@pytest.mark.parametrize("counts,N1,N2", [([0, 1, 300, 45, 0, 512, 77], 96, 160), ([1000], 256, 512),
                                          ([0, 0, 3], 32, 32)])
def test_wgrad_gemm_matches_oracle(counts, N1, N2):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(N1 + N2 + sum(counts))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    a = workloads._bf16(rng.standard_normal((M, N1)).astype(np.float32) * 1e-3)
    b = workloads._bf16(rng.standard_normal((M, N2)).astype(np.float32))
    am_a, am_b = np.float32(np.abs(a).max() if M else 0), np.float32(np.abs(b).max() if M else 0)
    og = to_gpu(off, torch.int32)
    ca = ops.nvfp4_quantize_colwise(to_gpu(a, torch.bfloat16), og, to_gpu(np.array([am_a]), torch.float32))
    cb = ops.nvfp4_quantize_colwise(to_gpu(b, torch.bfloat16), og, to_gpu(np.array([am_b]), torch.float32))
    E = len(counts)
    c = torch.full((E, N1, N2), 7.0, dtype=torch.float32, device="cuda")
    ops.grouped_gemm_w4a4_wgrad(ca, cb, og, M, out=c)
    torch.cuda.synchronize()
    ra, ga = nvfp4.quantize_colwise(a, off, am_a)
    rb, gb = nvfp4.quantize_colwise(b, off, am_b)
    ref, ab = gemm.grouped_gemm_w4a4_wgrad(ra, ga, rb, gb)
    assert_gemm_close(to_np(c), ref, ab, what="wgrad")


def _nv_run(d, T, k, E, D, F):
    from nvfp4_quantized_moe_token_amd import moe_layer
    dev = torch.device("cuda:0")
    x, w_gu, w_dn, dy = (to_gpu(d[n], torch.bfloat16) for n in ("x", "w_gu", "w_dn", "dy"))
    ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
    wq_gu, wq_dn = moe_layer.quantize_expert_weights(w_gu), moe_layer.quantize_expert_weights(w_dn)
    wt_gu = moe_layer.quantize_expert_weights_t(w_gu, amax=wq_gu["amax"])
    wt_dn = moe_layer.quantize_expert_weights_t(w_dn, amax=wq_dn["amax"])
    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=True)
    nb = moe_layer.NVFP4BackwardBuffers(T, k, E, D, F, dev)
    meta = moe_layer.forward(x, ids, tw, wq_gu, wq_dn, buf)
    moe_layer.backward_nvfp4(dy, tw, wt_gu, wt_dn, meta, buf, nb)
    torch.cuda.synchronize()
    return meta, buf, nb, wt_gu, wt_dn


def test_nvfp4_backward_stagewise_small():
    require_gpu()
    T, k, E, D, F = 256, 8, 16, 256, 128
    d = workloads.moe(T, 1.1, 0.01, 32.0, with_dy=True, E=E, k=k, D=D, F=F, name="nvbwd")
    meta, buf, nb, wt_gu, wt_dn = _nv_run(d, T, k, E, D, F)
    off, dest, src = (to_np(meta[n]) for n in ("offsets", "dest", "src"))
    ref_wt_gu, ref_wt_dn = layer.quantize_weights_t(d["w_gu"]), layer.quantize_weights_t(d["w_dn"])
    for got, ref in ((wt_gu, ref_wt_gu), (wt_dn, ref_wt_dn)):
        np.testing.assert_array_equal(to_np(got["q"]), ref[0])
        np.testing.assert_array_equal(to_np(got["g"]), ref[2])
    amax = to_np(buf.amax)
    g = dict(x_perm=to_np(buf.x_perm), y1=to_np(buf.y1), h=to_np(buf.h), amax_x=amax[0], amax_h=amax[1],
             dy2=to_np(buf.dy2), dh=to_np(buf.dh), dy1=to_np(buf.dy1), dx_perm=to_np(buf.dx_perm),
             amax_dy2=to_np(nb.amax)[0], amax_dy1=to_np(nb.amax)[1],
             a_dy2=tuple(to_np(t) for t in nb.a_dy2), a_dy1=tuple(to_np(t) for t in nb.a_dy1))
    assert g["amax_dy2"] == np.abs(g["dy2"]).max() and g["amax_dy1"] == np.abs(g["dy1"]).max()
    st = lambda n: layer.backward_nvfp4_stage(n, g, d["dy"], d["topk_w"], ref_wt_gu, ref_wt_dn, off, dest, src)  # noqa: E731
    assert_bf16_close(g["dy2"], st("dy2")[0], what="dY2")
    for name in ("a_dy2", "a_dy1"):
        for got, want in zip(g[name], st(name)[0]):
            np.testing.assert_array_equal(got, want, err_msg=name)
    for name in ("dh", "dx_perm"):
        ref, ab = st(name)
        assert_gemm_close(g[name], ref, ab, bf16_out=True, what=name)
    for name, t in (("dw_dn", buf.dw_dn), ("dw_gu", buf.dw_gu)):
        ref, ab = st(name)
        assert_gemm_close(to_np(t), ref, ab, what=name)
    dy1_ref, _ = st("dy1")
    scale = np.abs(dy1_ref) + 1e-3 * np.abs(np.concatenate([g["dh"], g["dh"]], axis=1)) * (np.abs(g["y1"]) + 1)
    assert_bf16_close(g["dy1"], dy1_ref, scale=scale, what="dY1")
    ref, bound = st("dx")
    assert_bf16_close(to_np(buf.dx), ref, scale=bound, what="dX")
    # the column-wise operands the wgrad GEMMs read, bit for bit
    Kp = nb.Kp
    _check_colwise(nb.c_dy2[0], nb.c_dy2[1], nb.c_dy2[2], g["dy2"], off, g["amax_dy2"], Kp)
    _check_colwise(nb.c_h[0], nb.c_h[1], nb.c_h[2], g["h"], off, g["amax_h"], Kp)
    _check_colwise(nb.c_dy1[0], nb.c_dy1[1], nb.c_dy1[2], g["dy1"], off, g["amax_dy1"], Kp)
    _check_colwise(nb.c_x[0], nb.c_x[1], nb.c_x[2], g["x_perm"], off, g["amax_x"], Kp)


def test_nvfp4_backward_full_size_sampled():
    """The 8k-update shapes (65536 routed rows, 128 experts, D 2048, F 768):
    sampled rows of dH and dX_perm, two experts' full weight gradients and
    column-wise operands, seeded tokens of dX."""
    require_gpu()
    d = workloads.moe_8k_update()
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    meta, buf, nb, wt_gu, wt_dn = _nv_run(d, T, k, E, D, F)
    off, dest, src = (to_np(meta[n]).astype(np.int64) for n in ("offsets", "dest", "src"))
    rng = np.random.default_rng(12)
    counts = np.diff(off)
    experts = sorted({0, int(counts.argmax()), E - 1})
    rows = np.unique(np.concatenate([[off[e], off[e + 1] - 1] + rng.integers(off[e], off[e + 1], 5).tolist()
                                     for e in experts]).astype(np.int64))
    sel = torch.from_numpy(rows).cuda()
    wtg = (to_np(wt_gu["q"]), to_np(wt_gu["s"]), to_np(wt_gu["g"]))
    wtd = (to_np(wt_dn["q"]), to_np(wt_dn["s"]), to_np(wt_dn["g"]))
    g = dict(a_dy2=tuple(to_np(t[sel]) if t.dim() == 2 else to_np(t) for t in nb.a_dy2),
             a_dy1=tuple(to_np(t[sel]) if t.dim() == 2 else to_np(t) for t in nb.a_dy1))
    st = lambda n: layer.backward_nvfp4_stage(n, g, d["dy"], d["topk_w"], wtg, wtd, off, dest, src, rows=rows)  # noqa: E731
    for name, t in (("dh", buf.dh), ("dx_perm", buf.dx_perm)):
        ref, ab = st(name)
        assert_gemm_close(to_np(t[sel]), ref, ab, bf16_out=True, what=name)
    q, s, gg, _ = nvfp4.quantize(to_np(buf.dy2[sel]), amax=[to_np(nb.amax)[0]])
    np.testing.assert_array_equal(g["a_dy2"][0], q)
    np.testing.assert_array_equal(g["a_dy2"][1], s)
    amax = to_np(buf.amax)
    for e in (experts[0], experts[-1]):
        lo, hi = int(off[e]), int(off[e + 1])
        er = torch.arange(lo, hi, device="cuda")
        se = dict(dy2=to_np(buf.dy2[er]), h=to_np(buf.h[er]), dy1=to_np(buf.dy1[er]), x_perm=to_np(buf.x_perm[er]),
                  amax_dy2=to_np(nb.amax)[0], amax_dy1=to_np(nb.amax)[1], amax_h=amax[1], amax_x=amax[0])
        one = np.array([0, hi - lo], dtype=np.int64)
        for name, dw in (("dw_dn", buf.dw_dn), ("dw_gu", buf.dw_gu)):
            ref, ab = layer.backward_nvfp4_stage(name, se, d["dy"], d["topk_w"], None, None, one, dest, src)
            assert_gemm_close(to_np(dw[e]), ref[0], ab[0], what="%s expert %d" % (name, e))
    toks = np.sort(rng.choice(T, 32, replace=False))
    sub = dest.reshape(-1, k)[toks].reshape(-1)
    dxs = to_np(buf.dx_perm[torch.from_numpy(sub).cuda()])
    local = np.arange(sub.size)
    ref = moe.unpermute(dxs, local, k, None)
    assert_bf16_close(to_np(buf.dx[torch.from_numpy(toks).cuda()]), ref,
                      scale=moe.unpermute_absbound(dxs, local, k, None), what="dX")
