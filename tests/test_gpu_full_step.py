"""Full-size parity of the step the benchmark times (the MoE layer full
update: 8192 tokens, d_model 2048, 128 experts, top-8, FFN 768), launched
exactly as bench.py launches it (moe_layer.forward / backward on full-size
buffers).  Every stage is checked against the oracle fed with the GPU's own
stored input of that stage, on what the oracle can afford at this size:
the whole routing metadata, and for four experts (the first, the largest,
the last and a seeded one) the first and last row of every 256-row tile plus
seeded rows; the full weight gradients of two experts; seeded tokens of the
two combines.  The reference of each stage is the oracle's own stage
function (oracle.layer.forward_stage / backward_stage), whose wiring the CPU
tests pin.  Integer outputs are compared bit for bit,
GEMMs within |C - C_ref| <= 1e-3 * sum|a*b| (+ bf16 output rounding)."""

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_bf16_close, assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from oracle import gemm, layer, moe, nvfp4
from oracle.layer import bf16_round

pytestmark = gpu


@pytest.fixture(scope="module")
def step():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    d = workloads.moe_8k_update()
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    dev = torch.device("cuda:0")
    x, w_gu, w_dn, dy = (to_gpu(d[n], torch.bfloat16) for n in ("x", "w_gu", "w_dn", "dy"))
    ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
    wq_gu = moe_layer.quantize_expert_weights(w_gu)
    wq_dn = moe_layer.quantize_expert_weights(w_dn)
    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=True)
    meta = moe_layer.forward(x, ids, tw, wq_gu, wq_dn, buf)
    moe_layer.backward(dy, tw, w_gu, w_dn, meta, buf)
    torch.cuda.synchronize()
    off = to_np(meta["offsets"]).astype(np.int64)
    counts = np.diff(off)
    rng = np.random.default_rng(7)
    experts = sorted({0, int(counts.argmax()), E - 1, int(rng.integers(1, E - 1))})
    rows = []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        for t0 in range(lo, hi, 256):
            rows += [t0, min(t0 + 255, hi - 1)]
        rows += rng.integers(lo, hi, 6).tolist()
    rows = np.unique(np.array(rows, dtype=np.int64))
    return dict(d=d, meta=meta, buf=buf, wq_gu=wq_gu, wq_dn=wq_dn, off=off, rows=rows, experts=experts, rng=rng)


def _rows(t, rows):
    return to_np(t[torch.from_numpy(rows).to(t.device)])


def test_metadata_and_fused_permute_quantize(step):
    d, meta, buf, rows = step["d"], step["meta"], step["buf"], step["rows"]
    off, dest, src = moe.permute_metadata(d["topk_ids"], d["E"])
    np.testing.assert_array_equal(to_np(meta["offsets"]), off)
    np.testing.assert_array_equal(to_np(meta["dest"]), dest)
    np.testing.assert_array_equal(to_np(meta["src"]), src)
    amax = to_np(buf.amax)
    assert amax[0] == np.abs(d["x"]).max()
    xr = d["x"][src[rows] // d["k"]]
    np.testing.assert_array_equal(_rows(buf.x_perm, rows), xr)
    q, s, g, _ = nvfp4.quantize(xr, amax=[amax[0]])
    np.testing.assert_array_equal(_rows(buf.a1_q, rows), q)
    np.testing.assert_array_equal(_rows(buf.a1_s, rows), s)
    assert to_np(buf.a1_g)[0] == g[0]


def _stage_args(step):
    d, meta = step["d"], step["meta"]
    return step["off"], to_np(meta["dest"]), to_np(meta["src"])


def test_gate_up_silu_requantize_down_combine(step):
    """Forward stages on sampled rows, each from the oracle's stage function
    (oracle.layer's wiring) fed the GPU's stored rows."""
    d, meta, buf, rows = step["d"], step["meta"], step["buf"], step["rows"]
    off, dest, src = _stage_args(step)
    wq_gu, wq_dn = step["wq_gu"], step["wq_dn"]
    wg = (to_np(wq_gu["q"]), to_np(wq_gu["s"]), to_np(wq_gu["g"]))
    wd = (to_np(wq_dn["q"]), to_np(wq_dn["s"]), to_np(wq_dn["g"]))
    amax = to_np(buf.amax)
    g = dict(a1=(_rows(buf.a1_q, rows), _rows(buf.a1_s, rows), to_np(buf.a1_g)), y1=_rows(buf.y1, rows),
             h=_rows(buf.h, rows), a2=(_rows(buf.a2_q, rows), _rows(buf.a2_s, rows), to_np(buf.a2_g)),
             amax_x=amax[0], amax_h=amax[1])
    fs = lambda n, s=g, r=rows, dst=dest, tw=d["topk_w"]: layer.forward_stage(  # noqa: E731
        n, s, d["x"], tw, wg, wd, off, dst, src, rows=r)
    ref, ab = fs("y1")
    assert_gemm_close(g["y1"], ref, ab, bf16_out=True, what="gate+up (fused epilogue)")
    assert_bf16_close(g["h"], fs("h")[0], what="fused SiLU gate")
    assert amax[1] == np.abs(to_np(buf.h)).max()
    q2, s2, g2 = layer.forward_stage("a2", g, None, d["topk_w"], wg, wd, off, dest, src)[0]
    np.testing.assert_array_equal(g["a2"][0], q2)
    np.testing.assert_array_equal(g["a2"][1], s2)
    assert to_np(buf.a2_g)[0] == g2[0]
    ref, ab = fs("y2")
    assert_gemm_close(_rows(buf.y2, rows), ref, ab, bf16_out=True, what="down")
    # combine: seeded tokens, from the GPU's own Y2 rows
    k = d["k"]
    toks = np.sort(step["rng"].choice(d["T"], 32, replace=False))
    sub = dest.reshape(-1, k)[toks].reshape(-1)
    local = np.arange(sub.size, dtype=np.int64)
    ref, bound = fs("out", s=dict(y2=_rows(buf.y2, sub)), r=None, dst=local, tw=d["topk_w"][toks])
    assert_bf16_close(_rows(buf.out, toks), ref, scale=bound, what="combine")


def test_backward(step):
    """Backward stages on sampled rows, two experts' full weight gradients
    and seeded tokens of the dX combine, each from the oracle's stage
    function fed the GPU's stored inputs."""
    d, meta, buf, rows = step["d"], step["meta"], step["buf"], step["rows"]
    off, dest, src = _stage_args(step)
    k = d["k"]
    g = dict(dy2=_rows(buf.dy2, rows), dh=_rows(buf.dh, rows), y1=_rows(buf.y1, rows), dy1=_rows(buf.dy1, rows))
    bs = lambda n, s=g, r=rows, o=off, dst=dest, tw=d["topk_w"]: layer.backward_stage(  # noqa: E731
        n, s, d["dy"], tw, d["w_gu"], d["w_dn"], o, dst, src, rows=r)
    assert_bf16_close(g["dy2"], bs("dy2")[0], what="dY2")
    ref, ab = bs("dh")
    assert_gemm_close(g["dh"], ref, ab, bf16_out=True, what="dH")
    dy1_ref, _ = bs("dy1")
    scale = np.abs(dy1_ref) + 1e-3 * np.abs(np.concatenate([g["dh"], g["dh"]], axis=1)) * (np.abs(g["y1"]) + 1)
    assert_bf16_close(g["dy1"], dy1_ref, scale=scale, what="dY1")
    ref, ab = bs("dx_perm")
    assert_gemm_close(_rows(buf.dx_perm, rows), ref, ab, bf16_out=True, what="dX_perm")
    # weight gradients of two experts in full, over all their rows
    for e in (step["experts"][0], step["experts"][-1]):
        lo, hi = int(off[e]), int(off[e + 1])
        er = np.arange(lo, hi, dtype=np.int64)
        se = dict(dy2=_rows(buf.dy2, er), h=_rows(buf.h, er), dy1=_rows(buf.dy1, er), x_perm=_rows(buf.x_perm, er))
        one = np.array([0, hi - lo], dtype=np.int64)
        for name, dw in (("dw_dn", buf.dw_dn), ("dw_gu", buf.dw_gu)):
            ref, ab = layer.backward_stage(name, se, d["dy"], d["topk_w"], d["w_gu"][e:e + 1],
                                           d["w_dn"][e:e + 1], one, dest, src)
            assert_gemm_close(to_np(dw[e]), ref[0], ab[0], what="%s expert %d" % (name, e))
    # dX combine: seeded tokens, from the GPU's own dX_perm rows
    toks = np.sort(step["rng"].choice(d["T"], 32, replace=False))
    sub = dest.reshape(-1, k)[toks].reshape(-1)
    local = np.arange(sub.size, dtype=np.int64)
    ref, bound = bs("dx", s=dict(dx_perm=_rows(buf.dx_perm, sub)), r=None, dst=local, tw=d["topk_w"][toks])
    assert_bf16_close(_rows(buf.dx, toks), ref, scale=bound, what="dX")


@pytest.mark.parametrize("cfg", ["moe_4k", "moe_16k_skew"])
def test_forward_only_workloads(cfg):
    """The forward-only workloads as bench.py --workload runs them (no bf16
    X_perm, no stored Y1): routing metadata in full, sampled rows of every
    stage for the largest expert and three seeded non-empty ones, seeded
    tokens of the combine."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer
    d = workloads.CONFIGS[cfg]()
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    dev = torch.device("cuda:0")
    x = to_gpu(d["x"], torch.bfloat16)
    ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
    wq_gu = moe_layer.quantize_expert_weights(to_gpu(d["w_gu"], torch.bfloat16))
    wq_dn = moe_layer.quantize_expert_weights(to_gpu(d["w_dn"], torch.bfloat16))
    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=False)
    meta = moe_layer.forward(x, ids, tw, wq_gu, wq_dn, buf, keep_y1=False, keep_x_perm=False)
    torch.cuda.synchronize()
    off, dest, src = moe.permute_metadata(d["topk_ids"], E)
    np.testing.assert_array_equal(to_np(meta["offsets"]), off)
    np.testing.assert_array_equal(to_np(meta["dest"]), dest)
    counts = np.diff(off)
    rng = np.random.default_rng(3)
    nz = np.nonzero(counts)[0]
    experts = sorted({int(counts.argmax())} | set(rng.choice(nz, 3, replace=False).tolist()))
    rows = []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        for t0 in range(lo, hi, 256):
            rows += [t0, min(t0 + 255, hi - 1)]
        rows += rng.integers(lo, hi, 6).tolist()
    rows = np.unique(np.array(rows, dtype=np.int64))
    amax = to_np(buf.amax)
    assert amax[0] == np.abs(d["x"]).max()
    q, s, g, _ = nvfp4.quantize(d["x"][src[rows] // k], amax=[amax[0]])
    np.testing.assert_array_equal(_rows(buf.a1_q, rows), q)
    np.testing.assert_array_equal(_rows(buf.a1_s, rows), s)
    wg = (to_np(wq_gu["q"]), to_np(wq_gu["s"]), to_np(wq_gu["g"]))
    wd = (to_np(wq_dn["q"]), to_np(wq_dn["s"]), to_np(wq_dn["g"]))
    a1 = (to_np(buf.a1_q), to_np(buf.a1_s), to_np(buf.a1_g))
    y1_ref, ab1 = gemm.grouped_gemm_w4a4(*a1, *wg, off, rows=rows)
    # Y1 is not stored on this path: H is checked against the oracle's SiLU
    # gate of the oracle's Y1 rounded to bf16, within the GEMM tolerance
    # carried through the gate.
    h = _rows(buf.h, rows)
    y1_bf = bf16_round(y1_ref.astype(np.float32))
    h_ref = moe.silu_gate_fwd(y1_bf)
    Fh = h_ref.shape[1]
    g_ab, u_ab = ab1[:, :Fh], ab1[:, Fh:]
    gv, uv = y1_bf[:, :Fh].astype(np.float64), y1_bf[:, Fh:].astype(np.float64)
    # |d silu(g) u| <= (1.1 |u| dg + |silu(g)| du) with dg, du the Y1 errors
    dg = 1e-3 * g_ab + 2.0 ** -8 * (np.abs(gv) + 1e-3 * g_ab)
    du = 1e-3 * u_ab + 2.0 ** -8 * (np.abs(uv) + 1e-3 * u_ab)
    tol = 1.1 * np.abs(uv) * dg + np.abs(moe.silu(gv)) * du + 2.0 ** -8 * np.abs(h_ref) + 1e-30
    err = np.abs(h.astype(np.float64) - h_ref)
    assert (err <= tol).all(), "H: %d of %d out of tolerance" % (int((err > tol).sum()), err.size)
    amax_h = to_np(buf.amax)[1]
    assert amax_h == np.abs(to_np(buf.h)).max()
    q2, s2, _, _ = nvfp4.quantize(h, amax=[amax_h])
    np.testing.assert_array_equal(_rows(buf.a2_q, rows), q2)
    np.testing.assert_array_equal(_rows(buf.a2_s, rows), s2)
    a2 = (to_np(buf.a2_q), to_np(buf.a2_s), to_np(buf.a2_g))
    y2_ref, ab2 = gemm.grouped_gemm_w4a4(*a2, *wd, off, rows=rows)
    assert_gemm_close(_rows(buf.y2, rows), y2_ref, ab2, bf16_out=True, what="%s down" % cfg)
    toks = np.sort(rng.choice(T, 32, replace=False))
    sub = dest.reshape(-1, k)[toks].reshape(-1)
    y2s = _rows(buf.y2, sub.astype(np.int64))
    local = np.arange(sub.size, dtype=np.int64)
    ref = moe.unpermute(y2s, local, k, d["topk_w"][toks])
    bound = moe.unpermute_absbound(y2s, local, k, d["topk_w"][toks])
    assert_bf16_close(_rows(buf.out, toks), ref, scale=bound, what="%s combine" % cfg)
