"""GPU parity of the W4A8 variant (MXFP8 activations x MXFP4 weights):
mx_quantize bit for bit against the oracle (hand-worked blocks, every
rounding threshold, every finite bf16 value in several block contexts,
random fp32 over a wide range), the grouped W4A8 GEMM within
|C - C_ref| <= 1e-3 * sum|a*b| against the fp64 oracle (empty and one-row
experts, row and column tails, fp32 and bf16 outputs, the full 8k-update
gate+up shape on sampled rows), and the SiLU-gate epilogue bit for bit
against the GEMM followed by silu_gate_fwd; the MXFP8 quantization fused
into the permutation bit for bit against quantize-then-gather."""

import os

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_gemm_close, gpu, require_gpu, to_gpu, to_np
from conftest import GOLDEN
from oracle import gemm, moe, mx
from oracle.layer import bf16_round

pytestmark = gpu

ELEM = {"e4m3": 0, "e2m1": 1}


def _gpu_mx(x_np, dtype, elem):
    from nvfp4_quantized_moe_token_amd import ops
    q, s = ops.mx_quantize(to_gpu(x_np, dtype), ELEM[elem])
    torch.cuda.synchronize()
    return to_np(q), to_np(s)


def _assert_same(x_np, dtype, elem):
    q, s = _gpu_mx(x_np, dtype, elem)
    xv = np.asarray(x_np, np.float32) if dtype == torch.float32 else bf16_round(x_np)
    rq, rs = mx.quantize(xv, elem)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


def _golden():
    blocks, cur = [], None
    for line in open(os.path.join(GOLDEN, "mx_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *rest = line.split()
        if k == "block":
            cur = dict(name=rest[0], elem=rest[1])
            blocks.append(cur)
        elif k == "in":
            cur["in"] = [float(m) * 2.0 ** int(e) if "p" in v else float(v)
                         for v in rest for m, e in [v.split("p") if "p" in v else (v, 0)]]
        elif k == "scale":
            cur["scale"] = int(rest[0], 16)
        elif k == "codes":
            cur["codes"] = [int(v, 16) for v in rest]
    return blocks


def test_golden_blocks_gpu():
    require_gpu()
    for b in _golden():
        x = np.zeros((1, 32), np.float32)
        x[0, :len(b["in"])] = b["in"]
        q, s = _gpu_mx(x, torch.float32, b["elem"])
        assert s[0, 0] == b["scale"], b["name"]
        if b["elem"] == "e2m1":
            codes = np.empty(32, np.uint8)
            codes[0::2], codes[1::2] = q[0] & 15, q[0] >> 4
        else:
            codes = q[0]
        want = np.zeros(32, np.uint8)
        want[:len(b["codes"])] = b["codes"]
        np.testing.assert_array_equal(codes, want, err_msg=b["name"])


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_threshold_sweep_unit_scale(elem):
    # A block holding the format's top value has scale 1 (floor(log2 amax)
    # = emax), so every other element is encoded as itself: sweep every
    # rounding threshold of the format +-3 ulps, both signs.
    require_gpu()
    top = 448.0 if elem == "e4m3" else 6.0
    if elem == "e4m3":
        vals = sorted({m * 2.0 ** -9 for m in range(8)} |
                      {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)} - {480.0})
    else:
        vals = [0, .5, 1, 1.5, 2, 3, 4, 6]
    pts = set(vals) | {(a + b) / 2 for a, b in zip(vals, vals[1:])}
    out = []
    for p in sorted(pts):
        p = np.float32(p)
        lo = hi = p
        out.append(p)
        for _ in range(3):
            lo = np.nextafter(lo, np.float32(-1))
            hi = np.nextafter(hi, np.float32(1e9))
            out += [lo, hi]
    v = np.array([x for x in out if 0 <= x <= top], np.float32)
    v = np.concatenate([v, -v])
    n = (v.size + 30) // 31
    v = np.concatenate([v, np.zeros(n * 31 - v.size, np.float32)]).reshape(n, 31)
    x = np.concatenate([np.full((n, 1), top, np.float32), v], axis=1)
    _assert_same(x, torch.float32, elem)


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_all_bf16_values_in_several_blocks(elem):
    # Every finite bf16 value, laid out in blocks in three orders (sorted:
    # block amax near each value; shuffled: amax far above most values; and
    # each value alone in a block of zeros), bf16 input.
    require_gpu()
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    n = f.size - f.size % 32
    rng = np.random.default_rng(4)
    srt = np.sort(f)[:n].reshape(-1, 32)
    shf = rng.permutation(f)[:n].reshape(-1, 32)
    alone = np.zeros((f.size, 32), np.float32)
    alone[np.arange(f.size), rng.integers(0, 32, f.size)] = f
    for x in (srt, shf, alone):
        _assert_same(x, torch.bfloat16, elem)


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_random_fp32_wide_range(elem):
    require_gpu()
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((512, 256)) * np.exp2(rng.integers(-140, 120, (512, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.02] = -0.0
    x[7] = 0.0
    x[9, 3] = np.float32(3.0e38)
    _assert_same(x, torch.float32, elem)
    _assert_same(x[:, :96], torch.float32, elem)   # a K that is not a multiple of 64


def _mx_operands(rng, M, N, K, E, a_scale=1.0):
    a = rng.standard_normal((M, K)).astype(np.float32) * a_scale
    a[rng.random(a.shape) < 0.01] *= 25
    w = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    aq, as_ = mx.quantize(a, "e4m3")
    bq, bs = mx.quantize(w, "e2m1")
    return aq, as_, bq.reshape(E, N, K // 2), bs.reshape(E, N, K // 32)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("counts,N,K", [
    ([0, 1, 300, 0, 37, 256, 511], 96, 256),     # empty, one-row, tails; N not a tile multiple
    ([700], 512, 384),                           # dense special case (one expert), K % 256 != 0
    ([3] * 40 + [257, 0], 2048, 128),            # many tiny experts, one-stage K
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w4a8_gemm_parity(counts, N, K, out_dtype):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(sum(counts) + N + K)
    E = len(counts)
    off = _offsets(counts)
    M = int(off[-1]) + 5                   # rows past offsets[E] are not written
    aq, as_, bq, bs = _mx_operands(rng, M, N, K, E)
    c = torch.full((M, N), 7.0, dtype=out_dtype, device="cuda")
    ops.grouped_gemm_w4a8(*(to_gpu(t, torch.uint8) for t in (aq, as_, bq, bs)), to_gpu(off, torch.int32), out=c)
    torch.cuda.synchronize()
    ref, ab = gemm.grouped_gemm_w4a8(aq, as_, bq, bs, off)
    got = to_np(c)
    assert_gemm_close(got[:off[-1]], ref[:off[-1]], ab[:off[-1]], bf16_out=out_dtype == torch.bfloat16,
                      what="w4a8")
    assert (got[off[-1]:] == 7.0).all()


def test_w4a8_silu_epilogue_equals_gemm_then_silu():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(77)
    counts = [0, 5, 260, 1, 513, 64]
    E, F, K = len(counts), 256, 384
    off = _offsets(counts)
    M = int(off[-1])
    aq, as_, bq, bs = _mx_operands(rng, M, 2 * F, K, E, a_scale=2.0)
    g = [to_gpu(t, torch.uint8) for t in (aq, as_, bq, bs)]
    offs = to_gpu(off, torch.int32)
    y1 = ops.grouped_gemm_w4a8(*g, offs, out_dtype=torch.bfloat16)
    h_ref, amax_ref = ops.silu_gate_fwd(y1)
    y1f, h, amax = ops.grouped_gemm_w4a8_silu_gate(*g, offs)
    torch.cuda.synchronize()
    assert torch.equal(y1f.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    assert to_np(amax)[0] == to_np(amax_ref)[0] == np.abs(to_np(h)).max()
    ref, ab = gemm.grouped_gemm_w4a8(aq, as_, bq, bs, off)
    assert_gemm_close(to_np(y1), ref, ab, bf16_out=True, what="w4a8 gate+up")
    hv = to_np(h)
    assert (np.abs(hv - moe.silu_gate_fwd(to_np(y1))) <= 2.0 ** -7 * np.abs(hv) + 1e-6).all()



@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [512, 320])
def test_permute_mx_equals_quantize_then_gather(dtype, D):
    """moe_permute_mx (MXFP8 quantization fused into the permutation, each
    token row read once) against the oracle's quantization of the gathered
    rows and, where the scale rows are whole 16-byte units (D = 512), bit for
    bit against mx_quantize followed by the row gathers of codes and scales;
    out-of-range ids are skipped, the rows they leave past offsets[E] are
    zeros, and the metadata equals moe_permute's."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(71 + D)
    T, k, E = 500, 8, 24
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[7, 2] = E + 3
    ids[300, 0] = -1
    x_np = (rng.standard_normal((T, D)) * np.exp(rng.uniform(-6, 6, (T, 1)))).astype(np.float32)
    x_np[11, 40:72] = 0.0                      # an all-zero block: scale 2^-127
    x = to_gpu(x_np, dtype)
    ids_g = to_gpu(ids, torch.int32)
    got = ops.moe_permute_mx(ids_g, E, x)
    xq, xs = ops.mx_quantize(x, ELEM["e4m3"])
    pm = ops.moe_permute(ids_g, E, x=xq)
    torch.cuda.synchronize()
    for name in ("offsets", "dest", "src"):
        assert torch.equal(got[name], pm[name]), name
    assert torch.equal(got["q"], pm["x_perm"])
    if (D // 32) % 16 == 0:
        assert torch.equal(got["scales"], ops.moe_gather(xs, pm["src"], k))
    off = to_np(got["offsets"])
    R_valid = int(off[-1])
    assert R_valid == T * k - 2
    assert (to_np(got["q"])[R_valid:] == 0).all() and (to_np(got["scales"])[R_valid:] == 0).all()
    src = to_np(got["src"])[:R_valid]
    xv = x_np if dtype == torch.float32 else bf16_round(x_np)
    rq, rs = mx.quantize(xv[src // k], "e4m3")
    np.testing.assert_array_equal(to_np(got["q"])[:R_valid], rq)
    np.testing.assert_array_equal(to_np(got["scales"])[:R_valid], rs)


def test_permute_mx_zero_tokens_and_zero_width():
    """No tokens: the offsets are all zero.  D = 0: only the routing
    metadata, equal to moe_permute's (every token on one expert, the others
    empty)."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    r = ops.moe_permute_mx(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 16,
                           torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert (to_np(r["offsets"]) == 0).all() and r["q"].numel() == 0 and r["scales"].numel() == 0
    ids = torch.full((300, 4), 5, dtype=torch.int32, device="cuda")
    ids[17, 3] = 2
    got = ops.moe_permute_mx(ids, 9, torch.zeros((300, 0), dtype=torch.float32, device="cuda"))
    want = ops.moe_permute(ids, 9)
    torch.cuda.synchronize()
    for name in ("offsets", "dest", "src"):
        assert torch.equal(got[name], want[name]), name
    np.testing.assert_array_equal(to_np(got["offsets"]), [0, 0, 0, 1, 1, 1, 1200, 1200, 1200, 1200])


@pytest.mark.parametrize("counts,F,K", [([0, 1, 300, 0, 37, 256, 511], 128, 256), ([700, 33], 384, 512)])
def test_w4a8_silu_mx_epilogue_equals_silu_then_quantize(counts, F, K):
    """The gate+up epilogue's MXFP8 quantization of H equals, bit for bit,
    mx_quantize of the bf16 H of the plain SiLU-gate epilogue (empty and
    one-row experts, row tails, several tiles); H, Y1 and the amax written
    beside the codes equal the plain epilogue's."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(sum(counts) + F + K)
    E, M = len(counts), sum(counts)
    off = to_gpu(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), torch.int32)
    a = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((E, 2 * F, K)) * 0.05).astype(np.float32)
    aq, as_ = ops.mx_quantize(to_gpu(a, torch.bfloat16), ELEM["e4m3"])
    bq, bs = ops.mx_quantize(to_gpu(b.reshape(E * 2 * F, K), torch.bfloat16), ELEM["e2m1"])
    bq, bs = bq.view(E, 2 * F, K // 2), bs.view(E, 2 * F, K // 32)
    y1, h, amax = ops.grouped_gemm_w4a8_silu_gate(aq, as_, bq, bs, off)
    y1b = torch.empty_like(y1)
    hb = torch.empty_like(h)
    amax_b = torch.empty_like(amax)
    q_h, s_h = ops.grouped_gemm_w4a8_silu_gate_mx(aq, as_, bq, bs, off, y1=y1b, h=hb, amax_out=amax_b)
    q_only, s_only = ops.grouped_gemm_w4a8_silu_gate_mx(aq, as_, bq, bs, off)
    rq, rs = ops.mx_quantize(h, ELEM["e4m3"])
    torch.cuda.synchronize()
    assert torch.equal(q_h, rq) and torch.equal(s_h, rs)
    assert torch.equal(q_only, rq) and torch.equal(s_only, rs)
    assert torch.equal(y1b, y1) and torch.equal(hb, h) and torch.equal(amax_b, amax)

def test_w4a8_full_size_gate_up_sampled():
    """The moe_8k_update gate+up shape (65536 routed rows, 128 experts,
    2F = 1536, K = 2048) as the W4A8 layer runs it: quantize X, permute the
    packed rows, GEMM with the SiLU epilogue; sampled rows of four experts
    against the oracle, the routing metadata bit-exact."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import moe_layer, ops
    d = workloads.moe_8k_update()
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    x = to_gpu(d["x"], torch.bfloat16)
    ids, tw = to_gpu(d["topk_ids"], torch.int32), to_gpu(d["topk_w"], torch.float32)
    wq_gu = moe_layer.quantize_expert_weights_mx(to_gpu(d["w_gu"], torch.bfloat16))
    wq_dn = moe_layer.quantize_expert_weights_mx(to_gpu(d["w_dn"], torch.bfloat16))
    buf = moe_layer.BuffersW4A8(T, k, E, D, F, torch.device("cuda:0"))
    meta = moe_layer.forward_w4a8(x, ids, tw, wq_gu, wq_dn, buf, keep_h=True)
    torch.cuda.synchronize()
    # H's MXFP8 codes from the gate+up epilogue equal mx_quantize of its bf16 H
    hq, hs = ops.mx_quantize(buf.h, ELEM["e4m3"])
    torch.cuda.synchronize()
    R_valid = int(to_np(meta["offsets"])[-1])
    assert torch.equal(buf.a2_q[:R_valid], hq[:R_valid])
    assert torch.equal(buf.a2_s[:R_valid], hs[:R_valid])
    off, dest, src = moe.permute_metadata(d["topk_ids"], E)
    np.testing.assert_array_equal(to_np(meta["offsets"]), off)
    rng = np.random.default_rng(5)
    counts = np.diff(off)
    experts = sorted({0, int(counts.argmax()), E - 1, int(rng.integers(1, E - 1))})
    rows = np.unique(np.concatenate([[off[e], off[e + 1] - 1] + rng.integers(off[e], off[e + 1], 6).tolist()
                                     for e in experts]).astype(np.int64))
    sel = torch.from_numpy(rows).cuda()
    # X quantized per token, then permuted: equals the oracle's quantize of the permuted rows
    xq, xs = mx.quantize(d["x"][src[rows] // k], "e4m3")
    np.testing.assert_array_equal(to_np(buf.a1_q[sel]), xq)
    np.testing.assert_array_equal(to_np(buf.a1_s[sel]), xs)
    bq, bs = to_np(wq_gu["q"]), to_np(wq_gu["s"])
    ref, ab = gemm.grouped_gemm_w4a8(xq, xs, bq, bs, off, rows=rows)
    # the fused epilogue stores H; compare H with the SiLU gate of the
    # oracle's Y1 rounded to bf16, within the GEMM tolerance carried through
    h = to_np(buf.h[sel]).astype(np.float64)
    y1b = bf16_round(ref.astype(np.float32)).astype(np.float64)
    g_ab, u_ab = ab[:, :F], ab[:, F:]
    gv, uv = y1b[:, :F], y1b[:, F:]
    dg = 1e-3 * g_ab + 2.0 ** -8 * (np.abs(gv) + 1e-3 * g_ab)
    du = 1e-3 * u_ab + 2.0 ** -8 * (np.abs(uv) + 1e-3 * u_ab)
    h_ref = moe.silu_gate_fwd(y1b)
    tol = 1.1 * np.abs(uv) * dg + np.abs(moe.silu(gv)) * du + 2.0 ** -8 * np.abs(h_ref) + 1e-30
    err = np.abs(h - h_ref)
    assert (err <= tol).all(), "H: %d of %d out of tolerance" % (int((err > tol).sum()), err.size)
    # H requantized (MXFP8, no amax needed) and the down projection
    hq, hs = mx.quantize(to_np(buf.h[sel]), "e4m3")
    np.testing.assert_array_equal(to_np(buf.a2_q[sel]), hq)
    np.testing.assert_array_equal(to_np(buf.a2_s[sel]), hs)
    ref2, ab2 = gemm.grouped_gemm_w4a8(hq, hs, to_np(wq_dn["q"]), to_np(wq_dn["s"]), off, rows=rows)
    assert_gemm_close(to_np(buf.y2[sel]), ref2, ab2, bf16_out=True, what="w4a8 down")
    # combine of seeded tokens from the GPU's own Y2 rows
    toks = np.sort(rng.choice(T, 32, replace=False))
    sub = dest.reshape(-1, k)[toks].reshape(-1).astype(np.int64)
    y2s = to_np(buf.y2[torch.from_numpy(sub).cuda()])
    local = np.arange(sub.size)
    ref3 = moe.unpermute(y2s, local, k, d["topk_w"][toks])
    got = to_np(buf.out[torch.from_numpy(toks).cuda()])
    bound = moe.unpermute_absbound(y2s, local, k, d["topk_w"][toks])
    assert (np.abs(got - ref3) <= 2.0 ** -8 * np.abs(ref3) + 2.0 ** -16 * bound + 1e-30).all()
