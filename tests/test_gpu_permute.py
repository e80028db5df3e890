"""GPU parity of moe_permute / moe_gather / moe_unpermute.  Offsets, dest,
src and gathered rows must equal the oracle's exactly; weighted sums are
checked within their fp32/bf16 rounding."""

import os

import numpy as np
import pytest
import torch

import workloads
from _helpers import assert_bf16_close, gpu, require_gpu, to_gpu, to_np
from conftest import GOLDEN
from oracle import moe, nvfp4
from oracle.layer import bf16_round

pytestmark = gpu


def _meta(ids_np, E, x_np=None, dtype=torch.bfloat16, status=None):
    from nvfp4_quantized_moe_token_amd import ops
    ids = to_gpu(ids_np, torch.int32)
    x = None if x_np is None else to_gpu(x_np, dtype)
    r = ops.moe_permute(ids, E, x=x, want_amax=x is not None, status=status)
    torch.cuda.synchronize()
    return r


def _check_meta(ids_np, E, r):
    off, dest, src = moe.permute_metadata(ids_np, E)
    np.testing.assert_array_equal(to_np(r["offsets"]), off)
    np.testing.assert_array_equal(to_np(r["dest"]), dest)
    np.testing.assert_array_equal(to_np(r["src"]), src)
    return off, dest, src


def test_worked_example():
    require_gpu()
    d = {}
    for line in open(os.path.join(GOLDEN, "permute_example.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            d[key] = [int(v) for v in vals]
    ids = np.array(d["ids"], np.int32).reshape(d["T"][0], d["k"][0])
    r = _meta(ids, d["E"][0])
    assert to_np(r["offsets"]).tolist() == d["offsets"]
    assert to_np(r["dest"]).tolist() == d["dest"]
    assert to_np(r["src"]).tolist() == d["src"]


@pytest.mark.parametrize("cfg", ["moe_4k", "moe_16k_skew", "moe_8k_update"])
def test_config_routing_and_gather(cfg):
    require_gpu()
    d = workloads.CONFIGS[cfg](weights=False)
    r = _meta(d["topk_ids"], d["E"], d["x"])
    off, dest, src = _check_meta(d["topk_ids"], d["E"], r)
    xp = to_np(r["x_perm"])
    rows = np.random.default_rng(0).choice(xp.shape[0], 4096, replace=False)
    np.testing.assert_array_equal(xp[rows], d["x"][src[rows] // d["k"]])
    assert to_np(r["amax"])[0] == np.abs(d["x"]).max()


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (5, 3, 4, 1), (1000, 8, 16, 2), (777, 2, 3, 3),
                                        (3000, 8, 2000, 4), (4096, 8, 128, 5)])
def test_random_routing(T, k, E, seed):
    require_gpu()
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)   # duplicates inside a token allowed
    _check_meta(ids, E, _meta(ids, E))


def test_all_to_one_expert_and_empty_experts():
    require_gpu()
    ids = np.full((2000, 4), 5, np.int32)
    _check_meta(ids, 9, _meta(ids, 9))


def test_zero_tokens():
    require_gpu()
    ids = np.zeros((0, 8), np.int32)
    r = _meta(ids, 16, np.zeros((0, 64), np.float32))
    assert to_np(r["offsets"]).tolist() == [0] * 17
    assert to_np(r["amax"])[0] == 0.0


def test_bad_expert_ids_flagged_and_skipped():
    require_gpu()
    ids = np.array([[0, 1], [7, 2], [1, -1], [2, 0]], np.int32)   # 7 and -1 are out of range for E = 4
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    r = _meta(ids, 4, status=status)
    from nvfp4_quantized_moe_token_amd import _lib
    assert int(status.item()) & _lib.STATUS_BAD_EXPERT
    dest = to_np(r["dest"])
    assert dest[2] == -1 and dest[5] == -1
    off = to_np(r["offsets"])
    assert off[-1] == 6
    valid = ids.reshape(-1)
    keep = (valid >= 0) & (valid < 4)
    o2, d2, s2 = moe.permute_metadata(np.where(keep, valid, 0)[keep].reshape(1, -1), 4)
    np.testing.assert_array_equal(off, o2)
    src = to_np(r["src"])
    assert (src[6:] == -1).all()
    np.testing.assert_array_equal(np.nonzero(keep)[0][s2], src[:6])


def test_deterministic():
    require_gpu()
    d = workloads.moe_4k(weights=False)
    a = _meta(d["topk_ids"], 128)
    b = _meta(d["topk_ids"], 128)
    for key in ("offsets", "dest", "src"):
        np.testing.assert_array_equal(to_np(a[key]), to_np(b[key]))


def test_packed_gather_commutes_with_quantize():
    # quantize(permute(X)) == permute(quantize(X)) bit for bit on the GPU.
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.moe(512, 1.1, 0.01, 32.0, weights=False, name="t")
    x = to_gpu(d["x"], torch.bfloat16)
    ids = to_gpu(d["topk_ids"], torch.int32)
    r = ops.moe_permute(ids, 128, x=x, want_amax=True)
    q1, s1, g1, _ = ops.nvfp4_quantize(r["x_perm"], amax_in=r["amax"])
    q0, s0, g0, _ = ops.nvfp4_quantize(x)
    q2 = ops.moe_gather(q0, r["src"], 8)
    s2 = ops.moe_gather(s0, r["src"], 8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(q1), to_np(q2))
    np.testing.assert_array_equal(to_np(s1), to_np(s2))
    assert to_np(g0)[0] == to_np(g1)[0]


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
def test_weighted_gather(in_dt, out_dt):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(7)
    T, k, E, D = 300, 4, 10, 136
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    dy = (rng.standard_normal((T, D)) * 1e-3).astype(np.float32)
    r = _meta(ids, E)
    out = ops.moe_gather(to_gpu(dy, in_dt), r["src"], k, topk_w=to_gpu(w, torch.float32), out_dtype=out_dt)
    torch.cuda.synchronize()
    src = to_np(r["src"])
    dyv = to_np(to_gpu(dy, in_dt))
    ref = moe.gather_rows(dyv, src, k, w)
    if out_dt == torch.float32:
        np.testing.assert_allclose(to_np(out), ref, rtol=2.0 ** -23, atol=0)
    else:
        assert_bf16_close(to_np(out), ref, what="weighted gather")


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                           (torch.float32, torch.float32), (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("k", [3, 8, 11])
def test_scatter_equals_weighted_gather(in_dt, out_dt, weighted, k):
    """moe_scatter (token side) and moe_gather (row side) write the same bits
    for one permutation, including invalid ids (skipped, rows past
    offsets[E] zero); with the amax, top-k below, at and above the eight ids
    the amax variant's kernel holds per piece (past eight: the plain loop)."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(41 + k)
    T, E, D = 700, 24, 264
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[5, k - 1] = E + 1
    ids[99, 0] = -2
    r = _meta(ids, E)
    x = to_gpu(rng.standard_normal((T, D)).astype(np.float32) * 3, in_dt)
    w = to_gpu(rng.random((T, k)).astype(np.float32), torch.float32) if weighted else None
    g = ops.moe_gather(x, r["src"], k, topk_w=w, out_dtype=out_dt) if weighted else None
    if not weighted:
        # unweighted moe_gather copies verbatim (no dtype change): compare in the input dtype
        g = ops.moe_gather(x, r["src"], k).to(out_dt)
    sc = ops.moe_scatter(x, r["dest"], r["offsets"], k, topk_w=w, out_dtype=out_dt)
    amax = torch.full((1,), 123.0, dtype=torch.float32, device="cuda")   # cleared by the call
    sc2 = ops.moe_scatter(x, r["dest"], r["offsets"], k, topk_w=w, out_dtype=out_dt, amax_out=amax)
    torch.cuda.synchronize()
    assert torch.equal(sc, g)
    assert torch.equal(sc2, sc)                 # the amax changes nothing written
    assert float(amax) == float(sc.float().abs().max())
    R_valid = int(to_np(r["offsets"])[-1])
    assert R_valid == T * k - 2 and (to_np(sc)[R_valid:] == 0).all()


def test_scatter_moe_8k_matches_oracle_sampled():
    """dY2 of the 8k update by scatter against the oracle's gather (fp32
    product rounded once to bf16), on every row, and its fused amax."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.moe_8k_update(weights=False)
    T, k, E = d["T"], d["k"], d["E"]
    r = _meta(d["topk_ids"], E)
    dy = to_gpu(d["dy"], torch.bfloat16)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    out = ops.moe_scatter(dy, r["dest"], r["offsets"], k, topk_w=to_gpu(d["topk_w"], torch.float32),
                          amax_out=amax)
    torch.cuda.synchronize()
    src = to_np(r["src"])
    ref = moe.gather_rows(to_np(dy), src, k).astype(np.float32) * d["topk_w"].reshape(-1)[src][:, None]
    want = bf16_round(ref.astype(np.float32))
    np.testing.assert_array_equal(to_np(out), want)
    # the fused amax (capped grid, one atomic per workgroup) is max |dY2|
    assert np.float32(amax.item()) == np.abs(want).max()


@pytest.mark.parametrize("weighted", [True, False])
def test_unpermute(weighted):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.moe_4k(weights=False)
    T, k, D = d["T"], d["k"], d["D"]
    r = _meta(d["topk_ids"], 128)
    rng = np.random.default_rng(8)
    y = rng.standard_normal((T * k, D)).astype(np.float32)
    yg = to_gpu(y, torch.bfloat16)
    w = to_gpu(d["topk_w"], torch.float32) if weighted else None
    out = ops.moe_unpermute(yg, r["dest"], T, k, topk_w=w)
    out32 = ops.moe_unpermute(yg, r["dest"], T, k, topk_w=w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    dest = to_np(r["dest"])
    ref = moe.unpermute(to_np(yg), dest, k, d["topk_w"] if weighted else None)
    scale = moe.unpermute_absbound(to_np(yg), dest, k, d["topk_w"] if weighted else None)
    assert_bf16_close(to_np(out), ref, scale=scale, what="unpermute bf16")
    err = np.abs(to_np(out32) - ref)
    assert (err <= 2.0 ** -21 * scale + 1e-30).all()
    # The bf16 output is the fp32 output (same fma order) rounded once.
    assert torch.equal(out, out32.to(torch.bfloat16))


@pytest.mark.parametrize("weighted", [True, False])
def test_unpermute_skipped_assignments(weighted):
    """Assignments with dest = -1 (skipped by the permutation) add nothing:
    the reference is the oracle's sum with those weights set to zero."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(31)
    T, k, D, R = 300, 8, 256, 2400
    dest = rng.permutation(R).astype(np.int32)
    skip = rng.random(R) < 0.05
    dest_g = dest.copy()
    dest_g[skip] = -1
    y = workloads._bf16(rng.standard_normal((R, D)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32) if weighted else None
    out = ops.moe_unpermute(to_gpu(y, torch.bfloat16), to_gpu(dest_g, torch.int32), T, k,
                            topk_w=None if w is None else to_gpu(w, torch.float32), out_dtype=torch.float32)
    torch.cuda.synchronize()
    w_eff = (np.ones((T, k), np.float32) if w is None else w).reshape(-1).copy()
    w_eff[skip] = 0.0
    ref = moe.unpermute(y, dest, k, w_eff.reshape(T, k))
    scale = moe.unpermute_absbound(y, dest, k, w_eff.reshape(T, k))
    assert (np.abs(to_np(out) - ref) <= 2.0 ** -21 * scale + 1e-30).all()


@pytest.mark.parametrize("cfg", ["moe_4k", "moe_16k_skew", "moe_8k_update"])
@pytest.mark.parametrize("with_x_perm", [True, False])
def test_permute_nvfp4_matches_oracle(cfg, with_x_perm):
    """Fused gather + quantize: metadata, x_perm, codes and scales bit-exact
    against the oracle's quantize(permute(X)) with amax(X)."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    d = workloads.CONFIGS[cfg](weights=False)
    E, k = d["E"], d["k"]
    r = ops.moe_permute_nvfp4(to_gpu(d["topk_ids"], torch.int32), E, to_gpu(d["x"], torch.bfloat16),
                              want_x_perm=with_x_perm)
    torch.cuda.synchronize()
    off, dest, src = _check_meta(d["topk_ids"], E, r)
    amax = np.float32(np.abs(d["x"]).max())
    assert to_np(r["amax"])[0] == amax
    xp = moe.gather_rows(d["x"], src, k)
    if with_x_perm:
        np.testing.assert_array_equal(to_np(r["x_perm"]), xp)
    else:
        assert r["x_perm"] is None
    # Sampled rows (the full 16k-token oracle quantization is slow): every
    # expert's first and last row plus a seeded sample.
    rng = np.random.default_rng(5)
    rows = set(rng.choice(len(src), min(len(src), 3000), replace=False).tolist())
    for e in range(E):
        if off[e + 1] > off[e]:
            rows.update([int(off[e]), int(off[e + 1]) - 1])
    rows = np.array(sorted(rows))
    q, s, g, _ = nvfp4.quantize(xp[rows], amax=[amax])
    np.testing.assert_array_equal(to_np(r["q"])[rows], q)
    np.testing.assert_array_equal(to_np(r["scales"])[rows], s)
    assert to_np(r["gscale"])[0] == g[0]


def test_permute_nvfp4_equals_unfused_path():
    """moe_permute + nvfp4_quantize(amax_in) and the fused call agree bit for
    bit, with a given amax (reuse) and with invalid ids present."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(9)
    T, k, E, D = 700, 4, 9, 256
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[3, 1] = E + 2          # out of range: row past offsets[E]
    ids[10, 0] = -1
    x = workloads._bf16(rng.standard_normal((T, D)).astype(np.float32) * 3)
    ids_g, x_g = to_gpu(ids, torch.int32), to_gpu(x, torch.bfloat16)
    amax = to_gpu(np.array([np.abs(x).max() * 1.5], np.float32), torch.float32)  # a stale, larger amax
    st1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    st2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = ops.moe_permute(ids_g, E, x=x_g, status=st1)
    qa, sa, ga, _ = ops.nvfp4_quantize(a["x_perm"], amax_in=amax)
    b = ops.moe_permute_nvfp4(ids_g, E, x_g, amax_in=amax, status=st2)
    torch.cuda.synchronize()
    for key in ("offsets", "dest", "src", "x_perm"):
        np.testing.assert_array_equal(to_np(a[key]), to_np(b[key]))
    np.testing.assert_array_equal(to_np(qa), to_np(b["q"]))
    np.testing.assert_array_equal(to_np(sa), to_np(b["scales"]))
    np.testing.assert_array_equal(to_np(ga), to_np(b["gscale"]))
    assert to_np(st1)[0] == to_np(st2)[0] == 1
    R_valid = int(to_np(b["offsets"])[-1])
    assert (to_np(b["q"])[R_valid:] == 0).all() and (to_np(b["scales"])[R_valid:] == 0).all()


def test_permute_nvfp4_computed_amax_clears_stale_buffer_and_marks_tail():
    """Fused call with the amax computed: a stale amax_out (larger than any
    |x|) is cleared before the reduction, and with invalid ids the src rows
    past offsets[E] are -1 (written by the scan) on two calls in a row."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(21)
    T, k, E, D = 515, 8, 12, 128
    x = workloads._bf16(rng.standard_normal((T, D)).astype(np.float32))
    x_g = to_gpu(x, torch.bfloat16)
    amax_out = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    for bad in (3, 11):
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
        bad_at = rng.choice(T * k, bad, replace=False)
        ids.reshape(-1)[bad_at] = np.where(np.arange(bad) % 2 == 0, E, -3)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        r = ops.moe_permute_nvfp4(to_gpu(ids, torch.int32), E, x_g, amax_out=amax_out, status=st)
        torch.cuda.synchronize()
        assert to_np(amax_out)[0] == np.float32(np.abs(x).max())
        off = to_np(r["offsets"])
        assert off[-1] == T * k - bad
        src = to_np(r["src"])
        assert (src[T * k - bad:] == -1).all() and (src[:T * k - bad] >= 0).all()
        dest = to_np(r["dest"])
        assert (dest[bad_at] == -1).all()
        assert to_np(st)[0] == 1
        keep = np.ones(T * k, bool)
        keep[bad_at] = False
        flat = ids.reshape(-1)
        o2, _, s2 = moe.permute_metadata(np.where(keep, flat, 0)[keep].reshape(1, -1), E)
        np.testing.assert_array_equal(off, o2)
        np.testing.assert_array_equal(np.nonzero(keep)[0][s2], src[:T * k - bad])


def test_permute_nvfp4_zero_tokens():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    ids = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    r = ops.moe_permute_nvfp4(ids, 16, x)
    torch.cuda.synchronize()
    assert (to_np(r["offsets"]) == 0).all()
    assert to_np(r["amax"])[0] == 0.0 and to_np(r["gscale"])[0] == 1.0


def test_permute_nvfp4_amax_counts_unrouted_token():
    """A token whose ids are all invalid has no permuted row, yet the
    computed amax is over every row of x (the header's contract), and the
    codes are those of the oracle's quantize of the routed rows with that
    amax.  With D == 0 the computed amax is 0."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rng = np.random.default_rng(31)
    T, k, E, D = 40, 3, 6, 64
    x = workloads._bf16(rng.standard_normal((T, D)).astype(np.float32))
    x[7, 5] = 96.0                       # the largest |x| sits in the unrouted token
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[7] = [E, -1, E + 4]
    amax_out = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    r = ops.moe_permute_nvfp4(to_gpu(ids, torch.int32), E, to_gpu(x, torch.bfloat16), amax_out=amax_out)
    torch.cuda.synchronize()
    assert to_np(amax_out)[0] == np.float32(96.0)
    off = to_np(r["offsets"])
    R_valid = int(off[-1])
    assert R_valid == T * k - k
    src = to_np(r["src"])[:R_valid]
    q, s, g, _ = nvfp4.quantize(x[src // k], amax=[np.float32(96.0)])
    np.testing.assert_array_equal(to_np(r["q"])[:R_valid], q)
    np.testing.assert_array_equal(to_np(r["scales"])[:R_valid], s)
    assert to_np(r["gscale"])[0] == g[0]
    # no elements per row: the amax is cleared, the global scale is 1
    amax_out.fill_(5.0)
    x0 = torch.zeros((T, 0), dtype=torch.bfloat16, device="cuda")
    r0 = ops.moe_permute_nvfp4(to_gpu(ids, torch.int32), E, x0, amax_out=amax_out, want_x_perm=False)
    torch.cuda.synchronize()
    assert to_np(amax_out)[0] == 0.0 and to_np(r0["gscale"])[0] == 1.0
