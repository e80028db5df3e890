"""Pins for the oracle's NVFP4 backward variant (CPU only).

* column-wise quantization: a hand-worked block placed down one column of a
  segment encodes as the same block quantized along a row; blocks stop at a
  segment's end (the tail block is zero-padded, never filled from the next
  expert); one segment equals the row quantizer on the transposed,
  zero-padded segment; the padded segment columns never overlap;
* every NVFP4 stage equals the BF16 stage (pinned against autograd in
  test_oracle_layer.py) evaluated on the dequantized operands: the wiring of
  the variant is the BF16 backward's, with each GEMM operand replaced by its
  NVFP4 value;
* the whole variant stays within the format's error of the BF16 backward,
  and a planted wiring mistake does not.
"""

import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import gemm, layer, moe, nvfp4
import workloads


def _golden_b1():
    for line in open(os.path.join(GOLDEN, "quant_blocks.txt")):
        if line.strip().startswith("b1"):
            name, amax, xs, ss, qs = [p.strip() for p in line.split(";")]
            return (np.array([float(t) for t in xs.split(",")], np.float32), float(amax),
                    bytes.fromhex(ss.replace(" ", "")), bytes.fromhex(qs.replace(" ", "")))
    raise AssertionError("golden block b1 missing")


def test_colwise_hand_worked_block_down_a_column():
    vals, amax, s_want, q_want = _golden_b1()
    x = np.zeros((16, 3), np.float32)
    x[:, 1] = vals                       # the block runs down column 1 of one 16-row segment
    cols, g = nvfp4.quantize_colwise(x, [0, 16], amax)
    q, s = cols[0]
    assert q.shape == (3, 8) and s.shape == (3, 1)
    assert s[1].tobytes() == s_want and q[1].tobytes() == q_want
    assert (q[[0, 2]] == 0).all() and (s[[0, 2]] == 0).all()
    assert g[0] == nvfp4.global_scale(np.float32(amax))


def test_colwise_blocks_stop_at_segment_ends():
    # expert 0: 20 rows (blocks of 16 + 4 padded), expert 1: 13 rows, expert 2 empty
    rng = np.random.default_rng(2)
    x = rng.standard_normal((33, 4)).astype(np.float32) * 0.01
    x[20, :] = 50.0                      # the first row of expert 1: must not reach expert 0's tail block
    cols, g = nvfp4.quantize_colwise(x, [0, 20, 33, 33], 50.0)
    assert [c[0].shape for c in cols] == [(4, 16), (4, 8), (4, 0)]
    # expert 0's tail block holds rows 16..19 only: its scale is that of those small values
    tail = np.zeros((4, 16), np.float32)
    tail[:, :4] = x[16:20].T
    q_t, s_t, _, _ = nvfp4.quantize(tail, amax=[50.0])
    np.testing.assert_array_equal(cols[0][1][:, 1], s_t[:, 0])
    np.testing.assert_array_equal(cols[0][0][:, 8:], q_t)
    # expert 1's first block contains the large row
    assert (cols[1][1][:, 0] == nvfp4.e4m3_encode(np.float32(50.0 / 6) / nvfp4.global_scale(np.float32(50.0)))).all()


def test_colwise_segment_equals_row_quantizer_on_transpose():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((45, 32)) * np.exp2(rng.integers(-4, 4, (45, 1)))).astype(np.float32)
    amax = np.float32(np.abs(x).max())
    cols, g = nvfp4.quantize_colwise(x, [0, 45], amax)
    xt = np.zeros((32, 48), np.float32)
    xt[:, :45] = x.T
    q, s, g2, _ = nvfp4.quantize(xt, amax=[amax])
    np.testing.assert_array_equal(cols[0][0], q)
    np.testing.assert_array_equal(cols[0][1], s)
    assert g[0] == g2[0]


def test_segment_pad_offsets_do_not_overlap():
    rng = np.random.default_rng(6)
    for _ in range(200):
        E = int(rng.integers(1, 40))
        counts = rng.integers(0, 300, E) * (rng.random(E) < 0.8)
        off = np.concatenate([[0], np.cumsum(counts)])
        p = nvfp4.segment_pad_offset(off)
        padded = -(-counts // 64) * 64
        assert (p % 64 == 0).all()
        assert (p[1:] >= p[:-1] + padded[:-1]).all()
        assert p[-1] + padded[-1] <= nvfp4.padded_extent(off[-1], E)


def _layer(seed, T=48, k=3, E=6, D=64, F=32):
    d = workloads.moe(T, 0.5, with_dy=True, E=E, k=k, D=D, F=F, seed=seed, name="t")
    f = layer.forward(d["x"], d["topk_ids"], d["topk_w"], d["w_gu"], d["w_dn"])
    b = layer.backward(f, d["dy"], d["topk_w"], d["w_gu"], d["w_dn"])
    wt_gu, wt_dn = layer.quantize_weights_t(d["w_gu"]), layer.quantize_weights_t(d["w_dn"])
    bn = layer.backward_nvfp4(f, d["dy"], d["topk_w"], wt_gu, wt_dn)
    return d, f, b, bn, wt_gu, wt_dn


def _deq_colwise_rows(x, offsets, amax):
    """The column-wise NVFP4 of x, dequantized back into x's row layout."""
    cols, g = nvfp4.quantize_colwise(x, offsets, amax)
    out = np.zeros(x.shape)
    for e, (q, s) in enumerate(cols):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            out[lo:hi] = nvfp4.dequantize(q, s, g)[:, :hi - lo].T
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_nvfp4_stages_are_bf16_stages_on_dequantized_operands(seed):
    d, f, b, bn, wt_gu, wt_dn = _layer(seed)
    off, dest, src = f["offsets"], f["dest"], f["src"]
    E = len(off) - 1
    s = dict(f, **bn)
    deq_w = lambda wt: np.stack([nvfp4.dequantize(wt[0][e], wt[1][e], wt[2][e:e + 1]).T for e in range(E)])  # noqa: E731
    close = lambda a, r: np.testing.assert_allclose(a, r, rtol=1e-12, atol=1e-12 * np.abs(r).max())  # noqa: E731
    # data gradients: the BF16 NN stage on the dequantized gradient and weight
    for name, a, w, wt in (("dh", "a_dy2", "w_dn", wt_dn), ("dx_perm", "a_dy1", "w_gu", wt_gu)):
        nv, _ = layer.backward_nvfp4_stage(name, s, d["dy"], d["topk_w"], wt_gu, wt_dn, off, dest, src)
        ref_s = {("dy2" if a == "a_dy2" else "dy1"): nvfp4.dequantize(*s[a])}
        kw = {"w_gu": deq_w(wt_gu) if w == "w_gu" else None, "w_dn": deq_w(wt_dn) if w == "w_dn" else None}
        ref, _ = layer.backward_stage(name, ref_s, d["dy"], d["topk_w"], kw["w_gu"], kw["w_dn"], off, dest, src)
        close(nv, ref)
    # weight gradients: the BF16 TN stage on the dequantized column-wise operands
    for name, ga, gb, am_a, am_b in (("dw_dn", "dy2", "h", s["amax_dy2"], s["amax_h"]),
                                     ("dw_gu", "dy1", "x_perm", s["amax_dy1"], s["amax_x"])):
        nv, _ = layer.backward_nvfp4_stage(name, s, d["dy"], d["topk_w"], wt_gu, wt_dn, off, dest, src)
        ref_s = {ga: _deq_colwise_rows(s[ga], off, am_a), gb: _deq_colwise_rows(s[gb], off, am_b)}
        ref, _ = layer.backward_stage(name, ref_s, d["dy"], d["topk_w"], None, None, off, dest, src)
        close(nv, ref)
    # the transposed weights reuse the forward weights' per-expert global scales
    np.testing.assert_array_equal(wt_gu[2], layer.quantize_weights(d["w_gu"])[2])


def test_nvfp4_backward_within_format_error_of_bf16():
    for seed in (0, 1, 2):
        d, f, b, bn, _, _ = _layer(seed)
        fro = lambda g, r: np.linalg.norm(g - r) / np.linalg.norm(r)  # noqa: E731
        for n in ("dx", "dw_gu", "dw_dn", "dh", "dx_perm"):
            assert fro(bn[n], b[n]) < 0.3, (seed, n, fro(bn[n], b[n]))
        # planted: the routing weight applied again at the dX combine; dW_dn from Y1's gate half
        assert fro(moe.unpermute(bn["dx_perm"], f["dest"], 3, d["topk_w"]), b["dx"]) > 0.4
        assert fro(gemm.grouped_gemm_bf16("TN", b["dy2"], f["y1"][:, :32], f["offsets"])[0], b["dw_dn"]) > 0.4
