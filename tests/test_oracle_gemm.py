"""Pins for the oracle's grouped GEMMs (CPU only).

* brute-force pure-Python triple loops on tiny shapes, including an empty
  expert and a one-row expert;
* the grouped W4A4 GEMM with one group equals the dense GEMM;
* the TN (weight-gradient) layout gives zeros for an empty expert;
* the absolute-value sum bounds the result.
"""

import numpy as np
import pytest

from oracle import gemm, layer, nvfp4


def _nv(rng, rows, K, groups=1, scale=1.0):
    x = (rng.standard_normal((rows, K)) * scale).astype(np.float32)
    return nvfp4.quantize(x, groups=groups)


@pytest.mark.parametrize("M,N,K,offs", [
    (3, 5, 32, [0, 2, 2, 3]),        # expert 1 empty, expert 2 one row
    (6, 4, 16, [0, 0, 6]),           # first expert empty
    (4, 3, 48, [0, 4]),              # one expert
])
def test_w4a4_brute_force(M, N, K, offs):
    rng = np.random.default_rng(M * 100 + K)
    E = len(offs) - 1
    aq, as_, ag, _ = _nv(rng, M, K)
    bq, bs, bg, _ = _nv(rng, E * N, K, groups=E, scale=0.02)
    bq, bs = bq.reshape(E, N, K // 2), bs.reshape(E, N, K // 16)
    C, AB = gemm.grouped_gemm_w4a4(aq, as_, ag, bq, bs, bg, offs)
    A = nvfp4.dequantize(aq, as_, ag)
    for e in range(E):
        Be = nvfp4.dequantize(bq[e], bs[e], bg[e:e + 1])
        for r in range(offs[e], offs[e + 1]):
            ref = gemm.brute_force_matmul_nt(A[r:r + 1].tolist(), Be.tolist())
            np.testing.assert_allclose(C[r:r + 1], ref, rtol=1e-13, atol=1e-300)
    assert (np.abs(C) <= AB * (1 + 1e-12)).all()


def test_w4a4_row_subset_equals_full():
    rng = np.random.default_rng(11)
    M, N, K, offs = 20, 8, 64, [0, 5, 5, 12, 20]
    aq, as_, ag, _ = _nv(rng, M, K)
    bq, bs, bg, _ = _nv(rng, 4 * N, K, groups=4)
    bq, bs = bq.reshape(4, N, K // 2), bs.reshape(4, N, K // 16)
    C, AB = gemm.grouped_gemm_w4a4(aq, as_, ag, bq, bs, bg, offs)
    rows = np.array([19, 0, 7, 5, 11])
    Cs, ABs = gemm.grouped_gemm_w4a4(aq, as_, ag, bq, bs, bg, offs, rows=rows)
    # BLAS may sum in another order for another row count: fp64 rounding only.
    np.testing.assert_allclose(Cs, C[rows], rtol=1e-12, atol=1e-12 * np.abs(AB).max())
    np.testing.assert_allclose(ABs, AB[rows], rtol=1e-12)


def test_w4a4_single_group_is_dense():
    rng = np.random.default_rng(12)
    aq, as_, ag, _ = _nv(rng, 9, 32)
    bq, bs, bg, _ = _nv(rng, 7, 32)
    C, _ = gemm.dense_gemm_w4a4(aq, as_, ag, bq, bs, bg)
    ref = gemm.brute_force_matmul_nt(nvfp4.dequantize(aq, as_, ag).tolist(),
                                     nvfp4.dequantize(bq, bs, bg).tolist())
    np.testing.assert_allclose(C, ref, rtol=1e-13)


def test_w4a4_global_scales_factor_out():
    # C scales exactly with gA * gB[e] (power-of-two change of the tensors).
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    w = rng.standard_normal((3, 32)).astype(np.float32)
    a = nvfp4.quantize(x)
    b = nvfp4.quantize(w)
    a2 = nvfp4.quantize(x * np.float32(8))
    C1, _ = gemm.dense_gemm_w4a4(*a[:3], *b[:3])
    C2, _ = gemm.dense_gemm_w4a4(*a2[:3], *b[:3])
    np.testing.assert_array_equal(C2, 8 * C1)


def _bf(rng, shape, scale=1.0):
    return layer.bf16_round(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_bf16_layouts_brute_force(layout):
    rng = np.random.default_rng(14)
    offs = [0, 3, 3, 5]
    M, K, N, E = 5, 4, 6, 3
    if layout == "NT":
        a, b = _bf(rng, (M, K)), _bf(rng, (E, N, K))
    elif layout == "NN":
        a, b = _bf(rng, (M, K)), _bf(rng, (E, K, N))
    else:
        a, b = _bf(rng, (M, K)), _bf(rng, (M, N))
    C, AB = gemm.grouped_gemm_bf16(layout, a, b, offs)
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        if layout == "TN":
            ref = gemm.brute_force_matmul_nt(a[lo:hi].T.tolist(), b[lo:hi].T.tolist()) \
                if hi > lo else np.zeros((K, N))
            np.testing.assert_allclose(C[e], ref.reshape(K, N), rtol=1e-13, atol=0)
        else:
            Bt = b[e] if layout == "NT" else b[e].T
            for r in range(lo, hi):
                ref = gemm.brute_force_matmul_nt(a[r:r + 1].tolist(), Bt.tolist())
                np.testing.assert_allclose(C[r:r + 1], ref, rtol=1e-13)
    assert (np.abs(C) <= AB * (1 + 1e-12)).all()
    if layout == "TN":
        assert (C[1] == 0).all()


def test_layer_forward_backward_shapes():
    rng = np.random.default_rng(15)
    T, k, E, D, F = 16, 2, 4, 32, 16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = _bf(rng, (T, D))
    w_gu = _bf(rng, (E, 2 * F, D), 0.1)
    w_dn = _bf(rng, (E, D, F), 0.1)
    f = layer.forward(x, ids, w, w_gu, w_dn)
    assert f["out"].shape == (T, D) and f["h"].shape == (T * k, F)
    b = layer.backward(f, _bf(rng, (T, D), 1e-3), w, w_gu, w_dn)
    assert b["dx"].shape == (T, D) and b["dw_gu"].shape == (E, 2 * F, D) and b["dw_dn"].shape == (E, D, F)
    # dX of a linear-in-X check: the forward output is finite, gradients finite
    assert np.isfinite(f["out"]).all() and np.isfinite(b["dx"]).all()
