"""Pins for the oracle's MoE layer composition (CPU only).

The layer's stages are pinned one by one elsewhere (quantizer, permutation,
GEMMs, SiLU gate, combine).  What these tests pin is the wiring between
them, against things that do not share it:

* the forward against a per-token loop with no permutation at all: for each
  token t and slot j, the expert e = ids[t, j], the quantized chain of that
  one row, then sum_j w[t, j] * y2;
* the backward against torch.autograd in float64 on a tiny unquantized
  layer, fed that layer's own Y1 and H (the BF16 backward differentiates the
  bf16 tensors, not the quantized ones);
* the row-restricted stage functions (used by the full-size GPU tests)
  against the full-tensor stages.

A wiring mistake -- the routing weight applied twice or not at all, the
wrong operand in a weight gradient, a transposed weight, dest used for src
-- fails one of these.
"""

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import layer, moe, nvfp4


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _routing(rng, T, k, experts):
    """Distinct experts per token drawn from ``experts`` (others stay empty)."""
    ids = np.stack([rng.choice(experts, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.2, 0.9, (T, k)).astype(np.float32)   # deliberately not normalised
    return ids, w


def _inputs(seed, T, k, E, D, F, experts):
    rng = np.random.default_rng(seed)
    ids, w = _routing(rng, T, k, experts)
    x = rng.standard_normal((T, D)).astype(np.float32)
    x[rng.random((T, D)) < 0.03] *= 12.0
    x = _bf(x)
    w_gu = _bf(rng.standard_normal((E, 2 * F, D)) * 0.1)
    w_dn = _bf(rng.standard_normal((E, D, F)) * 0.1)
    dy = _bf(rng.standard_normal((T, D)) * 1e-2)
    return ids, w, x, w_gu, w_dn, dy


def test_forward_matches_per_token_loop():
    T, k, E, D, F = 9, 3, 5, 64, 32
    ids, w, x, w_gu, w_dn, _ = _inputs(11, T, k, E, D, F, [0, 1, 2, 4])   # expert 3 empty
    f = layer.forward(x, ids, w, w_gu, w_dn)

    # Independent composition: token by token, slot by slot, every expert
    # weight quantized on its own (one tensor each), no permutation.
    amax_x = np.float32(np.abs(x).max())
    deq_w = lambda wt: nvfp4.dequantize(*nvfp4.quantize(wt)[:3])  # noqa: E731
    y1 = np.zeros((T, k, 2 * F))
    h = np.zeros((T, k, F), np.float32)
    for t in range(T):
        xa = nvfp4.dequantize(*nvfp4.quantize(x[t:t + 1], amax=[amax_x])[:3])[0]
        for j in range(k):
            y = deq_w(w_gu[ids[t, j]]) @ xa
            y1[t, j] = _bf(y)
            g, u = y1[t, j, :F], y1[t, j, F:]
            h[t, j] = _bf(g * expit(g) * u)
    amax_h = np.float32(np.abs(h).max())
    y2 = np.zeros((T, k, D))
    out = np.zeros((T, D))
    for t in range(T):
        for j in range(k):
            ha = nvfp4.dequantize(*nvfp4.quantize(h[t, j][None], amax=[amax_h])[:3])[0]
            y2[t, j] = _bf(deq_w(w_dn[ids[t, j]]) @ ha)
            out[t] += np.float64(w[t, j]) * y2[t, j]
    out = _bf(out)

    dest = f["dest"].reshape(T, k)
    one_ulp = lambda ref: 2.0 ** -8 * np.abs(ref) + 1e-30  # noqa: E731
    assert f["amax_x"] == amax_x and f["amax_h"] == amax_h
    for t in range(T):
        for j in range(k):
            p = dest[t, j]
            assert (np.abs(f["y1"][p] - y1[t, j]) <= one_ulp(y1[t, j])).all()
            assert (np.abs(f["h"][p] - h[t, j]) <= one_ulp(h[t, j])).all()
            assert (np.abs(f["y2"][p] - y2[t, j]) <= one_ulp(y2[t, j])).all()
    assert (np.abs(f["out"] - out) <= one_ulp(out)).all()
    # the routing weight enters once: dropping it, or squaring it, is far off
    bad = _bf(np.einsum("tj,tjd->td", w.astype(np.float64) ** 2, y2))
    assert np.abs(f["out"] - bad).max() > 0.1 * np.abs(out).max()


def _autograd_layer(ids, w, x, w_gu, w_dn, dy):
    """Unquantized layer in float64 with torch.autograd: per token and slot,
    y1 = W_gu[e] x, h = silu(g) u, y2 = W_dn[e] h, out = sum_j w y2."""
    T, k = ids.shape
    F = w_dn.shape[2]
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    Wgu = torch.tensor(w_gu, dtype=torch.float64, requires_grad=True)
    Wdn = torch.tensor(w_dn, dtype=torch.float64, requires_grad=True)
    out = torch.zeros(T, x.shape[1], dtype=torch.float64)
    y1s, hs = {}, {}
    for t in range(T):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(k):
            e = int(ids[t, j])
            y1 = Wgu[e] @ X[t]
            hh = torch.nn.functional.silu(y1[:F]) * y1[F:]
            y1s[(t, j)], hs[(t, j)] = y1.detach().numpy(), hh.detach().numpy()
            acc = acc + float(w[t, j]) * (Wdn[e] @ hh)
        out[t] = acc
    (out * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return X.grad.numpy(), Wgu.grad.numpy(), Wdn.grad.numpy(), y1s, hs


@pytest.mark.parametrize("T,k,E,D,F,experts", [
    (6, 2, 4, 32, 16, [0, 1, 3]),          # expert 2 empty
    (10, 3, 5, 48, 32, [0, 1, 2, 3, 4]),
])
def test_backward_matches_autograd(T, k, E, D, F, experts):
    ids, w, x, w_gu, w_dn, dy = _inputs(T * 7 + k, T, k, E, D, F, experts)
    dx_ref, dwgu_ref, dwdn_ref, y1s, hs = _autograd_layer(ids, w, x, w_gu, w_dn, dy)
    off, dest, src = moe.permute_metadata(ids, E)
    fwd = dict(offsets=off, dest=dest, src=src, x_perm=x[src // k].astype(np.float64),
               y1=np.zeros((T * k, 2 * F)), h=np.zeros((T * k, F)))
    for t in range(T):
        for j in range(k):
            fwd["y1"][dest[t * k + j]] = y1s[(t, j)]
            fwd["h"][dest[t * k + j]] = hs[(t, j)]
    b = layer.backward(fwd, dy, w, w_gu, w_dn)
    # bf16 storage of dY2, dH, dY1, dX_perm and dX: a few 2^-9 relative
    # roundings compound; 3% of the tensor's largest entry bounds them.
    for name, got, ref in (("dx", b["dx"], dx_ref), ("dw_gu", b["dw_gu"], dwgu_ref),
                           ("dw_dn", b["dw_dn"], dwdn_ref)):
        assert got.shape == ref.shape, name
        err = np.abs(got.astype(np.float64) - ref).max()
        assert err <= 0.03 * np.abs(ref).max(), (name, err, np.abs(ref).max())
    for e in set(range(E)) - set(experts):
        assert (b["dw_gu"][e] == 0).all() and (b["dw_dn"][e] == 0).all()
        assert (dwgu_ref[e] == 0).all()


def test_backward_planted_wiring_mistakes_fail():
    # The autograd pin is sharp enough to see the plausible mistakes: each
    # planted variant of one stage (on the CPU, in a copy of the chain)
    # leaves the tolerance of test_backward_matches_autograd.
    T, k, E, D, F = 10, 3, 5, 48, 32
    ids, w, x, w_gu, w_dn, dy = _inputs(73, T, k, E, D, F, [0, 1, 2, 3, 4])
    dx_ref, dwgu_ref, dwdn_ref, y1s, hs = _autograd_layer(ids, w, x, w_gu, w_dn, dy)
    off, dest, src = moe.permute_metadata(ids, E)
    fwd = dict(offsets=off, dest=dest, src=src, x_perm=x[src // k].astype(np.float64),
               y1=np.zeros((T * k, 2 * F)), h=np.zeros((T * k, F)))
    for t in range(T):
        for j in range(k):
            fwd["y1"][dest[t * k + j]] = y1s[(t, j)]
            fwd["h"][dest[t * k + j]] = hs[(t, j)]
    good = layer.backward(fwd, dy, w, w_gu, w_dn)

    def far(got, ref):
        return np.abs(got - ref).max() > 0.03 * np.abs(ref).max()

    assert not far(good["dx"], dx_ref)
    # routing weight applied a second time at the dX combine
    dx_twice = moe.unpermute(good["dx_perm"], dest, k, w)
    assert far(dx_twice, dx_ref)
    from oracle import gemm
    # dW_dn from the gate half of Y1 instead of H (wrong stored operand)
    assert far(gemm.grouped_gemm_bf16("TN", good["dy2"], fwd["y1"][:, :F], off)[0], dwdn_ref)
    # the weight gradient of the gate+up projection with gate and up swapped
    dy1_sw = np.concatenate([good["dy1"][:, F:], good["dy1"][:, :F]], axis=1)
    assert far(gemm.grouped_gemm_bf16("TN", dy1_sw, fwd["x_perm"], off)[0], dwgu_ref)
    # dX_perm through W_gu transposed the wrong way is a shape error; through
    # the wrong expert's weights it is far off
    wrong = np.roll(w_gu, 1, axis=0)
    dxp = gemm.grouped_gemm_bf16("NN", good["dy1"], wrong, off)[0]
    assert far(moe.unpermute(dxp, dest, k, None), dx_ref)
    # src in place of dest at the combine
    assert far(moe.unpermute(good["dx_perm"], src, k, None), dx_ref)


@pytest.mark.parametrize("seed", [0, 1])
def test_row_restricted_stages_equal_full(seed):
    T, k, E, D, F = 12, 4, 6, 64, 32
    ids, w, x, w_gu, w_dn, dy = _inputs(seed, T, k, E, D, F, [0, 2, 3, 4, 5])
    wq_gu, wq_dn = layer.quantize_weights(w_gu), layer.quantize_weights(w_dn)
    f = layer.forward(x, ids, w, w_gu, w_dn, wq_gu=wq_gu, wq_dn=wq_dn)
    b = layer.backward(f, dy, w, w_gu, w_dn)
    off, dest, src = f["offsets"], f["dest"], f["src"]
    rows = np.random.default_rng(seed).choice(T * k, 17, replace=False)
    sub = lambda a: a[rows] if not isinstance(a, tuple) else tuple(v[rows] if v.ndim == 2 else v for v in a)  # noqa: E731
    s = {n: sub(f[n]) for n in ("x_perm", "a1", "y1", "h", "a2")}
    s.update(amax_x=f["amax_x"], amax_h=f["amax_h"])
    for name in ("x_perm", "y1", "h", "y2"):
        full, _ = layer.forward_stage(name, f, x, w, wq_gu, wq_dn, off, dest, src)
        part, _ = layer.forward_stage(name, s, x, w, wq_gu, wq_dn, off, dest, src, rows=rows)
        # fp64 matmuls of a few rows may differ from the full ones in the last bits
        np.testing.assert_allclose(part, full[rows], rtol=1e-12, atol=1e-300, err_msg=name)
    sb = {n: sub(v) for n, v in list(b.items()) + [("y1", f["y1"])] if n in ("dy2", "dh", "dy1", "y1")}
    full_s = dict(b, y1=f["y1"], h=f["h"], x_perm=f["x_perm"])
    for name in ("dy2", "dh", "dy1", "dx_perm"):
        full, _ = layer.backward_stage(name, full_s, dy, w, w_gu, w_dn, off, dest, src)
        part, _ = layer.backward_stage(name, sb, dy, w, w_gu, w_dn, off, dest, src, rows=rows)
        np.testing.assert_allclose(part, full[rows], rtol=1e-12, atol=1e-300, err_msg=name)
