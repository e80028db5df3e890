"""Pins for the oracle's permutation, gather/unpermute, SiLU gate and bf16
rounding (CPU only).

* permutation: the hand-worked example (tests/golden/permute_example.txt) and
  a brute-force counting loop written out element by element;
* gather / unpermute: brute-force loops on tiny inputs;
* SiLU gate: scipy's logistic function, closed forms at 0, and a central
  finite difference for the backward;
* bf16 rounding: torch's float32 -> bfloat16 conversion;
* invariants: quantize commutes with the permutation, amax is unchanged.
"""

import os

import numpy as np
import pytest
import scipy.special
import torch

from conftest import GOLDEN
from oracle import layer, moe, nvfp4


def _load_example():
    d = {}
    with open(os.path.join(GOLDEN, "permute_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = [int(v) for v in vals]
    return d


def test_permute_worked_example():
    ex = _load_example()
    ids = np.array(ex["ids"], dtype=np.int32).reshape(ex["T"][0], ex["k"][0])
    off, dest, src = moe.permute_metadata(ids, ex["E"][0])
    assert off.tolist() == ex["offsets"]
    assert dest.tolist() == ex["dest"]
    assert src.tolist() == ex["src"]
    assert (src // ex["k"][0]).tolist() == ex["tokens"]


def _brute_counting_sort(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    cursor = offsets[:E]
    dest = [0] * len(flat)
    src = [0] * len(flat)
    for i, e in enumerate(flat):
        dest[i] = cursor[e]
        src[cursor[e]] = i
        cursor[e] += 1
    return offsets, dest, src


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 2, 5, 1), (64, 8, 16, 2),
                                        (200, 8, 128, 3), (33, 3, 4, 4)])
def test_permute_brute_force(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)   # duplicates allowed
    off, dest, src = moe.permute_metadata(ids, E)
    bo, bd, bs = _brute_counting_sort(ids, E)
    assert off.tolist() == bo and dest.tolist() == bd and src.tolist() == bs


def test_permute_invariants():
    rng = np.random.default_rng(5)
    T, k, E = 300, 8, 32
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, dest, src = moe.permute_metadata(ids, E)
    assert off[0] == 0 and off[-1] == T * k and (np.diff(off) >= 0).all()
    assert (src[dest] == np.arange(T * k)).all()
    flat = ids.reshape(-1)
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_permute_empty_and_range():
    off, dest, src = moe.permute_metadata(np.zeros((0, 8), np.int32), 4)
    assert off.tolist() == [0] * 5 and dest.size == 0 and src.size == 0
    with pytest.raises(ValueError):
        moe.permute_metadata(np.array([[4]], np.int32), 4)


def test_gather_unpermute_brute_force():
    rng = np.random.default_rng(6)
    T, k, E, D = 5, 3, 4, 7
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = rng.standard_normal((T, D))
    off, dest, src = moe.permute_metadata(ids, E)
    xp = moe.gather_rows(x, src, k)
    xpw = moe.gather_rows(x, src, k, w)
    for t in range(T):
        for j in range(k):
            p = dest[t * k + j]
            for c in range(D):
                assert xp[p, c] == x[t, c]
                assert xpw[p, c] == float(w[t, j]) * x[t, c]
    y = rng.standard_normal((T * k, D))
    out = moe.unpermute(y, dest, k, w)
    out1 = moe.unpermute(y, dest, k, None)
    for t in range(T):
        for c in range(D):
            acc = acc1 = 0.0
            for j in range(k):
                acc += float(w[t, j]) * y[dest[t * k + j], c]
                acc1 += y[dest[t * k + j], c]
            assert abs(out[t, c] - acc) <= 1e-12 * (1 + abs(acc))
            assert abs(out1[t, c] - acc1) <= 1e-12 * (1 + abs(acc1))


def test_quantize_commutes_with_permutation():
    rng = np.random.default_rng(7)
    T, k, E, D = 50, 4, 8, 64
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, D)).astype(np.float32)
    off, dest, src = moe.permute_metadata(ids, E)
    xp = moe.gather_rows(x, src, k).astype(np.float32)
    amax = float(np.abs(x).max())
    assert float(np.abs(xp).max()) == amax            # every token is routed
    q1, s1, g1, _ = nvfp4.quantize(xp, amax=[amax])
    q0, s0, g0, _ = nvfp4.quantize(x)
    np.testing.assert_array_equal(q1, q0[src // k])
    np.testing.assert_array_equal(s1, s0[src // k])
    assert g0[0] == g1[0]


def test_silu_matches_scipy_and_closed_forms():
    v = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(moe.silu(v), v * scipy.special.expit(v), rtol=1e-14, atol=1e-300)
    assert moe.silu(np.array([0.0]))[0] == 0.0
    y1 = np.array([[0.0, 2.0]])            # G = 0, U = 2 -> H = 0, dG = dh*U/2
    assert moe.silu_gate_fwd(y1)[0, 0] == 0.0
    np.testing.assert_allclose(moe.silu_gate_bwd(y1, np.array([[3.0]])), [[3.0, 0.0]])


def test_silu_gate_bwd_finite_difference():
    rng = np.random.default_rng(8)
    R, F = 6, 5
    y1 = rng.standard_normal((R, 2 * F)) * 3
    dh = rng.standard_normal((R, F))
    g = moe.silu_gate_bwd(y1, dh)
    eps = 1e-6
    num = np.zeros_like(y1)
    for i in range(R):
        for j in range(2 * F):
            p = y1.copy(); p[i, j] += eps
            m = y1.copy(); m[i, j] -= eps
            num[i, j] = ((moe.silu_gate_fwd(p) - moe.silu_gate_fwd(m)) * dh).sum() / (2 * eps)
    np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        np.array([0.0, -0.0, 1e-40, -3e38, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = layer.bf16_round(x)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
