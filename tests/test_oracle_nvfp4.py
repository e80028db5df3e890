"""Pins for the oracle's NVFP4 codecs and quantizer (CPU only).

What pins what:
* hand-worked blocks (tests/golden/quant_blocks.txt) -> the full Q1..Q7 chain;
* brute-force nearest-value search over the 8 E2M1 / 127 E4M3 values, ties to
  the even code, on every rounding threshold +-ulps -> both codecs;
* torch's float8_e4m3fn conversion (a library routine, RNE) -> E4M3;
* invariants (max element -> |code| 7, error bound, sign symmetry, block
  locality, power-of-two equivariance, per-group split).
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import nvfp4


# ---------------------------------------------------------------- golden blocks
def _load_blocks():
    out = []
    with open(os.path.join(GOLDEN, "quant_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, amax, xs, ss, qs = [p.strip() for p in line.split(";")]
            vals = []
            for tok in xs.split(","):
                tok = tok.strip()
                vals.append(float.fromhex(tok) if tok.lower().startswith(("0x", "-0x")) else float(tok))
            out.append(dict(
                name=name,
                amax=None if amax == "-" else float(amax),
                x=np.array(vals, dtype=np.float32)[None, :],
                scales=bytes.fromhex(ss.replace(" ", "")),
                q=bytes.fromhex(qs.replace(" ", "")),
            ))
    return out


BLOCKS = _load_blocks()


@pytest.mark.parametrize("blk", BLOCKS, ids=[b["name"] for b in BLOCKS])
def test_golden_block(blk):
    amax = None if blk["amax"] is None else [blk["amax"]]
    q, s, g, a = nvfp4.quantize(blk["x"], amax=amax)
    assert s.tobytes() == blk["scales"], s.tobytes().hex()
    assert q.tobytes() == blk["q"], q.tobytes().hex()


def test_golden_block_count():
    assert len(BLOCKS) >= 9


# ------------------------------------------------------------ brute-force codecs
def _brute_e2m1(r):
    """Nearest of the 8 magnitudes; a tie goes to the even code; +inf -> 6."""
    grid = [Fraction(g) for g in (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)]
    out = []
    for v in np.asarray(r, dtype=np.float64):
        if np.isinf(v):
            out.append(7)
            continue
        dist = [abs(Fraction(float(v)) - gv) for gv in grid]  # exact
        best = min(dist)
        cands = [c for c, dv in enumerate(dist) if dv == best]
        out.append(cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0])
    return np.array(out, dtype=np.uint8)


def _e4m3_values():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _brute_e4m3(u):
    grid = [Fraction(float(g)) for g in _e4m3_values()]
    out = []
    for v in np.asarray(u, dtype=np.float64):
        if np.isinf(v):
            out.append(0x7E)
            continue
        fv = Fraction(float(v))
        dist = np.array([abs(fv - gv) for gv in grid], dtype=object)  # exact
        best = min(dist)
        cands = np.array([i for i, dv in enumerate(dist) if dv == best])
        out.append(int(cands[0]) if cands.size == 1 else int([c for c in cands if c % 2 == 0][0]))
    return np.array(out, dtype=np.uint8)


def _around(points, n_ulp=3):
    vals = []
    for p in points:
        p = np.float32(p)
        lo = hi = p
        vals.append(p)
        for _ in range(n_ulp):
            lo = np.nextafter(lo, np.float32(-np.inf))
            hi = np.nextafter(hi, np.float32(np.inf))
            vals += [lo, hi]
    v = np.array(vals, dtype=np.float32)
    return v[v >= 0]


def test_e2m1_thresholds_brute_force():
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    mids = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])]
    specials = [0.0, 1e-45, 1.17549435e-38, 6.0, 7.0, 8.0, 100.0, 3.4e38]
    r = np.concatenate([_around(grid + mids + specials), np.array([np.inf], np.float32)])
    np.testing.assert_array_equal(nvfp4.e2m1_encode_mag(r), _brute_e2m1(r))


def test_e2m1_random_brute_force():
    rng = np.random.default_rng(1)
    r = np.exp2(rng.uniform(-12, 5, 20000)).astype(np.float32)
    np.testing.assert_array_equal(nvfp4.e2m1_encode_mag(r), _brute_e2m1(r))


def test_e4m3_thresholds_brute_force():
    grid = _e4m3_values()
    mids = (grid[:-1] + grid[1:]) / 2
    specials = [0.0, 1e-45, 2.0 ** -10, 2.0 ** -9, 448, 464, 465, 480, 1e6, 3.4e38]
    u = np.concatenate([_around(np.concatenate([grid, mids, specials]), 2),
                        np.array([np.inf], np.float32)])
    np.testing.assert_array_equal(nvfp4.e4m3_encode(u), _brute_e4m3(u))


def test_e4m3_matches_torch_rne():
    rng = np.random.default_rng(2)
    grid = _e4m3_values()
    mids = (grid[:-1] + grid[1:]) / 2
    u = np.concatenate([_around(np.concatenate([grid, mids]), 2),
                        np.exp2(rng.uniform(-14, np.log2(464), 50000)).astype(np.float32)])
    u = u[u <= 464]
    ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(nvfp4.e4m3_encode(u), ref)


def test_e4m3_decode_matches_torch():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(nvfp4.e4m3_decode(codes), ref)


def test_e2m1_decode_values():
    # Sign-magnitude with the magnitude list of the format.
    assert list(nvfp4.e2m1_decode(np.arange(8))) == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert list(nvfp4.e2m1_decode(np.arange(8, 16))) == [-0.0, -.5, -1, -1.5, -2, -3, -4, -6]


# ------------------------------------------------------------------ invariants
def _rand(shape, seed=0, outliers=0.01):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    m = rng.random(shape) < outliers
    x[m] *= 20
    return x


def test_global_scale_convention():
    q, s, g, a = nvfp4.quantize(_rand((4, 64)))
    assert g[0] == np.float32(a[0]) / np.float32(2688)
    _, _, g0, _ = nvfp4.quantize(np.zeros((2, 32), np.float32))
    assert g0[0] == 1.0


def test_block_max_maps_to_largest_code():
    x = _rand((64, 256), seed=3)
    q, s, g, _ = nvfp4.quantize(x)
    codes = nvfp4.unpack_codes(q).reshape(64, 16, 16)
    blocks = np.abs(x).reshape(64, 16, 16)
    arg = blocks.argmax(axis=2)
    top = np.take_along_axis(codes, arg[..., None], axis=2)[..., 0] & 7
    normal = nvfp4.e4m3_decode(s) >= 2.0 ** -6
    assert normal.all()
    assert (top[normal] == 7).all()


def test_dequant_error_bound():
    x = _rand((32, 512), seed=4)
    q, s, g, _ = nvfp4.quantize(x)
    xh = nvfp4.dequantize(q, s, g)
    d = np.repeat(nvfp4.e4m3_decode(s).astype(np.float64) * float(g[0]), 16, axis=1)
    r = np.abs(x) / d
    # E2M1 spacing at r: 0.5 below 2, then 1 in [2,4), 2 in [4,6].
    spacing = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    unsat = r <= 6
    err = np.abs(x.astype(np.float64) - xh)
    bound = (spacing / 2 + 2.0 ** -20 * r) * d
    assert (err[unsat] <= bound[unsat]).all()
    # saturated elements land on +-6*d
    assert np.allclose(np.abs(xh[~unsat]), 6 * d[~unsat])


def test_sign_symmetry():
    x = _rand((16, 128), seed=5)
    x[x == 0] = 1.0
    q1, s1, _, _ = nvfp4.quantize(x)
    q2, s2, _, _ = nvfp4.quantize(-x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(q1 ^ 0x88, q2)


def test_block_locality():
    x = _rand((8, 128), seed=6)
    amax = [float(np.abs(x).max()) * 2]
    q1, s1, _, _ = nvfp4.quantize(x, amax=amax)
    y = x.copy()
    y[3, 32:48] = np.float32(0.125)
    q2, s2, _, _ = nvfp4.quantize(y, amax=amax)
    diff_s = np.argwhere(s1 != s2)
    diff_q = np.argwhere(q1 != q2)
    assert all(r == 3 and c == 2 for r, c in diff_s)
    assert all(r == 3 and 16 <= c < 24 for r, c in diff_q)


@pytest.mark.parametrize("k", [-8, -3, 5, 9])
def test_power_of_two_equivariance(k):
    # Scaling the tensor by 2^k scales g by 2^k exactly and leaves every code
    # and block scale unchanged (no under/overflow at these sizes).
    x = _rand((16, 256), seed=7)
    q1, s1, g1, _ = nvfp4.quantize(x)
    q2, s2, g2, _ = nvfp4.quantize(np.ldexp(x, k).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)
    assert g2[0] == np.ldexp(g1[0], k)


def test_groups_equal_separate_tensors():
    x = _rand((3 * 40, 64), seed=8)
    q, s, g, a = nvfp4.quantize(x, groups=3)
    for i in range(3):
        qi, si, gi, ai = nvfp4.quantize(x[40 * i:40 * (i + 1)])
        np.testing.assert_array_equal(q[40 * i:40 * (i + 1)], qi)
        np.testing.assert_array_equal(s[40 * i:40 * (i + 1)], si)
        assert g[i] == gi[0] and a[i] == ai[0]


def test_stale_amax_saturates():
    # amax_in far below the true amax: scales saturate at 448 and codes at 7.
    x = _rand((4, 64), seed=9) * 100
    q, s, g, _ = nvfp4.quantize(x, amax=[1.0])
    codes = nvfp4.unpack_codes(q)
    big = np.abs(x) > 6 * 448 * (1.0 / 2688) * 1.01
    assert (s == 0x7E).any()
    assert ((codes[big] & 7) == 7).all()


def test_bad_shapes():
    with pytest.raises(ValueError):
        nvfp4.quantize(np.zeros((2, 24), np.float32))
    with pytest.raises(ValueError):
        nvfp4.quantize(np.zeros((3, 32), np.float32), groups=2)


def test_empty_tensor():
    q, s, g, a = nvfp4.quantize(np.zeros((0, 64), np.float32))
    assert q.shape == (0, 32) and s.shape == (0, 4) and g[0] == 1.0
