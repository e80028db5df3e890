"""Pins for the oracle's MX formats (MXFP8 E4M3 / MXFP4 E2M1 elements with
E8M0 scales per 32) and the W4A8 grouped GEMM (CPU only).

* hand-worked blocks (tests/golden/mx_blocks.txt): zero block, the top-
  binade clip, subnormal elements, ties, the clamped smallest scale;
* the shared exponent against an integer search for the binade of the
  block's amax;
* every element against a brute-force nearest search over the format's
  values (exact fractions) with ties to the even code;
* E4M3 elements against torch's float8_e4m3fn conversion (RNE) where it
  does not saturate differently;
* power-of-two equivariance, block locality, the rounding error bound;
* the grouped W4A8 GEMM against pure-Python triple loops.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import gemm, mx


def _parse(v):
    if "p" in v:
        m, e = v.split("p")
        return float(m) * 2.0 ** int(e)
    return float(v)


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
            cur["in"] = [_parse(v) for v in rest]
        elif k == "scale":
            cur["scale"] = int(rest[0], 16)
        elif k == "codes":
            cur["codes"] = [int(v, 16) for v in rest]
    return blocks


def _unpack4(q):
    c = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    c[:, 0::2] = q & 15
    c[:, 1::2] = q >> 4
    return c


@pytest.mark.parametrize("blk", _golden(), ids=lambda b: b["name"])
def test_golden_blocks(blk):
    x = np.zeros((1, 32), np.float32)
    x[0, :len(blk["in"])] = blk["in"]
    q, s = mx.quantize(x, blk["elem"])
    codes = _unpack4(q)[0] if blk["elem"] == "e2m1" else q[0]
    want = np.zeros(32, np.uint8)
    want[:len(blk["codes"])] = blk["codes"]
    assert s[0, 0] == blk["scale"]
    np.testing.assert_array_equal(codes, want)


# exact value tables (Fractions), index = magnitude code
E2M1_VALUES = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]
E4M3_VALUES = [Fraction(m, 2 ** 9) for m in range(8)] + \
    [(1 + Fraction(m, 8)) * Fraction(2) ** (e - 7) for e in range(1, 16) for m in range(8)][:-1]   # drop NaN 0x7F


def _nearest_code(r, table):
    """Brute force: the nearest table value, ties to the even code, values
    beyond the largest saturate."""
    r = Fraction(r)
    if r >= table[-1]:
        return len(table) - 1
    best = min(range(len(table)), key=lambda c: (abs(table[c] - r), c & 1))
    return best


def _binade(a):
    """Integer e with 2^e <= a < 2^(e+1), by comparisons (a > 0)."""
    e = 0
    while math.ldexp(1.0, e) > a:
        e -= 1
    while math.ldexp(1.0, e + 1) <= a:
        e += 1
    return e


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_brute_force_random_blocks(elem):
    rng = np.random.default_rng(5 if elem == "e4m3" else 6)
    rows = 24
    x = (rng.standard_normal((rows, 64)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.05] *= 30
    x[3] = 0.0
    x[4, :32] = 0.0
    x[5, 7] = -0.0
    q, s = mx.quantize(x, elem)
    codes = _unpack4(q) if elem == "e2m1" else q
    emax = mx.ELEM[elem][0]
    table = E4M3_VALUES if elem == "e4m3" else E2M1_VALUES
    sign_bit = 0x80 if elem == "e4m3" else 0x8
    for r in range(rows):
        for b in range(2):
            blk = x[r, 32 * b:32 * b + 32]
            amax = float(np.abs(blk).max())
            se = max(-127, min(127, _binade(amax) - emax)) if amax > 0 else -127
            assert s[r, b] == se + 127
            X = Fraction(2) ** se
            for i, v in enumerate(blk):
                c = int(codes[r, 32 * b + i])
                assert (c & sign_bit != 0) == bool(np.signbit(v))
                assert c & (sign_bit - 1) == _nearest_code(abs(Fraction(float(v))) / X, table), (r, b, i, v)


def test_e4m3_elements_match_torch():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    q, s = mx.quantize(x, "e4m3")
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    r = (x / X).astype(np.float32)
    ok = np.abs(r) <= 448      # torch returns NaN above 464 where the format saturates
    t = torch.from_numpy(np.where(ok, r, 0).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q[ok], t[ok])


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_invariants(elem):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((16, 96)).astype(np.float32)
    q, s = mx.quantize(x, elem)
    # power-of-two equivariance: the codes stay, the scales move
    for j in (-9, 5):
        q2, s2 = mx.quantize(np.ldexp(x, j).astype(np.float32), elem)
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2.astype(int), s.astype(int) + j)
    # block locality: changing block 1 of a row leaves blocks 0 and 2
    y = x.copy()
    y[:, 32:64] *= 1000
    qy, sy = mx.quantize(y, elem)
    cols = slice(0, 16) if elem == "e2m1" else slice(0, 32)
    np.testing.assert_array_equal(qy[:, cols], q[:, cols])
    np.testing.assert_array_equal(sy[:, [0, 2]], s[:, [0, 2]])
    # error bound: half a step of the element's binade, unless clipped
    xd = mx.dequantize(q, s, elem)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    r = np.abs(x) / X
    top = mx.ELEM[elem][1]
    mbits = 3 if elem == "e4m3" else 1
    emin = -6 if elem == "e4m3" else 0
    _, e = np.frexp(np.maximum(r, 1e-300))
    step = np.ldexp(1.0, np.maximum(e - 1, emin) - mbits)
    unclipped = r <= top
    assert (np.abs(x - xd)[unclipped] <= 0.5 * (step * X)[unclipped] * (1 + 1e-12)).all()
    assert (np.abs(xd)[~unclipped] == (top * X)[~unclipped]).all()
    # the block's largest element lies in the format's top binade (or clips)
    bm = np.abs(xd).reshape(16, 3, 32).max(axis=2)
    Xb = np.ldexp(1.0, s.astype(np.int64) - 127)
    assert ((bm / Xb) >= 2.0 ** mx.ELEM[elem][0]).all()


@pytest.mark.parametrize("M,N,K,offs", [(3, 5, 64, [0, 2, 2, 3]), (4, 3, 32, [0, 0, 4])])
def test_w4a8_gemm_brute_force(M, N, K, offs):
    rng = np.random.default_rng(M + 10 * K)
    E = len(offs) - 1
    aq, as_ = mx.quantize(rng.standard_normal((M, K)).astype(np.float32) * 3, "e4m3")
    bq, bs = mx.quantize((rng.standard_normal((E * N, K)) * 0.05).astype(np.float32), "e2m1")
    bq, bs = bq.reshape(E, N, K // 2), bs.reshape(E, N, K // 32)
    C, AB = gemm.grouped_gemm_w4a8(aq, as_, bq, bs, offs)
    # brute force from exact element values and scales, pure Python
    A = [[Fraction(float(v)) for v in row] for row in mx.dequantize(aq, as_, "e4m3")]
    for e in range(E):
        B = mx.dequantize(bq[e], bs[e], "e2m1")
        for r in range(offs[e], offs[e + 1]):
            for n in range(N):
                ref = sum(A[r][kk] * Fraction(float(B[n, kk])) for kk in range(K))
                assert abs(C[r, n] - float(ref)) <= 1e-12 * max(1.0, abs(float(ref)))
    assert (np.abs(C) <= AB * (1 + 1e-12)).all()
    np.testing.assert_array_equal(C[offs[-1]:], 0)
