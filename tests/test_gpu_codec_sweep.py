"""Exhaustive fp32 sweeps of the GPU NVFP4 codecs against the oracle.

Both codecs are monotone step functions of one fp32 input:

* the element code of x >= 0 inside a block whose scale is fixed
  (magnitude code = E2M1 of fl32(|x| / d), d = fl32(s * g)), and
* the E4M3 scale byte of a block as a function of its max |x| (S = E4M3 of
  fl32(fl32(a / 6) / g)).

So the GPU encodes every fp32 value of the range that matters, in bit order,
and the test compares only where the code changes -- with the levels it
changes to -- against the change points of the oracle, found by binary
search over fp32 bit patterns on the oracle's own `quantize` of single
blocks.  A GPU code that differs from the oracle at any input shows up as a
missing, extra or misplaced step.  Element sweeps run at 32 block scales
(4 global amax values x 8 E4M3 scale codes, subnormal and saturating ones
included) and again with every value negated (the sign bit, also of -0);
scale sweeps at 3 global scales, up to past the 448 saturation.
"""

import numpy as np
import pytest
import torch

from _helpers import gpu, require_gpu
from oracle import nvfp4

pytestmark = gpu

AMAX = [2688.0, 1.0, 37500.0, 0.007]
SCALE_CODES = [0x01, 0x03, 0x08, 0x2C, 0x38, 0x3B, 0x55, 0x7E]


def _bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def _f32(b):
    return np.array([b], np.uint32).view(np.float32)[0]


def _oracle_block(vals, amax):
    blk = np.zeros((1, 16), np.float32)
    blk[0, :len(vals)] = vals
    q, s, g, _ = nvfp4.quantize(blk, amax=[amax])
    return nvfp4.unpack_codes(q)[0], int(s[0, 0]), g[0]


def _first_at_least(fn, level, lo, hi):
    """Smallest bit pattern b in [lo, hi] with fn(b) >= level (fn monotone),
    or None."""
    if fn(hi) < level:
        return None
    while lo < hi:
        mid = (lo + hi) // 2
        if fn(mid) >= level:
            hi = mid
        else:
            lo = mid + 1
    return lo


def _steps(codes):
    """Change points of a 1-D code sequence: (positions, new levels)."""
    idx = torch.nonzero(codes[1:] != codes[:-1]).flatten() + 1
    return idx.cpu().numpy().astype(np.int64), codes[idx].cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("amax", AMAX)
def test_element_codec_every_fp32_value(amax):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    dev = torch.device("cuda:0")
    g = nvfp4.global_scale(np.float32(amax))
    amax_t = torch.tensor([amax], dtype=torch.float32, device=dev)
    for code in SCALE_CODES:
        # a block maximum that gives (about) this scale code; the oracle says
        # which code and block scale it actually gives
        pilot = np.float32(np.float32(6.0) * np.float32(nvfp4.e4m3_decode(code) * g))
        _, S, _ = _oracle_block([pilot], amax)
        n = _bits(pilot) + 1                      # every fp32 in [0, pilot]
        blocks = -(-n // 15)
        flat = torch.zeros(blocks * 15, dtype=torch.float32, device=dev)
        flat[:n] = torch.arange(n, dtype=torch.int32, device=dev).view(torch.float32)
        x = torch.empty((blocks, 16), dtype=torch.float32, device=dev)
        x[:, 0] = float(pilot)
        x[:, 1:] = flat.view(blocks, 15)
        del flat
        q, s, gs, _ = ops.nvfp4_quantize(x, amax_in=amax_t)
        assert bool((s == S).all()), (amax, code)
        assert gs.cpu().numpy().view(np.uint32)[0] == np.float32(g).view(np.uint32)
        codes = torch.stack([q & 15, q >> 4], dim=-1).view(blocks, 16)[:, 1:].reshape(-1)
        mag = codes[:n]
        assert int(mag.max()) <= 7 and int(mag[0]) == 0
        pos, lev = _steps(mag)

        def oracle_code(b):
            return int(_oracle_block([pilot, _f32(b)], amax)[0][1] & 7)

        want_pos, want_lev = [], []
        for level in range(1, 8):
            b = _first_at_least(oracle_code, level, 0, n - 1)
            if b is not None and (not want_pos or b != want_pos[-1]):
                want_pos.append(b)
                want_lev.append(oracle_code(b))
            elif b is not None:
                want_lev[-1] = oracle_code(b)
        np.testing.assert_array_equal(pos, want_pos, err_msg="amax %r scale code %#x" % (amax, code))
        np.testing.assert_array_equal(lev, want_lev, err_msg="amax %r scale code %#x" % (amax, code))
        # the same values negated: the sign bit, magnitudes unchanged (-0 too)
        x[:, 1:] = -x[:, 1:]
        q2, s2, _, _ = ops.nvfp4_quantize(x, amax_in=amax_t)
        codes2 = torch.stack([q2 & 15, q2 >> 4], dim=-1).view(blocks, 16)[:, 1:].reshape(-1)
        assert bool((s2 == S).all())
        assert torch.equal(codes2, codes | 8), (amax, code)
        del x, q, q2, codes, codes2, mag
        torch.cuda.synchronize()


@pytest.mark.parametrize("amax", AMAX[:3])
def test_scale_codec_every_fp32_block_max(amax):
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    dev = torch.device("cuda:0")
    g = nvfp4.global_scale(np.float32(amax))
    amax_t = torch.tensor([amax], dtype=torch.float32, device=dev)
    hi = np.float32(np.float32(6.0 * 464.0) * g)    # past the saturation to 448
    n = _bits(hi) + 1
    chunk = 1 << 26
    pos, lev, prev = [], [], None
    for c0 in range(0, n, chunk):
        m = min(chunk, n - c0)
        x = torch.zeros((m, 16), dtype=torch.float32, device=dev)
        x[:, 0] = torch.arange(c0, c0 + m, dtype=torch.int32, device=dev).view(torch.float32)
        _, s, _, _ = ops.nvfp4_quantize(x, amax_in=amax_t)
        s = s.view(-1).to(torch.int64)
        if prev is None:
            assert int(s[0]) == 0                  # an all-zero block
        else:
            s = torch.cat([prev, s])
        p, l = _steps(s)
        off = c0 - (0 if prev is None else 1)
        pos += list(p + off)
        lev += list(l)
        prev = s[-1:].clone()
        del x, s
    torch.cuda.synchronize()

    def oracle_scale(b):
        return _oracle_block([_f32(b)], amax)[1]

    want_pos, want_lev = [], []
    for level in range(1, 0x7F):
        b = _first_at_least(oracle_scale, level, 0, n - 1)
        if b is None:
            continue
        if want_pos and b == want_pos[-1]:
            want_lev[-1] = oracle_scale(b)
        else:
            want_pos.append(b)
            want_lev.append(oracle_scale(b))
    assert want_lev[-1] == 0x7E
    np.testing.assert_array_equal(pos, want_pos, err_msg="amax %r" % amax)
    np.testing.assert_array_equal(lev, want_lev, err_msg="amax %r" % amax)
