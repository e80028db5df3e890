"""Oracle: MX (microscaling) formats for the W4A8 variant -- MXFP8 (E4M3)
activations and MXFP4 (E2M1) weights -- and their dequantization (test
infrastructure).

The pages' activation-precision ablation ("miniTE報告、NVFP4強化学習の安定性を
検証", third paragraph) compares W4A16, W4A8 with MXFP8 activations, and W4A4.
They do not define MXFP8, nor say which 4-bit weight format goes with it.
The readings taken here:

* MX is the published microscaling format: blocks of 32 consecutive
  elements along K share one E8M0 scale (a bare biased exponent, bias 127,
  value 2^(code - 127); code 0xFF is NaN and is never produced).
* The 4-bit weights of W4A8 are MXFP4 (E2M1 elements, E8M0 per 32), so that
  both operands carry power-of-two scales per 32 elements -- the pairing
  whose products the gfx950 scaled MFMA computes exactly.
* The shared scale of a block with amax a > 0 is
      X = 2^(floor(log2 a) - emax),
  emax the exponent of the element format's largest normal value
  (E4M3: 448 = 1.75 * 2^8, emax = 8; E2M1: 6 = 1.5 * 2^2, emax = 2),
  with floor(log2 a) - emax clamped to [-127, 127].  A block whose amax is
  0 gets the smallest scale, code 0 (2^-127).
* Elements: V / X (exact: a power-of-two scaling) rounded to nearest, ties
  to even, and saturated to the format's largest finite magnitude (448 for
  E4M3, 6 for E2M1) -- the published rule clips the top binade, since
  a / X can reach 2^(emax+1).  The sign bit is the sign of V (-0 and
  negatives that round to 0 keep it), as for NVFP4.
* Layout: MXFP8 codes one byte per element [rows][K]; MXFP4 codes two per
  byte [rows][K/2], the even-k element in the low nibble; scales [rows][K/32]
  row-major, unswizzled.

There is no global (per-tensor) scale: the E8M0 range covers every finite
fp32 value, so no amax reduction is needed.
"""

import numpy as np

from . import nvfp4

MX_BLOCK = 32
E8M0_BIAS = 127
ELEM = {
    # name: (emax, largest finite magnitude, bits)
    "e4m3": (8, 448.0, 8),
    "e2m1": (2, 6.0, 4),
}


def e8m0_decode(code):
    """fp64 value 2^(code - 127) of E8M0 scale codes 0..254."""
    code = np.asarray(code, dtype=np.int64)
    if np.any(code == 0xFF):
        raise ValueError("E8M0 NaN code")
    return np.ldexp(1.0, code - E8M0_BIAS)


def shared_exponent(amax, elem):
    """Unbiased shared exponent floor(log2 amax) - emax, clamped to
    [-127, 127]; -127 for amax == 0.  amax: float32 array, >= 0, finite."""
    a = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("amax must be finite and >= 0")
    emax = ELEM[elem][0]
    _, e = np.frexp(a)                  # a = m * 2^e, m in [0.5, 1): floor(log2 a) = e - 1
    se = np.where(a > 0, (e - 1) - emax, -E8M0_BIAS)
    return np.clip(se, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def _encode_mag(r, elem):
    """Magnitude code of r >= 0 (fp64, exact scaled values): RNE, saturating."""
    r32 = np.asarray(r, dtype=np.float64)
    if elem == "e2m1":
        return nvfp4.e2m1_encode_mag(np.minimum(r32, 6.0).astype(np.float32)).astype(np.int64)
    # E4M3: nvfp4.e4m3_encode rounds float32 input; r may not be an fp32
    # value when the scaled element is below fp32's range, so saturate and
    # flush far-below-subnormal values first (they round to 0 either way).
    r32 = np.where(r32 < 2.0 ** -12, 0.0, np.minimum(r32, 448.0))
    return nvfp4.e4m3_encode(r32.astype(np.float32)).astype(np.int64)


def quantize(x, elem):
    """Quantize a [rows, K] tensor (float values, K % 32 == 0) to MX.

    Returns (q uint8, scales uint8 [rows, K/32]); q is [rows, K] for e4m3,
    [rows, K/2] for e2m1 (packed, low nibble = even k).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    ax = np.abs(x).astype(np.float64)
    amax = ax.reshape(rows, K // MX_BLOCK, MX_BLOCK).max(axis=2) if K else np.zeros((rows, 0))
    se = shared_exponent(amax, elem)                       # [rows, K/32]
    scales = (se + E8M0_BIAS).astype(np.uint8)
    r = ax * np.ldexp(1.0, -np.repeat(se, MX_BLOCK, axis=1))   # V / X, exact in fp64
    mag = _encode_mag(r, elem)
    bits = ELEM[elem][2]
    sign = np.signbit(x).astype(np.int64) << (bits - 1)
    code = (sign | mag).astype(np.uint8)
    if elem == "e2m1":
        code = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return code, scales


def decode_elements(q, elem, K):
    """Signed fp64 element values (before the block scale) of packed codes."""
    q = np.asarray(q, dtype=np.uint8)
    if elem == "e2m1":
        return nvfp4.e2m1_decode(nvfp4.unpack_codes(q))[:, :K]
    mag = nvfp4.e4m3_decode(q & 0x7F).astype(np.float64)
    return np.where(q & 0x80, -mag, mag)


def dequantize(q, scales, elem):
    """Exact fp64 value of an MX tensor: element * 2^(scale - 127)."""
    scales = np.asarray(scales, dtype=np.uint8)
    K = scales.shape[1] * MX_BLOCK
    v = decode_elements(q, elem, K)
    return v * np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)
