"""Oracle: NVFP4 codecs, quantization and dequantization (test infrastructure).

The format (the pages name "native NVFP4, W4A4" in the key-facts list of
"miniTE ускоряет RL в NVFP4 на B300" but never define it) is taken as:

* E2M1 element codes: 1 sign bit, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
  (codes 0..7), rounded to nearest with ties to the even code, saturating at 6.
* one E4M3 (OCP E4M3FN: bias 7, largest finite 448 = 0x7E, 0x7F is NaN and is
  never produced) scale per 16 consecutive elements of a row along K,
  rounded to nearest-even and saturating at 448, subnormals kept;
* one FP32 global decode scale ``g`` per tensor (or per row-group, one group
  per expert weight matrix).

Quantization steps, all in IEEE binary32 with round-to-nearest-even and
correctly rounded division, in this order:

  Q1  A = max|x| over the group (or the amax handed in: "amax reuse", fourth
      paragraph of "miniTE報告、NVFP4強化学習の安定性を検証").
  Q2  g = A / (6*448) if A > 0 else 1.
  Q3  per 16-block: a = max|x|.
  Q4  t = a / 6;  u = t / g (u = 0 when t = 0);  S = E4M3(u);  s = decode(S).
  Q5  d = s * g.
  Q6  per element: magnitude code = E2M1(|x| / d) if d > 0 else 0;
      code = sign bit of x (bit 3) | magnitude.
  Q7  two codes per byte, the even-k element in the low nibble; scale bytes
      row-major, one per block, no swizzle.

Dequantized value: e2m1(code) * s * g, exact in fp64.
"""

import numpy as np

FP4_MAX = 6.0
FP8_MAX = 448.0
BLOCK = 16
GLOBAL_DIV = np.float32(FP4_MAX * FP8_MAX)  # 2688

# E2M1 magnitude grid, index = magnitude code.
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_encode_mag(r):
    """E2M1 magnitude code (0..7) of r >= 0 (float32 array), RNE, saturating.

    Values above 6 saturate to 6 first (6 is on the grid, and every r > 6
    would round to 6 or 8 and then saturate).  Inside a binade [2^e, 2^(e+1))
    the grid spacing is 2^(e-1), never below 0.5 (the subnormal step).
    """
    r = np.asarray(r, dtype=np.float32)
    if np.any(np.isnan(r)) or np.any(r < 0):
        raise ValueError("e2m1_encode_mag expects non-negative, non-NaN input")
    rc = np.minimum(r, np.float32(FP4_MAX)).astype(np.float64)
    _, e = np.frexp(rc)                       # rc = m * 2^e, m in [0.5, 1)
    quantum = np.maximum(np.ldexp(1.0, e - 2), 0.5)   # 2^(floor(log2 rc) - 1)
    v = np.rint(rc / quantum) * quantum       # rint: ties to even multiple
    code = np.searchsorted(E2M1_GRID, v)
    if not np.array_equal(E2M1_GRID[code], v):
        raise AssertionError("E2M1 rounding left the grid")
    return code.astype(np.uint8)


def e2m1_decode(code):
    """Signed fp64 value of 4-bit E2M1 codes (bit 3 = sign)."""
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_GRID[code & 7]
    return np.where(code & 8, -mag, mag)


def e4m3_encode(u):
    """OCP E4M3FN code of u >= 0 (float32, may be +inf): RNE, saturate at 448."""
    u = np.asarray(u, dtype=np.float32)
    if np.any(np.isnan(u)) or np.any(u < 0):
        raise ValueError("e4m3_encode expects non-negative, non-NaN input")
    uc = np.minimum(u, np.float32(FP8_MAX)).astype(np.float64)
    _, e = np.frexp(uc)
    quantum = np.maximum(np.ldexp(1.0, e - 4), 2.0 ** -9)  # 2^(floor(log2)-3)
    v = np.rint(uc / quantum) * quantum
    v = np.minimum(v, FP8_MAX)
    sub = v < 2.0 ** -6
    code = np.zeros(v.shape, dtype=np.int64)
    code[sub] = np.rint(v[sub] * 2.0 ** 9).astype(np.int64)   # k * 2^-9 -> k
    m, ev = np.frexp(v[~sub])                 # v = m * 2^ev, m in [0.5, 1)
    exp_field = (ev - 1) + 7
    mant = np.rint((m * 2.0 - 1.0) * 8.0).astype(np.int64)
    code[~sub] = (exp_field << 3) | mant
    return code.astype(np.uint8)


def e4m3_decode(code):
    """float32 value of E4M3FN codes 0x00..0x7E (exact)."""
    code = np.asarray(code, dtype=np.int64)
    if np.any((code & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN code")
    sign = np.where(code & 0x80, -1.0, 1.0)
    ef = (code >> 3) & 0xF
    mf = code & 7
    val = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7))
    return (sign * val).astype(np.float32)


def global_scale(amax):
    """Q2: decode-side FP32 global scale g = amax / 2688 (1 when amax == 0)."""
    a = np.asarray(amax, dtype=np.float32)
    g = a / GLOBAL_DIV
    return np.where(a > 0, g, np.float32(1.0)).astype(np.float32)


def quantize(x, groups=1, amax=None):
    """Quantize a [rows, K] tensor (float32 values) to NVFP4.

    ``groups`` equal row-groups each get their own global scale (one for an
    activation tensor, one per expert for a stacked [E*N, K] weight).
    ``amax`` (float32 [groups]) replaces Q1 when given ("amax reuse").

    Returns (q uint8 [rows, K/2], scales uint8 [rows, K/16], g float32
    [groups], amax float32 [groups]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    if groups < 1 or rows % groups:
        raise ValueError("rows must split into equal groups")
    rpg = rows // groups
    ax = np.abs(x)
    if amax is None:
        A = ax.reshape(groups, rpg * K).max(axis=1) if rows * K else np.zeros(groups, np.float32)
    else:
        A = np.asarray(amax, dtype=np.float32).reshape(groups)
    A = A.astype(np.float32)
    g = global_scale(A)                                    # Q2
    g_row = np.repeat(g, rpg)[:, None]                     # [rows, 1]

    blocks = ax.reshape(rows, K // BLOCK, BLOCK)
    a_b = blocks.max(axis=2) if K else np.zeros((rows, 0), np.float32)   # Q3
    t = a_b / np.float32(FP4_MAX)                          # Q4
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(t > 0, t / g_row, np.float32(0.0)).astype(np.float32)
    S = e4m3_encode(u)
    s = e4m3_decode(S)
    d = (s * g_row).astype(np.float32)                     # Q5

    d_el = np.repeat(d, BLOCK, axis=1)                     # per element
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d_el > 0, ax / d_el, np.float32(0.0)).astype(np.float32)
    mag = e2m1_encode_mag(r)                               # Q6
    mag = np.where(d_el > 0, mag, 0).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 3
    code = sign | mag
    q = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)   # Q7
    return q, S.astype(np.uint8), g, A


def unpack_codes(q):
    """[rows, K/2] packed bytes -> [rows, K] 4-bit codes (low nibble = even k)."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = q & 0xF
    out[:, 1::2] = q >> 4
    return out


def dequantize(q, scales, g, groups=1):
    """Exact fp64 value of an NVFP4 tensor: e2m1(code) * s * g."""
    codes = unpack_codes(q)
    rows, K = codes.shape
    s = e4m3_decode(scales).astype(np.float64)
    g = np.asarray(g, dtype=np.float32).astype(np.float64).reshape(groups)
    g_row = np.repeat(g, rows // groups)[:, None]
    return e2m1_decode(codes) * np.repeat(s, BLOCK, axis=1) * g_row


def segment_pad_offset(offsets):
    """Column of each expert's segment in the transposed (column-wise)
    layout: 64 * (floor(off_e / 64) + e), so that a segment padded to a
    multiple of 64 never reaches the next one, with no prefix sum over the
    padded counts.  Returns int64 [E]."""
    off = np.asarray(offsets, dtype=np.int64)
    e = np.arange(off.size - 1, dtype=np.int64)
    return 64 * (off[:-1] // 64 + e)


def padded_extent(M_total, E):
    """Length of the transposed layout's rows: 64 * (floor(M_total / 64) + E)."""
    return 64 * (int(M_total) // 64 + int(E))


def quantize_colwise(x, offsets, amax):
    """Column-wise NVFP4 of a row-grouped tensor (the reduction operand of a
    weight-gradient GEMM): within each expert's row segment [off_e,
    off_e+1), 16 consecutive rows of one column form a block, the segment's
    tail block padded with zeros; one global scale from ``amax`` (the
    tensor's amax, reused from its row-wise quantization).

    The gradient tensors of the NVFP4 backward are rounded like every other
    NVFP4 tensor here (the same Q1-Q7, round to nearest even): the pages do
    not say how the gradients are rounded.

    Equivalent, segment by segment, to quantize(X_e^T padded to a multiple
    of 16 columns, amax).  Returns a list of (q_e [N, L_e/2], s_e [N,
    L_e/16]) with L_e = cnt_e rounded up to 16, and g [1].
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    off = np.asarray(offsets, dtype=np.int64)
    N = x.shape[1]
    out = []
    g = None
    for e in range(off.size - 1):
        seg = x[off[e]:off[e + 1]]
        L = -(-seg.shape[0] // BLOCK) * BLOCK
        xt = np.zeros((N, L), np.float32)
        xt[:, :seg.shape[0]] = seg.T
        q, s, g, _ = quantize(xt, amax=[amax])
        out.append((q, s))
    if g is None:
        g = global_scale(np.float32(amax)).reshape(1)
    return out, g
