"""Thin Python binding of the nvfp4moe C ABI.

Same names as the C entry points.  torch supplies device memory (outputs are
allocated here with torch.empty) and the current HIP stream; every step of
the computation runs in the library's HIP kernels.  Argument marshalling
only: no arithmetic happens in Python.
"""

import torch

from . import _lib

F32, BF16, U8 = _lib.F32, _lib.BF16, _lib.U8
NT, NN, TN = _lib.NT, _lib.NN, _lib.TN

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: U8}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16, U8: torch.uint8}


class NVFP4MoEError(RuntimeError):
    def __init__(self, fn, rc):
        super().__init__("%s failed: %s (%d)" % (fn, _lib.status_string(rc), rc))
        self.rc = rc


def _check(fn, rc):
    if rc != _lib.OK:
        raise NVFP4MoEError(fn, rc)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("nvfp4moe ops take GPU tensors")
            if not t.is_contiguous():
                raise ValueError("nvfp4moe ops take contiguous tensors")


def nvfp4_quantize(x, groups=1, amax_in=None, amax_out=None, q=None, scales=None, gscale=None):
    """NVFP4-quantize a [rows, K] fp32/bf16 tensor.  Returns (q, scales,
    gscale, amax) where amax is amax_in when given, else the computed one."""
    _dev(x, amax_in, amax_out, q, scales, gscale)
    rows, K = x.shape
    dev = x.device
    q = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    gscale = torch.empty((groups,), dtype=torch.float32, device=dev) if gscale is None else gscale
    if amax_in is None and amax_out is None:
        amax_out = torch.empty((groups,), dtype=torch.float32, device=dev)
    lib = _lib.load()
    rc = lib.nvfp4_quantize(_ptr(x), _DT[x.dtype], rows, K, groups, _ptr(amax_in), _ptr(amax_out),
                            _ptr(q), _ptr(scales), _ptr(gscale), None, _stream())
    _check("nvfp4_quantize", rc)
    return q, scales, gscale, (amax_in if amax_in is not None else amax_out)



def nvfp4_quantize_onepass(x, groups=1, amax_out=None, q=None, scales=None, gscale=None, workspace=None):
    """nvfp4_quantize with the amax of each group computed, x read once
    (same outputs).  Returns (q, scales, gscale, amax)."""
    _dev(x, amax_out, q, scales, gscale, workspace)
    rows, K = x.shape
    dev = x.device
    q = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    gscale = torch.empty((groups,), dtype=torch.float32, device=dev) if gscale is None else gscale
    amax_out = torch.empty((groups,), dtype=torch.float32, device=dev) if amax_out is None else amax_out
    lib = _lib.load()
    ws_bytes = lib.nvfp4_quantize_onepass_workspace_size(rows, K, groups)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    rc = lib.nvfp4_quantize_onepass(_ptr(x), _DT[x.dtype], rows, K, groups, _ptr(amax_out), _ptr(q), _ptr(scales),
                                    _ptr(gscale), _ptr(workspace), workspace.numel(), _stream())
    _check("nvfp4_quantize_onepass", rc)
    return q, scales, gscale, amax_out

def moe_permute_workspace_size(T, k, E):
    return _lib.load().moe_permute_workspace_size(T, k, E)


def moe_permute(topk_ids, num_experts, x=None, x_perm=None, amax_out=None, want_amax=False, status=None,
                workspace=None):
    """Routing metadata (offsets, dest, src) and the optional gather of x
    rows into the contiguous per-expert layout.  Returns a dict."""
    _dev(topk_ids, x, x_perm, amax_out, status)
    T, k = topk_ids.shape
    dev = topk_ids.device
    R = T * k
    offsets = torch.empty((num_experts + 1,), dtype=torch.int32, device=dev)
    dest = torch.empty((R,), dtype=torch.int32, device=dev)
    src = torch.empty((R,), dtype=torch.int32, device=dev)
    lib = _lib.load()
    ws_bytes = lib.moe_permute_workspace_size(T, k, num_experts)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    row_elems = 0
    x_dtype = BF16
    if x is not None:
        row_elems = x.shape[1] if x.dim() == 2 else x[0].numel()
        x_dtype = _DT[x.dtype]
        if x_perm is None:
            x_perm = torch.empty((R,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
        if want_amax and amax_out is None:
            amax_out = torch.empty((1,), dtype=torch.float32, device=dev)
    rc = lib.moe_permute(_ptr(topk_ids), T, k, num_experts, _ptr(x), x_dtype, row_elems, _ptr(x_perm),
                         _ptr(offsets), _ptr(dest), _ptr(src), _ptr(amax_out), _ptr(workspace),
                         workspace.numel(), _ptr(status), _stream())
    _check("moe_permute", rc)
    return dict(offsets=offsets, dest=dest, src=src, x_perm=x_perm, amax=amax_out)



def moe_permute_mx(topk_ids, num_experts, x, q=None, scales=None, status=None, workspace=None):
    """moe_permute fused with the MXFP8 (E4M3) quantization of the permuted
    rows: codes [T*k, D] and E8M0 scales [T*k, D/32].  Returns a dict with
    offsets, dest, src, q and scales."""
    _dev(topk_ids, x, q, scales, status, workspace)
    T, k = topk_ids.shape
    D = x.shape[1]
    dev = x.device
    R = T * k
    lib = _lib.load()
    offsets = torch.empty((num_experts + 1,), dtype=torch.int32, device=dev)
    dest = torch.empty((R,), dtype=torch.int32, device=dev)
    src = torch.empty((R,), dtype=torch.int32, device=dev)
    q = torch.empty((R, D), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((R, D // 32), dtype=torch.uint8, device=dev) if scales is None else scales
    ws_bytes = lib.moe_permute_workspace_size(T, k, num_experts)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    rc = lib.moe_permute_mx(_ptr(topk_ids), T, k, num_experts, _ptr(x), _DT[x.dtype], D, _ptr(q), _ptr(scales),
                            _ptr(offsets), _ptr(dest), _ptr(src), _ptr(workspace), workspace.numel(), _ptr(status),
                            _stream())
    _check("moe_permute_mx", rc)
    return dict(offsets=offsets, dest=dest, src=src, q=q, scales=scales)

def moe_permute_nvfp4(topk_ids, num_experts, x, x_perm=None, want_x_perm=True, amax_in=None, amax_out=None,
                      q=None, scales=None, gscale=None, status=None, workspace=None):
    """moe_permute fused with the NVFP4 quantization of the gathered rows.
    Returns a dict with offsets, dest, src, x_perm (or None), q, scales,
    gscale and amax."""
    _dev(topk_ids, x, x_perm, amax_in, amax_out, q, scales, gscale, status)
    T, k = topk_ids.shape
    D = x.shape[1]
    dev = x.device
    R = T * k
    lib = _lib.load()
    offsets = torch.empty((num_experts + 1,), dtype=torch.int32, device=dev)
    dest = torch.empty((R,), dtype=torch.int32, device=dev)
    src = torch.empty((R,), dtype=torch.int32, device=dev)
    if x_perm is None and want_x_perm:
        x_perm = torch.empty((R, D), dtype=x.dtype, device=dev)
    q = torch.empty((R, D // 2), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((R, D // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    gscale = torch.empty((1,), dtype=torch.float32, device=dev) if gscale is None else gscale
    if amax_in is None and amax_out is None:
        amax_out = torch.empty((1,), dtype=torch.float32, device=dev)
    ws_bytes = lib.moe_permute_workspace_size(T, k, num_experts)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    if x.dtype != torch.bfloat16:
        raise ValueError("moe_permute_nvfp4 takes bf16 activations")
    rc = lib.moe_permute_nvfp4(_ptr(topk_ids), T, k, num_experts, _ptr(x), D, _ptr(x_perm), _ptr(amax_in),
                               _ptr(amax_out), _ptr(q), _ptr(scales), _ptr(gscale), _ptr(offsets), _ptr(dest),
                               _ptr(src), _ptr(workspace), workspace.numel(), _ptr(status), _stream())
    _check("moe_permute_nvfp4", rc)
    return dict(offsets=offsets, dest=dest, src=src, x_perm=x_perm, q=q, scales=scales, gscale=gscale,
                amax=amax_in if amax_in is not None else amax_out)


def moe_permute_nvfp4_noalloc(topk_ids, num_experts, x, x_perm=None, want_x_perm=True, amax_in=None,
                              amax_out=None, q=None, scales=None, gscale=None, status=None):
    """moe_permute_nvfp4 without a workspace: the library's own per-GPU
    scratch array holds the histograms (for callers that cannot allocate;
    every output buffer passed in is written, nothing else is allocated by
    the library).  Calls on one GPU must not overlap in time."""
    _dev(topk_ids, x, x_perm, amax_in, amax_out, q, scales, gscale, status)
    T, k = topk_ids.shape
    D = x.shape[1]
    dev = x.device
    R = T * k
    offsets = torch.empty((num_experts + 1,), dtype=torch.int32, device=dev)
    dest = torch.empty((R,), dtype=torch.int32, device=dev)
    src = torch.empty((R,), dtype=torch.int32, device=dev)
    if x_perm is None and want_x_perm:
        x_perm = torch.empty((R, D), dtype=x.dtype, device=dev)
    q = torch.empty((R, D // 2), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((R, D // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    gscale = torch.empty((1,), dtype=torch.float32, device=dev) if gscale is None else gscale
    if amax_in is None and amax_out is None:
        amax_out = torch.empty((1,), dtype=torch.float32, device=dev)
    if x.dtype != torch.bfloat16:
        raise ValueError("moe_permute_nvfp4_noalloc takes bf16 activations")
    rc = _lib.load().moe_permute_nvfp4_noalloc(_ptr(topk_ids), T, k, num_experts, _ptr(x), D, _ptr(x_perm),
                                               _ptr(amax_in), _ptr(amax_out), _ptr(q), _ptr(scales), _ptr(gscale),
                                               _ptr(offsets), _ptr(dest), _ptr(src), _ptr(status), _stream())
    _check("moe_permute_nvfp4_noalloc", rc)
    return dict(offsets=offsets, dest=dest, src=src, x_perm=x_perm, q=q, scales=scales, gscale=gscale,
                amax=amax_in if amax_in is not None else amax_out)


def moe_gather(x, src, k, topk_w=None, out=None, out_dtype=None):
    """out[p] = w[src[p]] * x[src[p] // k] (a verbatim row copy when no weights)."""
    _dev(x, src, topk_w, out)
    R = src.numel()
    row_elems = x.shape[1] if x.dim() == 2 else x[0].numel()
    odt = x.dtype if out_dtype is None else out_dtype
    out = torch.empty((R,) + tuple(x.shape[1:]), dtype=odt, device=x.device) if out is None else out
    rc = _lib.load().moe_gather(_ptr(x), _DT[x.dtype], row_elems, _ptr(src), _ptr(topk_w), k, R, _ptr(out),
                                _DT[out.dtype], _stream())
    _check("moe_gather", rc)
    return out


def moe_scatter(x, dest, offsets, k, topk_w=None, out=None, out_dtype=None, amax_out=None):
    """out[dest[t*k+j]] = w[t*k+j] * x[t]: the weighted gather written from the
    token side (each row of x read once); rows past offsets[E] are zeros.
    amax_out (fp32 [1], optional) receives max |out|."""
    _dev(x, dest, offsets, topk_w, out, amax_out)
    T = x.shape[0]
    R = T * k
    E = offsets.numel() - 1
    row_elems = x.shape[1] if x.dim() == 2 else x[0].numel()
    odt = x.dtype if out_dtype is None else out_dtype
    out = torch.empty((R,) + tuple(x.shape[1:]), dtype=odt, device=x.device) if out is None else out
    rc = _lib.load().moe_scatter(_ptr(x), _DT[x.dtype], row_elems, _ptr(dest), _ptr(topk_w), _ptr(offsets), E, T,
                                 k, _ptr(out), _DT[out.dtype], _ptr(amax_out), _stream())
    _check("moe_scatter", rc)
    return out


def moe_unpermute(y_perm, dest, T, k, topk_w=None, out=None, out_dtype=torch.bfloat16):
    """out[t] = sum_j w[t, j] * y_perm[dest[t*k + j]]."""
    _dev(y_perm, dest, topk_w, out)
    D = y_perm.shape[1]
    out = torch.empty((T, D), dtype=out_dtype, device=y_perm.device) if out is None else out
    rc = _lib.load().moe_unpermute(_ptr(y_perm), _DT[y_perm.dtype], _ptr(dest), _ptr(topk_w), T, k, D, _ptr(out),
                                   _DT[out.dtype], _stream())
    _check("moe_unpermute", rc)
    return out


def grouped_gemm_w4a4(a_q, a_s, a_g, b_q, b_s, b_g, offsets, out=None, out_dtype=torch.float32):
    """C[r] = a_g * b_g[e] * deq(A)[r] . deq(B_e)^T for rows r of expert e."""
    _dev(a_q, a_s, a_g, b_q, b_s, b_g, offsets, out)
    M = a_q.shape[0]
    K = a_q.shape[1] * 2
    E, N = b_q.shape[0], b_q.shape[1]
    out = torch.empty((M, N), dtype=out_dtype, device=a_q.device) if out is None else out
    rc = _lib.load().grouped_gemm_w4a4(_ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q), _ptr(b_s), _ptr(b_g),
                                       _ptr(offsets), E, M, N, K, _ptr(out), _DT[out.dtype], _lib.EPI_NONE,
                                       None, None, 0, _stream())
    _check("grouped_gemm_w4a4", rc)
    return out


def grouped_gemm_w4a4_scaled_mfma(a_q, a_s, a_g, b_q, b_s, b_g, offsets, out=None, out_dtype=torch.float32):
    """grouped_gemm_w4a4 by scale factoring onto the fp4 scaled MFMA (the
    alternative design, for measurement)."""
    _dev(a_q, a_s, a_g, b_q, b_s, b_g, offsets, out)
    M = a_q.shape[0]
    K = a_q.shape[1] * 2
    E, N = b_q.shape[0], b_q.shape[1]
    out = torch.empty((M, N), dtype=out_dtype, device=a_q.device) if out is None else out
    rc = _lib.load().grouped_gemm_w4a4_scaled_mfma(_ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q), _ptr(b_s), _ptr(b_g),
                                                   _ptr(offsets), E, M, N, K, _ptr(out), _DT[out.dtype], _stream())
    _check("grouped_gemm_w4a4_scaled_mfma", rc)
    return out


def grouped_gemm_w4a4_silu_gate(a_q, a_s, a_g, b_q, b_s, b_g, offsets, y1=None, want_y1=True, h=None,
                                amax_out=None, want_amax=True):
    """Gate+up W4A4 GEMM with the SiLU gate (and amax of H) in its epilogue.
    B_e = [gate; up] rows.  Returns (y1 or None, h, amax or None)."""
    _dev(a_q, a_s, a_g, b_q, b_s, b_g, offsets, y1, h, amax_out)
    M = a_q.shape[0]
    K = a_q.shape[1] * 2
    E, N = b_q.shape[0], b_q.shape[1]
    F = N // 2
    dev = a_q.device
    if y1 is None and want_y1:
        y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev) if h is None else h
    if amax_out is None and want_amax:
        amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    rc = _lib.load().grouped_gemm_w4a4_silu_gate(_ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q), _ptr(b_s), _ptr(b_g),
                                                 _ptr(offsets), E, M, F, K, _ptr(y1), _ptr(h), _ptr(amax_out),
                                                 _stream())
    _check("grouped_gemm_w4a4_silu_gate", rc)
    return y1, h, amax_out


def grouped_gemm_w4a4_silu_gate_nvfp4(a_q, a_s, a_g, b_q, b_s, b_g, offsets, amax_h_in, y1=None, h=None,
                                      amax_out=None, want_amax=True, q_h=None, s_h=None, g_h=None):
    """Gate+up W4A4 GEMM with the SiLU gate and the NVFP4 requantization of
    H (with the handed-in amax_h_in) in its epilogue.  Returns (q_h, s_h,
    g_h, amax or None); y1 and h are stored only when given."""
    _dev(a_q, a_s, a_g, b_q, b_s, b_g, offsets, amax_h_in, y1, h, amax_out, q_h, s_h, g_h)
    M = a_q.shape[0]
    K = a_q.shape[1] * 2
    E, N = b_q.shape[0], b_q.shape[1]
    F = N // 2
    dev = a_q.device
    q_h = torch.empty((M, F // 2), dtype=torch.uint8, device=dev) if q_h is None else q_h
    s_h = torch.empty((M, F // 16), dtype=torch.uint8, device=dev) if s_h is None else s_h
    g_h = torch.empty((1,), dtype=torch.float32, device=dev) if g_h is None else g_h
    if amax_out is None and want_amax:
        amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    rc = _lib.load().grouped_gemm_w4a4_silu_gate_nvfp4(
        _ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q), _ptr(b_s), _ptr(b_g), _ptr(offsets), E, M, F, K, _ptr(y1),
        _ptr(h), _ptr(amax_out), _ptr(amax_h_in), _ptr(q_h), _ptr(s_h), _ptr(g_h), _stream())
    _check("grouped_gemm_w4a4_silu_gate_nvfp4", rc)
    return q_h, s_h, g_h, amax_out


def padded_extent(M_total, E):
    """Row length of the column-wise layout: 64 * (M_total // 64 + E)."""
    return 64 * (M_total // 64 + E)


def nvfp4_quantize_colwise(x, offsets, amax_in, Kp=None, q_t=None, s_t=None, gscale=None):
    """Column-wise NVFP4 of a row-grouped [M_total, N] bf16 tensor, stored
    transposed ([N, Kp/2] codes, [N, Kp/16] scales; expert e's segment at
    column 64 * (offsets[e] // 64 + e)).  Returns (q_t, s_t, gscale)."""
    _dev(x, offsets, amax_in, q_t, s_t, gscale)
    M, N = x.shape
    E = offsets.numel() - 1
    Kp = padded_extent(M, E) if Kp is None else Kp
    dev = x.device
    q_t = torch.empty((N, Kp // 2), dtype=torch.uint8, device=dev) if q_t is None else q_t
    s_t = torch.empty((N, Kp // 16), dtype=torch.uint8, device=dev) if s_t is None else s_t
    gscale = torch.empty((1,), dtype=torch.float32, device=dev) if gscale is None else gscale
    rc = _lib.load().nvfp4_quantize_colwise(_ptr(x), _DT[x.dtype], M, N, _ptr(offsets), E, _ptr(amax_in), _ptr(q_t),
                                            _ptr(s_t), _ptr(gscale), Kp, _stream())
    _check("nvfp4_quantize_colwise", rc)
    return q_t, s_t, gscale


def nvfp4_quantize_transposed(x, amax_in=None, amax_out=None, q_t=None, s_t=None, gscale=None):
    """NVFP4 of each matrix of x [G, L, N] along its rows' index: codes of
    the transposed matrices, q_t [G, N, L/2], s_t [G, N, L/16], gscale [G].
    Returns (q_t, s_t, gscale, amax)."""
    _dev(x, amax_in, amax_out, q_t, s_t, gscale)
    G, L, N = x.shape
    dev = x.device
    q_t = torch.empty((G, N, L // 2), dtype=torch.uint8, device=dev) if q_t is None else q_t
    s_t = torch.empty((G, N, L // 16), dtype=torch.uint8, device=dev) if s_t is None else s_t
    gscale = torch.empty((G,), dtype=torch.float32, device=dev) if gscale is None else gscale
    if amax_in is None and amax_out is None:
        amax_out = torch.empty((G,), dtype=torch.float32, device=dev)
    rc = _lib.load().nvfp4_quantize_transposed(_ptr(x), _DT[x.dtype], G, L, N, _ptr(amax_in), _ptr(amax_out),
                                               _ptr(q_t), _ptr(s_t), _ptr(gscale), _stream())
    _check("nvfp4_quantize_transposed", rc)
    return q_t, s_t, gscale, amax_in if amax_in is not None else amax_out


def grouped_gemm_w4a4_wgrad(a, b, offsets, M_total, out=None, out_dtype=torch.float32):
    """NVFP4 weight gradient: C_e = deq(A_e)^T . deq(B_e) over expert e's
    rows, a and b the (q_t, s_t, gscale) of nvfp4_quantize_colwise.
    Returns C [E, N1, N2]."""
    (aq, as_, ag), (bq, bs, bg) = a, b
    _dev(aq, as_, ag, bq, bs, bg, offsets, out)
    E = offsets.numel() - 1
    N1, Kp = aq.shape[0], aq.shape[1] * 2
    N2 = bq.shape[0]
    out = torch.empty((E, N1, N2), dtype=out_dtype, device=aq.device) if out is None else out
    rc = _lib.load().grouped_gemm_w4a4_wgrad(_ptr(aq), _ptr(as_), _ptr(ag), _ptr(bq), _ptr(bs), _ptr(bg),
                                             _ptr(offsets), E, M_total, Kp, N1, N2, _ptr(out), _DT[out.dtype],
                                             _stream())
    _check("grouped_gemm_w4a4_wgrad", rc)
    return out


MX_E4M3, MX_E2M1 = _lib.MX_E4M3, _lib.MX_E2M1


def mx_quantize(x, elem=MX_E4M3, q=None, scales=None):
    """MX-quantize a [rows, K] fp32/bf16 tensor (E8M0 scale per 32 along K):
    elem MX_E4M3 (MXFP8, one byte per element) or MX_E2M1 (MXFP4, packed
    pairs).  Returns (q, scales)."""
    _dev(x, q, scales)
    rows, K = x.shape
    dev = x.device
    qcols = K if elem == MX_E4M3 else K // 2
    q = torch.empty((rows, qcols), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev) if scales is None else scales
    rc = _lib.load().mx_quantize(_ptr(x), _DT[x.dtype], rows, K, elem, _ptr(q), _ptr(scales), _stream())
    _check("mx_quantize", rc)
    return q, scales


def grouped_gemm_w4a8(a_q, a_s, b_q, b_s, offsets, out=None, out_dtype=torch.float32):
    """C[r] = deq(A)[r] . deq(B_e)^T for rows r of expert e; A MXFP8 [M, K],
    B MXFP4 [E, N, K/2], E8M0 scales per 32."""
    _dev(a_q, a_s, b_q, b_s, offsets, out)
    M, K = a_q.shape
    E, N = b_q.shape[0], b_q.shape[1]
    out = torch.empty((M, N), dtype=out_dtype, device=a_q.device) if out is None else out
    rc = _lib.load().grouped_gemm_w4a8(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), E, M, N, K,
                                       _ptr(out), _DT[out.dtype], _stream())
    _check("grouped_gemm_w4a8", rc)
    return out


def grouped_gemm_w4a8_silu_gate(a_q, a_s, b_q, b_s, offsets, y1=None, want_y1=True, h=None, amax_out=None,
                                want_amax=True):
    """Gate+up W4A8 GEMM with the SiLU gate (and amax of H) in its epilogue.
    Returns (y1 or None, h, amax or None)."""
    _dev(a_q, a_s, b_q, b_s, offsets, y1, h, amax_out)
    M, K = a_q.shape
    E, N = b_q.shape[0], b_q.shape[1]
    F = N // 2
    dev = a_q.device
    if y1 is None and want_y1:
        y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev) if h is None else h
    if amax_out is None and want_amax:
        amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    rc = _lib.load().grouped_gemm_w4a8_silu_gate(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), E, M,
                                                 F, K, _ptr(y1), _ptr(h), _ptr(amax_out), _stream())
    _check("grouped_gemm_w4a8_silu_gate", rc)
    return y1, h, amax_out


def grouped_gemm_w4a8_silu_gate_mx(a_q, a_s, b_q, b_s, offsets, q_h=None, s_h=None, y1=None, h=None,
                                   amax_out=None):
    """Gate+up W4A8 GEMM with the SiLU gate and the MXFP8 quantization of H
    in its epilogue.  y1, h (bf16) and amax_out are written only when given.
    Returns (q_h, s_h)."""
    _dev(a_q, a_s, b_q, b_s, offsets, q_h, s_h, y1, h, amax_out)
    M, K = a_q.shape
    E, N = b_q.shape[0], b_q.shape[1]
    F = N // 2
    dev = a_q.device
    q_h = torch.empty((M, F), dtype=torch.uint8, device=dev) if q_h is None else q_h
    s_h = torch.empty((M, F // 32), dtype=torch.uint8, device=dev) if s_h is None else s_h
    rc = _lib.load().grouped_gemm_w4a8_silu_gate_mx(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), E,
                                                    M, F, K, _ptr(y1), _ptr(h), _ptr(amax_out), _ptr(q_h), _ptr(s_h),
                                                    _stream())
    _check("grouped_gemm_w4a8_silu_gate_mx", rc)
    return q_h, s_h


def grouped_gemm_bf16(layout, a, b, offsets, num_experts=None, out=None, out_dtype=torch.float32, accumulate=False):
    """Grouped BF16 GEMM; layout NT / NN / TN as in the C header."""
    _dev(a, b, offsets, out)
    M = a.shape[0]
    E = offsets.numel() - 1 if num_experts is None else num_experts
    if layout == NT:
        K, N = a.shape[1], b.shape[1]
        shape = (M, N)
    elif layout == NN:
        K, N = a.shape[1], b.shape[2]
        shape = (M, N)
    elif layout == TN:
        K, N = a.shape[1], b.shape[1]
        shape = (E, K, N)
    else:
        raise ValueError("layout must be NT, NN or TN")
    out = torch.empty(shape, dtype=out_dtype, device=a.device) if out is None else out
    rc = _lib.load().grouped_gemm_bf16(layout, _ptr(a), _ptr(b), _ptr(offsets), E, M, N, K, _ptr(out),
                                       _DT[out.dtype], int(bool(accumulate)), None, 0, _stream())
    _check("grouped_gemm_bf16", rc)
    return out


def grouped_gemm_bf16_tn_gather(a, b, src, k, offsets, num_experts=None, out=None, out_dtype=torch.float32,
                                accumulate=False):
    """TN weight gradient with B rows gathered: C_e = sum_{r in e} a[r]^T b[src[r] // k]."""
    _dev(a, b, src, offsets, out)
    M, K = a.shape
    N = b.shape[1]
    E = offsets.numel() - 1 if num_experts is None else num_experts
    out = torch.empty((E, K, N), dtype=out_dtype, device=a.device) if out is None else out
    rc = _lib.load().grouped_gemm_bf16_tn_gather(_ptr(a), _ptr(b), _ptr(src), int(k), b.shape[0], _ptr(offsets), E,
                                                 M, N, K, _ptr(out), _DT[out.dtype], int(bool(accumulate)),
                                                 _stream())
    _check("grouped_gemm_bf16_tn_gather", rc)
    return out


def silu_gate_fwd(y1, h=None, amax_out=None, want_amax=True):
    """H = silu(G) * U for y1 = [G | U]; returns (h, amax)."""
    _dev(y1, h, amax_out)
    R, F2 = y1.shape
    F = F2 // 2
    h = torch.empty((R, F), dtype=torch.bfloat16, device=y1.device) if h is None else h
    if want_amax and amax_out is None:
        amax_out = torch.empty((1,), dtype=torch.float32, device=y1.device)
    rc = _lib.load().silu_gate_fwd(_ptr(y1), R, F, _ptr(h), _ptr(amax_out), _stream())
    _check("silu_gate_fwd", rc)
    return h, amax_out


def silu_gate_bwd(y1, dh, dy1=None, amax_out=None):
    """dY1 = [dG | dU] from Y1 and dH; amax_out (fp32 [1], optional)
    receives max |dY1|."""
    _dev(y1, dh, dy1, amax_out)
    R, F2 = y1.shape
    dy1 = torch.empty((R, F2), dtype=torch.bfloat16, device=y1.device) if dy1 is None else dy1
    rc = _lib.load().silu_gate_bwd(_ptr(y1), _ptr(dh), R, F2 // 2, _ptr(dy1), _ptr(amax_out), _stream())
    _check("silu_gate_bwd", rc)
    return dy1
