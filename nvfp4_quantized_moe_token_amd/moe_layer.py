"""One MoE layer on the NVFP4 token-wise path, chained from the C-ABI entry
points (every step runs in the library's HIP kernels; this module only
orders the calls and owns the buffers).

Forward ("miniTE報告、NVFP4強化学習の安定性を検証", fourth paragraph:
contiguous layout, device-side metadata, amax reuse, grouped GEMM, fusion):
  moe_permute_nvfp4 (amax of X once, metadata, gather fused with the NVFP4
  quantization of the gathered rows; the bf16 permuted rows are kept for the
  backward's gate+up weight gradient unless it gathers them from X)  ->  grouped_gemm_w4a4_silu_gate (gate+up with the SiLU gate and
  the amax of H in its epilogue; Y1 is stored only for the backward)  ->
  nvfp4_quantize(H, amax_in=amax_H)  ->  grouped_gemm_w4a4 (down)  ->
  moe_unpermute (routing-weighted combine).  When F is not a multiple of 128
  the gate+up GEMM and silu_gate_fwd run as two launches.
Backward in BF16 (same page, first paragraph), no amax reduction at all:
  moe_scatter(dY, weighted)  ->  NN dgrad of the down projection  ->
  silu_gate_bwd  ->  TN wgrad of the down projection  ->  NN dgrad of gate+up
  ->  moe_unpermute (unweighted sum back to tokens)  ->  TN wgrad of gate+up,
  on the kept permuted rows, or with its activation rows gathered from X
  through the routing's src (grouped_gemm_bf16_tn_gather: no 268 MB copy at
  8192 tokens, measured ~0.1 ms slower than the copy's TN plus its write).
W4A8 forward (same page, third paragraph: the W4A8 variant with MXFP8
activations; MXFP4 expert weights): MX scales are per 32-element block with
no tensor amax, so X is quantized once per token and the packed rows are
permuted afterwards (quantize(permute(X)) == permute(quantize(X)) row by
row):
  mx_quantize(X, E4M3)  ->  moe_permute (metadata + gather of the code rows)
  + moe_gather (scale rows)  ->  grouped_gemm_w4a8_silu_gate  ->
  mx_quantize(H, E4M3)  ->  grouped_gemm_w4a8 (down)  ->  moe_unpermute.
"""

import torch

from . import ops


def quantize_expert_weights(w):
    """NVFP4 weights of stacked experts [E, N, K] (one global scale per
    expert), each expert read once.  Runs once per optimizer step, outside
    the per-batch path."""
    E, N, K = w.shape
    q, s, g, amax = ops.nvfp4_quantize_onepass(w.reshape(E * N, K), groups=E)
    return dict(q=q.view(E, N, K // 2), s=s.view(E, N, K // 16), g=g, amax=amax)


class Buffers:
    """Device buffers of one layer step, allocated once and reused."""

    def __init__(self, T, k, E, D, F, device, backward=False):
        R = T * k
        bf, f32, u8, i32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        self.T, self.k, self.E, self.D, self.F = T, k, E, D, F
        self.ws = e(max(ops.moe_permute_workspace_size(T, k, E), 1), dt=u8)
        self.x_perm = e(R, D)
        self.amax = e(2, dt=f32)            # [amax_X, amax_H]
        self.a1_q, self.a1_s, self.a1_g = e(R, D // 2, dt=u8), e(R, D // 16, dt=u8), e(1, dt=f32)
        self.y1 = e(R, 2 * F)
        self.h = e(R, F)
        self.a2_q, self.a2_s, self.a2_g = e(R, F // 2, dt=u8), e(R, F // 16, dt=u8), e(1, dt=f32)
        self.y2 = e(R, D)
        self.out = e(T, D)
        if backward:
            self.dy2 = e(R, D)
            self.dh = e(R, F)
            self.dy1 = e(R, 2 * F)
            self.dx_perm = e(R, D)
            self.dx = e(T, D)
            self.dw_dn = e(E, D, F, dt=f32)
            self.dw_gu = e(E, 2 * F, D, dt=f32)


def forward(x, topk_ids, topk_w, wq_gu, wq_dn, buf, keep_y1=True, keep_x_perm=True, fuse_silu=True,
            amax_h_in=None, amax_x_in=None):
    """W4A4 MoE forward; returns the routing metadata dict.  Y1 (buf.y1) is
    written when keep_y1 and the bf16 permuted rows (buf.x_perm) when
    keep_x_perm (the BF16 backward needs Y1, and X_perm unless it gathers
    from X).

    With ``amax_h_in`` (a [1] fp32 device tensor: a delayed amax of H, e.g.
    the previous step's buf.amax[1]) H is requantized inside the gate+up
    GEMM's epilogue with that amax; bf16 H is then stored only when keep_y1
    (the backward needs it), and buf.amax[1] still receives this step's
    max |H|.  With ``amax_x_in`` ([1] fp32 device) X is quantized with that
    amax instead of its own (buf.amax[0] is then not written)."""
    E = buf.E
    meta = ops.moe_permute_nvfp4(topk_ids, E, x, x_perm=buf.x_perm if keep_x_perm else None,
                                 want_x_perm=keep_x_perm, amax_in=amax_x_in,
                                 amax_out=None if amax_x_in is not None else buf.amax[0:1], q=buf.a1_q,
                                 scales=buf.a1_s, gscale=buf.a1_g, workspace=buf.ws)
    wgu = (wq_gu["q"], wq_gu["s"], wq_gu["g"])
    if amax_h_in is not None and buf.F % 128 == 0:
        ops.grouped_gemm_w4a4_silu_gate_nvfp4(buf.a1_q, buf.a1_s, buf.a1_g, *wgu, meta["offsets"], amax_h_in,
                                              y1=buf.y1 if keep_y1 else None, h=buf.h if keep_y1 else None,
                                              amax_out=buf.amax[1:2], q_h=buf.a2_q, s_h=buf.a2_s, g_h=buf.a2_g)
        ops.grouped_gemm_w4a4(buf.a2_q, buf.a2_s, buf.a2_g, wq_dn["q"], wq_dn["s"], wq_dn["g"], meta["offsets"],
                              out=buf.y2)
        ops.moe_unpermute(buf.y2, meta["dest"], buf.T, buf.k, topk_w=topk_w, out=buf.out)
        return meta
    if fuse_silu and buf.F % 128 == 0:
        ops.grouped_gemm_w4a4_silu_gate(buf.a1_q, buf.a1_s, buf.a1_g, *wgu, meta["offsets"],
                                        y1=buf.y1 if keep_y1 else None, want_y1=keep_y1, h=buf.h,
                                        amax_out=buf.amax[1:2])
    else:
        ops.grouped_gemm_w4a4(buf.a1_q, buf.a1_s, buf.a1_g, *wgu, meta["offsets"], out=buf.y1)
        ops.silu_gate_fwd(buf.y1, h=buf.h, amax_out=buf.amax[1:2])
    ops.nvfp4_quantize(buf.h, amax_in=buf.amax[1:2], q=buf.a2_q, scales=buf.a2_s, gscale=buf.a2_g)
    ops.grouped_gemm_w4a4(buf.a2_q, buf.a2_s, buf.a2_g, wq_dn["q"], wq_dn["s"], wq_dn["g"], meta["offsets"],
                          out=buf.y2)
    ops.moe_unpermute(buf.y2, meta["dest"], buf.T, buf.k, topk_w=topk_w, out=buf.out)
    return meta


def backward(dy, topk_w, w_gu, w_dn, meta, buf, wgrad_stream=None, x=None):
    """BF16 backward of ``forward`` (weight gradients in fp32).  Each
    elementwise consumer runs right after its producer, before a weight-
    gradient GEMM streams its fp32 output through the caches.  With ``x``
    (the forward's [T, D] tokens) the gate+up weight gradient gathers its
    activation rows from x; without it, from buf.x_perm (forward with
    keep_x_perm=True).

    With ``wgrad_stream`` (a torch stream) the two weight-gradient GEMMs run
    there, each after the op whose output it reads, overlapping the rest of
    the backward; the current stream waits for them before returning, so the
    caller's next step cannot overwrite their inputs early."""
    main = torch.cuda.current_stream()
    off = meta["offsets"]

    def tn(a, b, out, gather):
        if gather:
            ops.grouped_gemm_bf16_tn_gather(a, b, meta["src"], buf.k, off, out=out)
        else:
            ops.grouped_gemm_bf16(ops.TN, a, b, off, out=out)

    def wgrad(a, b, out, gather=False):
        if wgrad_stream is None:
            tn(a, b, out, gather)
            return
        ready = torch.cuda.Event()
        ready.record(main)
        wgrad_stream.wait_event(ready)
        with torch.cuda.stream(wgrad_stream):
            tn(a, b, out, gather)

    ops.moe_scatter(dy, meta["dest"], meta["offsets"], buf.k, topk_w=topk_w, out=buf.dy2)
    if wgrad_stream is not None:
        wgrad(buf.dy2, buf.h, buf.dw_dn)
    ops.grouped_gemm_bf16(ops.NN, buf.dy2, w_dn, off, out=buf.dh)
    ops.silu_gate_bwd(buf.y1, buf.dh, dy1=buf.dy1)
    if wgrad_stream is None:
        wgrad(buf.dy2, buf.h, buf.dw_dn)
    ops.grouped_gemm_bf16(ops.NN, buf.dy1, w_gu, off, out=buf.dx_perm)
    ops.moe_unpermute(buf.dx_perm, meta["dest"], buf.T, buf.k, topk_w=None, out=buf.dx)
    if x is not None:
        wgrad(buf.dy1, x, buf.dw_gu, gather=True)
    else:
        wgrad(buf.dy1, buf.x_perm, buf.dw_gu)
    if wgrad_stream is not None:
        done = torch.cuda.Event()
        done.record(wgrad_stream)
        main.wait_event(done)


def quantize_expert_weights_mx(w):
    """MXFP4 weights of stacked experts [E, N, K] (E8M0 scale per 32 along
    K; no per-expert scale).  Once per optimizer step."""
    E, N, K = w.shape
    q, sc = ops.mx_quantize(w.reshape(E * N, K), ops.MX_E2M1)
    return dict(q=q.view(E, N, K // 2), s=sc.view(E, N, K // 32))


class BuffersW4A8:
    """Device buffers of one W4A8 forward step, allocated once and reused."""

    def __init__(self, T, k, E, D, F, device):
        R = T * k
        bf, u8 = torch.bfloat16, torch.uint8
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        self.T, self.k, self.E, self.D, self.F = T, k, E, D, F
        self.ws = e(max(ops.moe_permute_workspace_size(T, k, E), 1), dt=u8)
        self.a1_q, self.a1_s = e(R, D, dt=u8), e(R, D // 32, dt=u8)
        self.h = e(R, F)
        self.a2_q, self.a2_s = e(R, F, dt=u8), e(R, F // 32, dt=u8)
        self.y2 = e(R, D)
        self.out = e(T, D)


def forward_w4a8(x, topk_ids, topk_w, wq_gu, wq_dn, buf, keep_h=False):
    """W4A8 MoE forward (MXFP8 activations, MXFP4 weights); returns the
    routing metadata dict.  X is quantized inside the permutation and H
    inside the gate+up epilogue; H is kept in bf16 (buf.h) only with
    ``keep_h`` (a forward-only path)."""
    E = buf.E
    meta = ops.moe_permute_mx(topk_ids, E, x, q=buf.a1_q, scales=buf.a1_s, workspace=buf.ws)
    ops.grouped_gemm_w4a8_silu_gate_mx(buf.a1_q, buf.a1_s, wq_gu["q"], wq_gu["s"], meta["offsets"], q_h=buf.a2_q,
                                       s_h=buf.a2_s, h=buf.h if keep_h else None)
    ops.grouped_gemm_w4a8(buf.a2_q, buf.a2_s, wq_dn["q"], wq_dn["s"], meta["offsets"], out=buf.y2)
    ops.moe_unpermute(buf.y2, meta["dest"], buf.T, buf.k, topk_w=topk_w, out=buf.out)
    return meta


def quantize_expert_weights_t(w, amax=None):
    """NVFP4 of each expert weight transposed (W_e^T [K, N] of W [E, N, K]),
    blocks along the weight's output dimension: the B operand of the NVFP4
    backward's data gradients.  ``amax`` (the forward weights' per-expert
    amax, the same values) is reused when given.  Once per optimizer step."""
    q, sc, g, a = ops.nvfp4_quantize_transposed(w, amax_in=amax)
    return dict(q=q, s=sc, g=g, amax=a)


class NVFP4BackwardBuffers:
    """Buffers of the NVFP4 backward variant (besides Buffers(backward=True))."""

    def __init__(self, T, k, E, D, F, device):
        R = T * k
        Kp = ops.padded_extent(R, E)
        u8, f32 = torch.uint8, torch.float32
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        self.Kp = Kp
        self.amax = e(2, dt=f32)                      # [amax_dY2, amax_dY1]
        self.a_dy2 = (e(R, D // 2), e(R, D // 16), e(1, dt=f32))
        self.a_dy1 = (e(R, F), e(R, 2 * F // 16), e(1, dt=f32))
        self.c_dy2 = (e(D, Kp // 2), e(D, Kp // 16), e(1, dt=f32))
        self.c_h = (e(F, Kp // 2), e(F, Kp // 16), e(1, dt=f32))
        self.c_dy1 = (e(2 * F, Kp // 2), e(2 * F, Kp // 16), e(1, dt=f32))
        self.c_x = (e(D, Kp // 2), e(D, Kp // 16), e(1, dt=f32))


def backward_nvfp4(dy, topk_w, wt_gu, wt_dn, meta, buf, nb, amax_x=None):
    """The NVFP4 backward variant of ``backward``: the same dataflow with the
    four grouped GEMMs in W4A4.  Each gradient's amax comes out of the kernel
    that writes the gradient (the weighted scatter for dY2, the SiLU backward
    for dY1) and is reused by its row-wise and column-wise quantizations; H
    and X_perm reuse the forward's amaxes (buf.amax, or ``amax_x`` when the
    forward was given a fixed one).  wt_gu / wt_dn: quantize_expert_weights_t
    of the bf16 weights.  Weight gradients fp32, activation gradients bf16."""
    off = meta["offsets"]
    R = buf.T * buf.k
    amax_x = buf.amax[0:1] if amax_x is None else amax_x
    ops.moe_scatter(dy, meta["dest"], off, buf.k, topk_w=topk_w, out=buf.dy2, amax_out=nb.amax[0:1])
    q, sc, g = nb.a_dy2
    ops.nvfp4_quantize(buf.dy2, amax_in=nb.amax[0:1], q=q, scales=sc, gscale=g)
    ops.grouped_gemm_w4a4(q, sc, g, wt_dn["q"], wt_dn["s"], wt_dn["g"], off, out=buf.dh)
    ops.silu_gate_bwd(buf.y1, buf.dh, dy1=buf.dy1, amax_out=nb.amax[1:2])
    ops.nvfp4_quantize_colwise(buf.dy2, off, nb.amax[0:1], Kp=nb.Kp, q_t=nb.c_dy2[0], s_t=nb.c_dy2[1],
                               gscale=nb.c_dy2[2])
    ops.nvfp4_quantize_colwise(buf.h, off, buf.amax[1:2], Kp=nb.Kp, q_t=nb.c_h[0], s_t=nb.c_h[1], gscale=nb.c_h[2])
    ops.grouped_gemm_w4a4_wgrad(nb.c_dy2, nb.c_h, off, R, out=buf.dw_dn)
    q, sc, g = nb.a_dy1
    ops.nvfp4_quantize(buf.dy1, amax_in=nb.amax[1:2], q=q, scales=sc, gscale=g)
    ops.grouped_gemm_w4a4(q, sc, g, wt_gu["q"], wt_gu["s"], wt_gu["g"], off, out=buf.dx_perm)
    ops.moe_unpermute(buf.dx_perm, meta["dest"], buf.T, buf.k, topk_w=None, out=buf.dx)
    ops.nvfp4_quantize_colwise(buf.dy1, off, nb.amax[1:2], Kp=nb.Kp, q_t=nb.c_dy1[0], s_t=nb.c_dy1[1],
                               gscale=nb.c_dy1[2])
    ops.nvfp4_quantize_colwise(buf.x_perm, off, amax_x, Kp=nb.Kp, q_t=nb.c_x[0], s_t=nb.c_x[1], gscale=nb.c_x[2])
    ops.grouped_gemm_w4a4_wgrad(nb.c_dy1, nb.c_x, off, R, out=buf.dw_gu)
