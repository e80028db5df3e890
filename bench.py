"""Benchmark of the NVFP4 token-wise MoE hot path on one MI355X.

A step is one pass of the whole path over one batch: the MoE layer forward
on the NVFP4 token-wise path (amax + permute fused with the quantize, grouped
W4A4 GEMM gate+up with the SiLU gate + amax in its epilogue, requantize,
grouped W4A4 GEMM down, unpermute)
followed by its BF16 backward (weighted gather, grouped NN/TN GEMMs for both
projections, SiLU-gate backward, unpermute).  Default workload: the
Qwen3-30B-A3B-shaped full update at 8192 tokens (d_model 2048, 128 experts,
top-8, FFN 768), synthetic seeded inputs, inputs resident in HBM.  Expert
weight quantization runs once per optimizer step and is timed separately.

Per-op times are HIP events recorded inside the timed steps, on the stream
the library launches on (torch's current stream).  Beside the step, the
plain W4A4 gate+up GEMM (bf16 Y1, no epilogue) and the BF16 grouped GEMM on
the same shape and routing (the baseline the W4A4 GEMM is compared with) are
timed alone, and the CPU oracle runs on a bounded sample of the same
workload.

Prints one JSON line (N = 1).

    python bench.py [--steps K] [--warmup W] [--workload moe_8k_update]
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR   # HBM traffic summary
    python bench.py --kernel-stats-summary DIR          # rocprofv3 --stats table
"""

import argparse
import gc
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16/fp16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP4_TFLOPS = 10066.0   # dense fp4 MFMA
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA (the rate of the scaled MFMA with an 8-bit operand)
PEAK_HBM_GBS = 8000.0
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP/byte where the two ceilings meet
PEAK_CLOCK_GHZ = 2.4        # the clock the published MFMA peaks assume
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_moe_8k_update.txt")
CALIB_BYTES = 1 << 30       # the plain copy that calibrates the traffic counters


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest():
    """sha256 over the HIP sources with comments and blank space removed:
    recorded with PMC traffic so that a changed kernel invalidates it."""
    import re
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "nvfp4_quantized_moe_token_amd", "csrc", "*"))):
        with open(p) as f:
            code = re.sub(r"/\*.*?\*/", " ", f.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(os.path.basename(p).encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


def gemm_flops(R, D, F):
    """Algorithmic FLOPs of the two expert projections for R routed rows."""
    return 2.0 * R * (2 * F) * D, 2.0 * R * D * F


def op_work(name, T, k, E, D, F, backward=True):
    """(flops, algorithmic HBM bytes) of one launch of each op of the step:
    every operand read once and every result written once."""
    R = T * k
    f1, f2 = gemm_flops(R, D, F)
    nv = lambda rows, cols: rows * cols * (0.5 + 1.0 / 16)  # noqa: E731  NVFP4 bytes per element
    table = {
        # metadata, X read once (its amax pass reads it once more), the NVFP4
        # rows of X_perm written once, and its bf16 copy when the backward
        # keeps one (the full update)
        "permute_quantize_x": (0.0, T * D * 2 + nv(R, D) + R * 4 * 3 + (R * D * 2 if backward else 0)),
        "w4a4_gate_up": (f1, nv(R, D) + nv(E * 2 * F, D) + R * 2 * F * 2),
        "w4a4_gate_up_scaled_mfma": (f1, nv(R, D) + nv(E * 2 * F, D) + R * 2 * F * 2),
        # with the SiLU gate in the epilogue: Y1 (kept for the backward) and H written
        "w4a4_gate_up_silu": (f1, nv(R, D) + nv(E * 2 * F, D) + R * 2 * F * 2 + R * F * 2),
        "quantize_h": (0.0, R * F * 2 + nv(R, F)),
        "w4a4_down": (f2, nv(R, F) + nv(E * D, F) + R * D * 2),
        "unpermute": (0.0, R * D * 2 + T * D * 2 + R * 4),
        "gather_dy": (0.0, T * D * 2 + R * D * 2 + R * 4),
        "bf16_nn_down": (f2, R * D * 2 + E * D * F * 2 + R * F * 2),
        "bf16_tn_down": (f2, R * D * 2 + R * F * 2 + E * D * F * 4),
        "silu_gate_bwd": (0.0, R * 2 * F * 2 + R * F * 2 + R * 2 * F * 2),
        "bf16_nn_gate_up": (f1, R * 2 * F * 2 + E * 2 * F * D * 2 + R * D * 2),
        # dY1 and X_perm read once, fp32 dW written once
        "bf16_tn_gate_up": (f1, R * 2 * F * 2 + R * D * 2 + E * 2 * F * D * 4),
        "unpermute_dx": (0.0, R * D * 2 + T * D * 2),
        "bf16_nt_gate_up_baseline": (f1, R * D * 2 + E * 2 * F * D * 2 + R * 2 * F * 2),
        "quantize_x_perm_cold": (0.0, R * D * 2 + nv(R, D)),
        # X_perm of the 16384-token workload (16384 x 8 rows x D, 537 MB of bf16)
        "quantize_x_perm_16k_cold": (0.0, 16384 * k * D * 2 + nv(16384 * k, D)),
    }
    return table[name]


# Ops of the full-update step, in launch order (the PMC summary's rows).
STEP_OPS = ["permute_quantize_x", "w4a4_gate_up_silu", "quantize_h", "w4a4_down", "unpermute",
            "gather_dy", "bf16_nn_down", "silu_gate_bwd", "bf16_tn_down", "bf16_nn_gate_up", "unpermute_dx",
            "bf16_tn_gate_up"]
MARKER = "FillFunctor<int>"  # a one-element int fill between ops in --pmc-run


def build_inputs(cfg, torch, dev):
    import numpy as np
    import workloads
    d = workloads.CONFIGS[cfg]()
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)  # noqa: E731
    out = dict(d=d, x=t(d["x"], torch.bfloat16), w_gu=t(d["w_gu"], torch.bfloat16),
               w_dn=t(d["w_dn"], torch.bfloat16), ids=t(d["topk_ids"], torch.int32),
               tw=t(d["topk_w"], torch.float32))
    if "dy" in d:
        out["dy"] = t(d["dy"], torch.bfloat16)
    return out


def step_ops(ops, inp, wq_gu, wq_dn, buf, meta_box, backward):
    """The ops of one step, in launch order, as (name, thunk)."""
    E, k, T = buf.E, buf.k, buf.T

    def permute_quantize():
        # bf16 rows kept for the backward's weight gradient only
        meta_box["m"] = ops.moe_permute_nvfp4(inp["ids"], E, inp["x"], x_perm=buf.x_perm if backward else None,
                                              want_x_perm=backward, amax_out=buf.amax[0:1], q=buf.a1_q,
                                              scales=buf.a1_s, gscale=buf.a1_g, workspace=buf.ws)

    m = lambda: meta_box["m"]  # noqa: E731
    seq = [
        ("permute_quantize_x", permute_quantize),
        ("w4a4_gate_up_silu", lambda: ops.grouped_gemm_w4a4_silu_gate(
            buf.a1_q, buf.a1_s, buf.a1_g, wq_gu["q"], wq_gu["s"], wq_gu["g"], m()["offsets"],
            y1=buf.y1 if backward else None, want_y1=backward, h=buf.h, amax_out=buf.amax[1:2])),
        ("quantize_h", lambda: ops.nvfp4_quantize(buf.h, amax_in=buf.amax[1:2], q=buf.a2_q, scales=buf.a2_s,
                                                  gscale=buf.a2_g)),
        ("w4a4_down", lambda: ops.grouped_gemm_w4a4(buf.a2_q, buf.a2_s, buf.a2_g, wq_dn["q"], wq_dn["s"],
                                                    wq_dn["g"], m()["offsets"], out=buf.y2)),
        ("unpermute", lambda: ops.moe_unpermute(buf.y2, m()["dest"], T, k, topk_w=inp["tw"], out=buf.out)),
    ]
    if backward:
        seq += [
            ("gather_dy", lambda: ops.moe_scatter(inp["dy"], m()["dest"], m()["offsets"], k, topk_w=inp["tw"],
                                                  out=buf.dy2)),
            ("bf16_nn_down", lambda: ops.grouped_gemm_bf16(ops.NN, buf.dy2, inp["w_dn"], m()["offsets"],
                                                           out=buf.dh)),
            ("silu_gate_bwd", lambda: ops.silu_gate_bwd(buf.y1, buf.dh, dy1=buf.dy1)),
            ("bf16_tn_down", lambda: ops.grouped_gemm_bf16(ops.TN, buf.dy2, buf.h, m()["offsets"], out=buf.dw_dn)),
            ("bf16_nn_gate_up", lambda: ops.grouped_gemm_bf16(ops.NN, buf.dy1, inp["w_gu"], m()["offsets"],
                                                              out=buf.dx_perm)),
            ("unpermute_dx", lambda: ops.moe_unpermute(buf.dx_perm, m()["dest"], T, k, topk_w=None, out=buf.dx)),
            ("bf16_tn_gate_up", lambda: ops.grouped_gemm_bf16(ops.TN, buf.dy1, buf.x_perm, m()["offsets"],
                                                              out=buf.dw_gu)),
        ]
    return seq


# With --overlap, the weight-gradient GEMMs run on a second stream, each
# after the op whose output it reads; nothing in the step reads dW, and the
# main stream joins the second one at the end of the step.  The step is then
# faster, but kernels that share the GPU report inflated durations, so the
# default keeps the step serial for per-kernel rooflines.
WGRAD_DEPS = {"bf16_tn_down": "gather_dy", "bf16_tn_gate_up": "silu_gate_bwd"}


def delayed_amax_side(torch, ops, moe_layer, inp, wq_gu, wq_dn, T, k, E, D, F, nrep, keep_bf16):
    """The W4A4 forward with a delayed amax of H (the previous pass's, in a
    two-slot ping-pong): H is requantized in the gate+up GEMM's epilogue
    (grouped_gemm_w4a4_silu_gate_nvfp4), so no quantize launch and no bf16 H
    round trip (bf16 Y1 and H are still stored when keep_bf16, as the BF16
    backward needs them).  Per-op HIP events over nrep forward passes."""
    dev = inp["x"].device
    buf = moe_layer.Buffers(T, k, E, D, F, dev)
    slots = torch.zeros(2, dtype=torch.float32, device=dev)
    box = {"i": 0}

    def permute():
        box["m"] = ops.moe_permute_nvfp4(inp["ids"], E, inp["x"], x_perm=buf.x_perm if keep_bf16 else None,
                                         want_x_perm=keep_bf16, amax_out=buf.amax[0:1], q=buf.a1_q,
                                         scales=buf.a1_s, gscale=buf.a1_g, workspace=buf.ws)

    def gate_up():
        i = box["i"]
        box["i"] = i + 1
        ops.grouped_gemm_w4a4_silu_gate_nvfp4(
            buf.a1_q, buf.a1_s, buf.a1_g, wq_gu["q"], wq_gu["s"], wq_gu["g"], box["m"]["offsets"],
            slots[i % 2:i % 2 + 1], y1=buf.y1 if keep_bf16 else None, h=buf.h if keep_bf16 else None,
            amax_out=slots[(i + 1) % 2:(i + 1) % 2 + 1], q_h=buf.a2_q, s_h=buf.a2_s, g_h=buf.a2_g)

    seq = [
        ("permute_quantize_x", permute),
        ("w4a4_gate_up_silu_requant", gate_up),
        ("w4a4_down", lambda: ops.grouped_gemm_w4a4(buf.a2_q, buf.a2_s, buf.a2_g, wq_dn["q"], wq_dn["s"],
                                                    wq_dn["g"], box["m"]["offsets"], out=buf.y2)),
        ("unpermute", lambda: ops.moe_unpermute(buf.y2, box["m"]["dest"], T, k, topk_w=inp["tw"], out=buf.out)),
    ]
    for _ in range(3):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    evs = []
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(nrep):
        for name, fn in seq:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((name, e0, e1))
    t1.record()
    torch.cuda.synchronize()
    times = {}
    for name, e0, e1 in evs:
        times.setdefault(name, []).append(e0.elapsed_time(e1))
    f1, _ = gemm_flops(T * k, D, F)
    out = {"forward_ms": round(t0.elapsed_time(t1) / nrep, 4), "bf16_y1_h_stored": keep_bf16,
           "ops": {n: {"ms": round(sum(v) / len(v), 4)} for n, v in times.items()}}
    g = out["ops"]["w4a4_gate_up_silu_requant"]
    g["tflops"] = round(f1 / (g["ms"] * 1e-3) / 1e12, 1)
    return out


def nvfp4_backward_side(torch, ops, moe_layer, inp, wq_gu, wq_dn, buf, meta_box, T, k, E, D, F, nrep):
    """The NVFP4 backward variant after the step's forward (whose buffers it
    reads): every op bracketed by HIP events over nrep backward passes.
    Transposed weight quantization is done before the timer (once per
    optimizer step)."""
    dev = inp["x"].device
    wt_gu = moe_layer.quantize_expert_weights_t(inp["w_gu"], amax=wq_gu["amax"])
    wt_dn = moe_layer.quantize_expert_weights_t(inp["w_dn"], amax=wq_dn["amax"])
    nb = moe_layer.NVFP4BackwardBuffers(T, k, E, D, F, dev)
    m = meta_box["m"]
    off = m["offsets"]
    R = T * k
    seq = [
        ("gather_dy", lambda: ops.moe_scatter(inp["dy"], m["dest"], off, k, topk_w=inp["tw"], out=buf.dy2,
                                              amax_out=nb.amax[0:1])),
        ("quantize_dy2", lambda: ops.nvfp4_quantize(buf.dy2, amax_in=nb.amax[0:1], q=nb.a_dy2[0],
                                                    scales=nb.a_dy2[1], gscale=nb.a_dy2[2])),
        ("w4a4_dgrad_down", lambda: ops.grouped_gemm_w4a4(*nb.a_dy2, wt_dn["q"], wt_dn["s"], wt_dn["g"], off,
                                                          out=buf.dh)),
        ("silu_gate_bwd", lambda: ops.silu_gate_bwd(buf.y1, buf.dh, dy1=buf.dy1, amax_out=nb.amax[1:2])),
        ("colwise_dy2", lambda: ops.nvfp4_quantize_colwise(buf.dy2, off, nb.amax[0:1], Kp=nb.Kp, q_t=nb.c_dy2[0],
                                                           s_t=nb.c_dy2[1], gscale=nb.c_dy2[2])),
        ("colwise_h", lambda: ops.nvfp4_quantize_colwise(buf.h, off, buf.amax[1:2], Kp=nb.Kp, q_t=nb.c_h[0],
                                                         s_t=nb.c_h[1], gscale=nb.c_h[2])),
        ("w4a4_wgrad_down", lambda: ops.grouped_gemm_w4a4_wgrad(nb.c_dy2, nb.c_h, off, R, out=buf.dw_dn)),
        ("quantize_dy1", lambda: ops.nvfp4_quantize(buf.dy1, amax_in=nb.amax[1:2], q=nb.a_dy1[0],
                                                    scales=nb.a_dy1[1], gscale=nb.a_dy1[2])),
        ("w4a4_dgrad_gate_up", lambda: ops.grouped_gemm_w4a4(*nb.a_dy1, wt_gu["q"], wt_gu["s"], wt_gu["g"], off,
                                                             out=buf.dx_perm)),
        ("unpermute_dx", lambda: ops.moe_unpermute(buf.dx_perm, m["dest"], T, k, topk_w=None, out=buf.dx)),
        ("colwise_dy1", lambda: ops.nvfp4_quantize_colwise(buf.dy1, off, nb.amax[1:2], Kp=nb.Kp, q_t=nb.c_dy1[0],
                                                           s_t=nb.c_dy1[1], gscale=nb.c_dy1[2])),
        ("colwise_x", lambda: ops.nvfp4_quantize_colwise(buf.x_perm, off, buf.amax[0:1], Kp=nb.Kp, q_t=nb.c_x[0],
                                                         s_t=nb.c_x[1], gscale=nb.c_x[2])),
        ("w4a4_wgrad_gate_up", lambda: ops.grouped_gemm_w4a4_wgrad(nb.c_dy1, nb.c_x, off, R, out=buf.dw_gu)),
    ]
    for _ in range(2):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    evs = []
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(nrep):
        for name, fn in seq:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((name, e0, e1))
    t1.record()
    torch.cuda.synchronize()
    times = {}
    for name, e0, e1 in evs:
        times.setdefault(name, []).append(e0.elapsed_time(e1))
    f1, f2 = gemm_flops(R, D, F)
    fl = {"w4a4_dgrad_down": f2, "w4a4_wgrad_down": f2, "w4a4_dgrad_gate_up": f1, "w4a4_wgrad_gate_up": f1}
    ops_out = {}
    for n, v in times.items():
        ms = sum(v) / len(v)
        ent = {"ms": round(ms, 4)}
        if n in fl:
            ent["tflops"] = round(fl[n] / (ms * 1e-3) / 1e12, 1)
            ent["frac_bf16_mfma_peak"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
        ops_out[n] = ent
    gemm_ms = sum(ops_out[n]["ms"] for n in fl)
    return {"backward_ms": round(t0.elapsed_time(t1) / nrep, 4), "gemm_ms": round(gemm_ms, 4),
            "gemm_tflops": round(2 * (f1 + f2) / (gemm_ms * 1e-3) / 1e12, 1), "ops": ops_out}


def w4a8_side(torch, ops, moe_layer, inp, T, k, E, D, F, nrep):
    """The W4A8 variant (MXFP8 activations x MXFP4 weights on the scaled
    MFMA) on the same routing and shapes: its forward ops, each bracketed by
    HIP events over nrep forward passes, and the plain W4A8 gate+up GEMM
    (bf16 Y1, no epilogue) timed alone.  Expert weights are MX-quantized
    before the timer (once per optimizer step)."""
    dev = inp["x"].device
    wq_gu = moe_layer.quantize_expert_weights_mx(inp["w_gu"])
    wq_dn = moe_layer.quantize_expert_weights_mx(inp["w_dn"])
    buf = moe_layer.BuffersW4A8(T, k, E, D, F, dev)
    box = {}

    def permute():
        box["m"] = ops.moe_permute_mx(inp["ids"], E, inp["x"], q=buf.a1_q, scales=buf.a1_s, workspace=buf.ws)

    m = lambda: box["m"]  # noqa: E731
    seq = [
        ("permute_quantize_mx", permute),
        ("w4a8_gate_up_silu_mx", lambda: ops.grouped_gemm_w4a8_silu_gate_mx(
            buf.a1_q, buf.a1_s, wq_gu["q"], wq_gu["s"], m()["offsets"], q_h=buf.a2_q, s_h=buf.a2_s)),
        ("w4a8_down", lambda: ops.grouped_gemm_w4a8(buf.a2_q, buf.a2_s, wq_dn["q"], wq_dn["s"], m()["offsets"],
                                                    out=buf.y2)),
        ("unpermute", lambda: ops.moe_unpermute(buf.y2, m()["dest"], T, k, topk_w=inp["tw"], out=buf.out)),
    ]
    for _ in range(3):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    times = {}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    evs = []
    t0.record()
    for _ in range(nrep):
        for name, fn in seq:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((name, e0, e1))
    t1.record()
    torch.cuda.synchronize()
    for name, e0, e1 in evs:
        times.setdefault(name, []).append(e0.elapsed_time(e1))
    times = {n: sum(v) / len(v) for n, v in times.items()}
    fwd_ms = t0.elapsed_time(t1) / nrep
    # plain gate+up (bf16 Y1) alone
    y1 = torch.empty(T * k, 2 * F, dtype=torch.bfloat16, device=dev)
    plain = lambda: ops.grouped_gemm_w4a8(buf.a1_q, buf.a1_s, wq_gu["q"], wq_gu["s"], m()["offsets"], out=y1)  # noqa: E731
    for _ in range(3):
        plain()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record()
    for _ in range(nrep):
        plain()
    b1.record()
    torch.cuda.synchronize()
    times["w4a8_gate_up"] = b0.elapsed_time(b1) / nrep
    f1, f2 = gemm_flops(T * k, D, F)
    gemm_ms = times["w4a8_gate_up_silu_mx"] + times["w4a8_down"]
    out = {"forward_ms": round(fwd_ms, 4), "tokens_per_s_forward": round(T / (fwd_ms * 1e-3), 1),
           "gemm_ms": round(gemm_ms, 4), "tflops": round((f1 + f2) / (gemm_ms * 1e-3) / 1e12, 1)}
    out["frac_fp8_mfma_peak"] = round(out["tflops"] / PEAK_FP8_TFLOPS, 4)
    out["frac_bf16_mfma_peak"] = round(out["tflops"] / PEAK_BF16_TFLOPS, 4)
    ops_out = {}
    for name, ms in times.items():
        fl = {"w4a8_gate_up_silu_mx": f1, "w4a8_gate_up": f1, "w4a8_down": f2}.get(name)
        ent = {"ms": round(ms, 4)}
        if fl:
            tf = fl / (ms * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), frac_fp8_mfma_peak=round(tf / PEAK_FP8_TFLOPS, 4),
                       frac_bf16_mfma_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        ops_out[name] = ent
    out["ops"] = ops_out
    return out


def run_step(torch, seq, wstream, timed):
    """Enqueue one step; returns [(op, start event, end event)], each pair on
    the stream the op runs on."""
    main = torch.cuda.current_stream()
    done, out, last_w = {}, [], None
    for name, fn in seq:
        on_w = wstream is not None and name in WGRAD_DEPS
        st = wstream if on_w else main
        with torch.cuda.stream(st):
            if on_w:
                st.wait_event(done[WGRAD_DEPS[name]])
            e0 = torch.cuda.Event(enable_timing=timed)
            e0.record(st)
            fn()
            e1 = torch.cuda.Event(enable_timing=timed)
            e1.record(st)
        done[name] = e1
        if on_w:
            last_w = e1
        out.append((name, e0, e1))
    if last_w is not None:
        main.wait_event(last_w)
    return out


def cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the same workload:
    4096 tokens routed top-8 over 64 experts (512 rows per expert, the
    per-expert GEMM shape of the full update), forward + BF16 backward.
    Expert weight quantization happens before the timer, as on the GPU."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    host_cpus = os.cpu_count()
    T, k, E, D, F = 4096, 8, 64, 2048, 768
    d = workloads.moe(T, 0.0, with_dy=True, E=E, k=k, D=D, F=F, name="cpu_sample")
    wq_gu = oracle.layer.quantize_weights(d["w_gu"])
    wq_dn = oracle.layer.quantize_weights(d["w_dn"])
    t0 = time.perf_counter()
    f = oracle.layer.forward(d["x"], d["topk_ids"], d["topk_w"], d["w_gu"], d["w_dn"], wq_gu=wq_gu, wq_dn=wq_dn)
    oracle.layer.backward(f, d["dy"], d["topk_w"], d["w_gu"], d["w_dn"])
    dt = time.perf_counter() - t0
    f1, f2 = gemm_flops(T * k, D, F)
    flops = 3 * (f1 + f2)
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample="forward+backward of 4096 tokens x top-8 over 64 experts (512 rows per expert), "
                       "d_model 2048, FFN 768, fp64 GEMMs on %d BLAS threads (elementwise numpy on 1); "
                       "%.1f s" % (cores, dt),
                blas_threads=int(cores), host_cpus=host_cpus, seconds=round(dt, 2), tokens_per_s=round(T / dt, 1))


def load_traffic():
    """Per-op HBM bytes from the committed PMC summary, or {} when absent or
    taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    digest, out = None, {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 2 and parts[0] == "sources":
                digest = parts[1]
            elif len(parts) >= 7 and parts[0] == "op":
                out.setdefault(parts[1], {}).update(fetch=float(parts[3]), write=float(parts[5]))
            elif len(parts) == 3 and parts[0] == "clock":
                out.setdefault(parts[1], {})["clock_ghz"] = float(parts[2])
    return out if digest == source_digest() else {}


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_moe_8k_update.txt")


def load_mfma():
    """Per-op MFMA counters (executed GFLOP, MFMA busy fraction) from the
    committed summary, or {} when absent or taken on different sources."""
    if not os.path.exists(MFMA_FILE):
        return {}
    digest, out = None, {}
    with open(MFMA_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] == "sources":
                digest = parts[1]
            elif len(parts) == 8 and parts[0] in STEP_OPS:
                out[parts[0]] = {"executed_gflop": float(parts[1]), "mfma_busy": round(float(parts[7].rstrip("%")) / 100, 4)}
    return out if digest == source_digest() else {}


def short_name(n):
    """Kernel name without namespace, return type and parameter list."""
    n = n.replace("(anonymous namespace)::", "").replace("nvfp4moe::", "")
    n = n[5:] if n.startswith("void ") else n
    return n.split("(")[0].replace(" ", "")


def pmc_summary(fetch_dir, write_dir, clock_dir=None):
    """Turn two rocprofv3 --pmc runs of `bench.py --pmc-run` (FETCH_SIZE,
    then WRITE_SIZE; counters in KiB per dispatch) into per-op HBM bytes of
    the last step, scaled by what the counters read for a plain 1 GiB copy.
    In that run each op is preceded by a one-element int fill (the marker),
    so an op's dispatches are the ones between two markers."""
    import csv

    def read(d, counter, with_ns=False):
        rows, ns = {}, {}
        for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        i = int(r["Dispatch_Id"])
                        v = rows.get(i, (r["Kernel_Name"], 0.0))[1] + float(r["Counter_Value"])
                        rows[i] = (r["Kernel_Name"], v)
                        ns[i] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        if with_ns:
            return [(rows[i][0], rows[i][1], ns[i]) for i in sorted(rows)]
        return [rows[i] for i in sorted(rows)]

    def per_op(rows):
        cal = rows[-1][1] * 1024.0                      # the calibration copy comes last
        marks = [i for i, (n, _) in enumerate(rows) if MARKER in n]
        marks = marks[-(len(STEP_OPS) + 1):]            # the last step's markers
        out = []
        for j, name in enumerate(STEP_OPS):
            seg = rows[marks[j] + 1:marks[j + 1]]
            out.append((name, sum(v for _, v in seg) * 1024.0, sorted({short_name(n) for n, _ in seg})))
        return cal, out

    cal_f, fetch = per_op(read(fetch_dir, "FETCH_SIZE"))
    cal_w, write = per_op(read(write_dir, "WRITE_SIZE"))
    sf, sw = CALIB_BYTES / cal_f, CALIB_BYTES / cal_w
    lines = ["# HBM traffic per op of one moe_8k_update step, from two rocprofv3 --pmc runs of",
             "# `bench.py --pmc-run` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, summed over the op's",
             "# kernels) scaled by the counters' reading of a plain %d-byte device copy:" % CALIB_BYTES,
             "# fetch x%.4f, write x%.4f.  Bytes per launch; 'sources' fingerprints the HIP sources (code, comments removed)." % (sf, sw),
             "# commands ($REPO: the repository, $OUT: any output directory): cd /tmp && export TMPDIR=/tmp &&",
             "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o run -- python $REPO/bench.py",
             "#   --pmc-run --steps 2 --warmup 1 (the same with WRITE_SIZE into $OUT/pmc_write and with",
             "#   GRBM_GUI_ACTIVE into $OUT/pmc_clock), then python $REPO/bench.py --pmc-summary",
             "#   $OUT/pmc_fetch $OUT/pmc_write $OUT/pmc_clock",
             "sources %s" % source_digest()]
    for (name, fb, kn), (_, wb, _) in zip(fetch, write):
        lines.append("op %s fetch %.0f write %.0f kernels %s" % (name, fb * sf, wb * sw, ";".join(kn)))
    if clock_dir:
        # GRBM_GUI_ACTIVE counts GPU-busy cycles summed over the 8 XCDs; per
        # op, cycles / 8 / the dispatches' own duration is the shader clock
        # the op ran at.
        rows = read(clock_dir, "GRBM_GUI_ACTIVE", with_ns=True)
        marks = [i for i, r in enumerate(rows) if MARKER in r[0]][-(len(STEP_OPS) + 1):]
        lines.append("# sustained shader clock per op: GRBM_GUI_ACTIVE / 8 XCDs / dispatch time "
                     "(a third --pmc run with GRBM_GUI_ACTIVE); meaningful for the GEMMs (hundreds of us),")
        lines.append("# while short kernels read high (the counter window is wider than the kernel)")
        for j, name in enumerate(STEP_OPS):
            seg = [r for r in rows[marks[j] + 1:marks[j + 1]] if r[2] > 0]
            cyc, ns = sum(r[1] for r in seg), sum(r[2] for r in seg)
            if ns > 0:
                lines.append("clock %s %.3f" % (name, cyc / 8.0 / ns))
    print("\n".join(lines))


def _pmc_by_op(dirs):
    """Counter values of `bench.py --pmc-run` runs (rocprofv3 --pmc, csv),
    summed over each step op's GEMM dispatches (ops without a GEMM: all their
    dispatches) in the last step; {op: {counter: value}} and {op: us}."""
    import csv
    per_op, us = {}, {}
    for d in dirs:
        vals, names, ns = {}, {}, {}
        for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(p) as f:
                for r in csv.DictReader(f):
                    i = int(r["Dispatch_Id"])
                    names[i] = r["Kernel_Name"]
                    ns[i] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                    c = vals.setdefault(i, {})
                    c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ids = sorted(vals)
        marks = [j for j, i in enumerate(ids) if MARKER in names[i]][-(len(STEP_OPS) + 1):]
        if len(marks) != len(STEP_OPS) + 1:
            sys.exit("%s: not a --pmc-run counter run" % d)
        for j, name in enumerate(STEP_OPS):
            seg = [ids[x] for x in range(marks[j] + 1, marks[j + 1])]
            gem = [i for i in seg if "gemm_kernel" in names[i]]
            seg = gem or seg
            us.setdefault(name, sum(ns[i] for i in seg) / 1e3)
            o = per_op.setdefault(name, {})
            run = {}
            for i in seg:
                for c, v in vals[i].items():
                    run[c] = run.get(c, 0.0) + v
            # each counter keeps the clock count of the run that collected it
            for c, v in run.items():
                if c != "GRBM_GUI_ACTIVE":
                    o[c] = v
                    o["clk:" + c] = run.get("GRBM_GUI_ACTIVE", 0.0)
    return per_op, us


def counter_summary(dirs):
    """Where the GEMMs of one moe_8k_update step spend their time, from
    several rocprofv3 --pmc runs of `bench.py --pmc-run` (one counter set
    each): wave-cycle shares, MFMA busy, the load path (TA and TD busy, TD
    waiting on the L1/L2), L2 hit rate and read latencies, LDS bank
    conflicts.  Per-CU blocks are normalised by GRBM_GUI_ACTIVE / 8 XCDs x
    256 CUs, per-SIMD ones by x 1024 SIMDs."""
    per_op, us = _pmc_by_op(dirs)

    def ratio(o, a, b, scale=1.0):
        if b == "GRBM_GUI_ACTIVE":
            b = "clk:" + a
        return o[a] / o[b] * scale if a in o and o.get(b) else float("nan")

    cols = [("us", None),
            ("wait_any", lambda o: ratio(o, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
            ("wait_issue", lambda o: ratio(o, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
            ("active", lambda o: ratio(o, "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES")),
            ("mfma_busy", lambda o: ratio(o, "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", 8 / 1024)),
            ("ta_busy", lambda o: ratio(o, "TA_TA_BUSY_sum", "GRBM_GUI_ACTIVE", 8 / 256)),
            ("td_busy", lambda o: ratio(o, "TD_TD_BUSY_sum", "GRBM_GUI_ACTIVE", 8 / 256)),
            ("td_wait_l2", lambda o: ratio(o, "TD_TC_STALL_sum", "GRBM_GUI_ACTIVE", 8 / 256)),
            ("l2_hit", lambda o: o["TCC_HIT_sum"] / (o["TCC_HIT_sum"] + o["TCC_MISS_sum"])
             if o.get("TCC_HIT_sum", 0) + o.get("TCC_MISS_sum", 0) > 0 else float("nan")),
            ("l1l2_lat", lambda o: ratio(o, "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum")),
            ("miss_lat", lambda o: ratio(o, "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum")),
            ("lds_conf", lambda o: ratio(o, "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"))]
    lines = ["# Where the GEMMs of one moe_8k_update step spend their time (8192 tokens, d_model 2048,",
             "# 128 experts, top-8, FFN 768), from rocprofv3 --pmc runs of `bench.py --pmc-run`, one counter",
             "# set per run, summed over each op's GEMM dispatches of the last step.",
             "# wait_any / wait_issue / active: shares of SQ_WAVE_CYCLES waiting on s_waitcnt or a barrier,",
             "#   waiting to issue (a dependency or a busy unit), issuing; mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES",
             "#   per SIMD-cycle; ta_busy, td_busy, td_wait_l2: TA_TA_BUSY, TD_TD_BUSY, TD_TC_STALL per",
             "#   CU-cycle (the load path of each CU: address unit, data return, data return waiting on",
             "#   the L1/L2); l2_hit: TCC_HIT / (TCC_HIT + TCC_MISS); l1l2_lat: mean L1->L2 read latency",
             "#   (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ, cycles); miss_lat: mean L2-miss read latency",
             "#   (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ); lds_conf: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.",
             "# commands ($REPO: the repository, $OUT: any output directory): cd /tmp && export TMPDIR=/tmp &&",
             "#   rocprofv3 --pmc <set> --output-format csv -d $OUT/<n> -o run -- python $REPO/bench.py --pmc-run",
             "#   --steps 2 --warmup 1 --no-cpu-baseline, once per counter set:",
             "#   a: SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_LDS",
             "#      SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_MISC GRBM_GUI_ACTIVE",
             "#   b: SQ_WAIT_INST_LDS SQ_INST_LEVEL_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL",
             "#      SQ_LDS_CMD_FIFO_FULL SQ_INSTS_LDS SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE",
             "#   d: TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_UTCL1_TRANSLATION_MISS_sum",
             "#      TCP_UTCL1_REQUEST_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
             "#   e: TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum TCP_PENDING_STALL_CYCLES_sum",
             "#      TCP_TCR_TCP_STALL_CYCLES_sum GRBM_GUI_ACTIVE",
             "#   f: TA_TA_BUSY_sum TA_DATA_STALLED_BY_TC_CYCLES_sum TD_TD_BUSY_sum TD_TC_STALL_sum",
             "#      TCP_TD_TCP_STALL_CYCLES_sum TCP_PENDING_STALL_CYCLES_sum GRBM_GUI_ACTIVE",
             "# then python $REPO/bench.py --counter-summary $OUT/a $OUT/b $OUT/d $OUT/e $OUT/f",
             "sources %s" % source_digest(),
             "%-18s" % "op" + "".join("%11s" % c for c, _ in cols)]
    for name in STEP_OPS:
        o = per_op.get(name, {})
        if not o:
            continue
        row = "%-18s%11.1f" % (name, us[name])
        for c, fn in cols[1:]:
            v = fn(o)
            row += "%11.0f" % v if c.endswith("lat") else "%11.3f" % v
        lines.append(row)
    print("\n".join(lines))


def mfma_summary(d):
    """Per op of one moe_8k_update step, from a rocprofv3 --pmc run of
    `bench.py --pmc-run` with SQ_INSTS_VALU_MFMA_MOPS_F16,
    SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE:
    the MFMA FLOPs the hardware executed (MOPS x 512) against the algorithmic
    FLOPs (the difference is tile padding), the executed TFLOP/s over the ops'
    dispatch time, and the fraction of SIMD cycles the MFMA unit was busy."""
    import csv
    vals, names, ns = {}, {}, {}
    for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(p) as f:
            for r in csv.DictReader(f):
                i = int(r["Dispatch_Id"])
                names[i] = r["Kernel_Name"]
                ns[i] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                c = vals.setdefault(i, {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(vals)
    marks = [j for j, i in enumerate(ids) if MARKER in names[i]][-(len(STEP_OPS) + 1):]
    T, k, E, D, F = 8192, 8, 128, 2048, 768
    simds = 256 * 4
    lines = ["# MFMA work per op of one moe_8k_update step (8192 tokens, d_model 2048, 128 experts, top-8, FFN 768),",
             "# from one rocprofv3 --pmc run of `bench.py --pmc-run` (counters summed over each op's dispatches).",
             "# executed = (SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16) x 512 FLOPs; algorithmic = 2*M*N*K of the op;",
             "# busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); TFLOP/s over the",
             "# dispatch time; peak 2516.6 TFLOP/s (16-bit dense MFMA at 2.4 GHz).",
             "# command ($REPO: the repository, $OUT: any output directory): cd /tmp && export TMPDIR=/tmp &&",
             "#   rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES",
             "#   GRBM_GUI_ACTIVE --output-format csv -d $OUT/pmc_mfma -o run -- python $REPO/bench.py --pmc-run",
             "#   --steps 2 --warmup 1, then python $REPO/bench.py --mfma-summary $OUT/pmc_mfma",
             "sources %s" % source_digest(),
             "%-20s %12s %12s %8s %10s %10s %8s %8s" % ("op", "exec_GF", "algo_GF", "exec/alg", "us", "exec_TF",
                                                      "of_peak", "busy")]
    for j, name in enumerate(STEP_OPS):
        seg = ids[marks[j] + 1:marks[j + 1]]
        mops = sum(vals[i].get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + vals[i].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
                   for i in seg)
        if mops == 0:
            continue
        ex = mops * 512.0
        alg = op_work(name, T, k, E, D, F)[0]
        t = sum(ns[i] for i in seg)
        busy = sum(vals[i].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for i in seg)
        gui = sum(vals[i].get("GRBM_GUI_ACTIVE", 0.0) for i in seg) / 8.0
        lines.append("%-20s %12.1f %12.1f %8.3f %10.1f %10.1f %7.1f%% %7.1f%%" % (
            name, ex / 1e9, alg / 1e9, ex / alg, t / 1e3, ex / (t * 1e-9) / 1e12,
            100.0 * ex / (t * 1e-9) / 1e12 / PEAK_BF16_TFLOPS, 100.0 * busy / (gui * simds) if gui else 0.0))
    print("\n".join(lines))


# Ops that launch the same kernel (one template instance per GEMM mode): the
# roofline of a kernel averages over all of its launches in a step, as
# rocprofv3's per-kernel statistics do.
# Names as rocprofv3 prints them (first template argument = mode).
KERNEL_OF_OP = {"w4a4_gate_up_silu": "gemm_kernel<4,...> (W4A4 + SiLU gate)", "w4a4_down": "gemm_kernel<3,...> (W4A4)",
                "bf16_nn_down": "gemm_kernel<1,...> (BF16 NN)", "bf16_nn_gate_up": "gemm_kernel<1,...> (BF16 NN)",
                "bf16_tn_down": "gemm_kernel<2,...> (BF16 TN)", "bf16_tn_gate_up": "gemm_kernel<2,...> (BF16 TN)"}


def kernel_stats_summary(d):
    """Print the per-kernel table of a `rocprofv3 --kernel-trace --stats
    --output-format csv` run (durations in microseconds)."""
    import csv
    paths = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not paths:
        sys.exit("no *kernel_stats.csv under %s" % d)
    rows = []
    with open(paths[-1]) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["Percentage"])))
    rows.sort(key=lambda r: -r[2])
    print("# Kernel statistics of the default bench run (moe_8k_update: 5 warm-up and 20 timed steps, plus the\n"
          "# side measurements), durations in microseconds.\n"
          "# command ($REPO: the repository, $OUT: any output directory): cd /tmp && export TMPDIR=/tmp &&\n"
          "#   rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_kt -o kt -- python $REPO/bench.py,\n"
          "#   then python $REPO/bench.py --kernel-stats-summary $OUT/prof_kt\n"
          "sources %s" % source_digest())
    print("%-72s %6s %11s %10s %10s %10s %6s" % ("kernel", "calls", "total_us", "avg_us", "min_us", "max_us", "pct"))
    for n, c, t, a, lo, hi, p in rows:
        n = n.replace("(anonymous namespace)::", "")
        n = n if len(n) <= 72 else n[:69] + "..."
        print("%-72s %6d %11.1f %10.2f %10.2f %10.2f %6.2f" % (n, c, t, a, lo, hi, p))


def dispatch_summary(d, name):
    """Per-launch durations of the kernels whose name contains `name` in a
    `rocprofv3 --kernel-trace --output-format csv` run, grouped by grid size
    (one group per tensor size): count, median, min and max in microseconds."""
    import csv
    paths = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if not paths:
        sys.exit("no *kernel_trace.csv under %s" % d)
    groups = {}
    with open(paths[-1]) as f:
        for r in csv.DictReader(f):
            if name not in r["Kernel_Name"]:
                continue
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
            groups.setdefault(key, []).append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3)
    print("# Per-launch durations of the kernels named %r in the kernel trace of the default bench run,\n"
          "# grouped by grid size (one group per tensor size), in microseconds.\n"
          "# command ($REPO: the repository, $OUT: any output directory): cd /tmp && export TMPDIR=/tmp &&\n"
          "#   rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_kt -o kt -- python $REPO/bench.py,\n"
          "#   then python $REPO/bench.py --dispatch-summary $OUT/prof_kt %s\n"
          "sources %s" % (name, name, source_digest()))
    print("%-40s %14s %6s %10s %10s %10s" % ("kernel", "work-items", "calls", "median_us", "min_us", "max_us"))
    for (kn, grid), ts in sorted(groups.items(), key=lambda kv: kv[0][1]):
        ts.sort()
        print("%-40s %14d %6d %10.2f %10.2f %10.2f" % (kn[:40], grid, len(ts), ts[len(ts) // 2], ts[0], ts[-1]))


def dense_side(args):
    """The dense special case on the Qwen3-4B up-projection shape
    (X [4096, 2560], W [9728, 2560], one expert with offsets [0, M]): NVFP4
    quantize of X and of W (amax computed, cache flushed), the W4A4 GEMM to
    bf16, and this build's BF16 NT GEMM on the same shape, each the median
    of its timed repetitions (HIP events)."""
    import numpy as np
    import torch
    import workloads
    from nvfp4_quantized_moe_token_amd import ops

    dev = torch.device("cuda:0")
    d = workloads.qwen3_4b_up()
    x = torch.from_numpy(np.ascontiguousarray(d["x"])).to(dev).to(torch.bfloat16)
    w = torch.from_numpy(np.ascontiguousarray(d["w"])).to(dev).to(torch.bfloat16)
    M, K = x.shape
    N = w.shape[0]
    offs = torch.tensor([0, M], dtype=torch.int32, device=dev)
    flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)

    def timed(fn, reps, cold=False):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            if cold:
                flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    xq = ops.nvfp4_quantize(x)
    wq = ops.nvfp4_quantize(w)
    y4 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    yb = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    reps = max(7, min(args.steps, 20))
    ms_qx = timed(lambda: ops.nvfp4_quantize(x, amax_out=xq[3], q=xq[0], scales=xq[1], gscale=xq[2]), 7, cold=True)
    ms_qw = timed(lambda: ops.nvfp4_quantize(w, amax_out=wq[3], q=wq[0], scales=wq[1], gscale=wq[2]), 7, cold=True)
    wq3 = (wq[0].view(1, N, K // 2), wq[1].view(1, N, K // 16), wq[2])
    ms_w4 = timed(lambda: ops.grouped_gemm_w4a4(xq[0], xq[1], xq[2], *wq3, offs, out=y4), reps)
    ms_bf = timed(lambda: ops.grouped_gemm_bf16(ops.NT, x, w.view(1, N, K), offs, out=yb), reps)
    fl = 2.0 * M * N * K
    nvb = lambda r, c: r * c // 2 + r * c // 16  # noqa: E731

    def gemm_obj(ms, name, in_bytes):
        tf = fl / (ms * 1e-3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "ms": round(ms, 4),
                "algorithmic_bytes": in_bytes + M * N * 2}

    def quant_obj(ms, rows):
        # amax computed (amax_in not given): the amax pass reads the tensor
        # once more, 2 + 2 + 0.5625 B per element
        by = rows * K * 2 * 2 + nvb(rows, K)
        gbs = by / (ms * 1e-3) / 1e9
        return {"kernel": "amax + quantize (amax computed, cold)", "bound": "hbm", "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(ms, 4),
                "algorithmic_bytes": by}

    w4 = gemm_obj(ms_w4, "grouped_gemm_w4a4 (E=1)", nvb(M, K) + nvb(N, K))
    bf = gemm_obj(ms_bf, "grouped_gemm_bf16 NT (E=1)", (M + N) * K * 2)
    del flush
    return {"M": M, "N": N, "K": K, "reps": reps,
            "w4a4": {**w4, "frac_fp4_peak": round(w4["achieved"] / PEAK_FP4_TFLOPS, 4)},
            "bf16": bf, "w4a4_speedup_vs_bf16": round(ms_bf / ms_w4, 3),
            "quantize_x": quant_obj(ms_qx, M), "quantize_w": quant_obj(ms_qw, N)}


AB_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]
AB_KERNELS = [("gemm_kernel<3,", "W4A4 design A: E2M1 x E4M3 expanded exactly to fp16, fp16 MFMA 32x32x16"),
              ("gemm_kernel<9,", "W4A4 design B: fp4 scaled MFMA 32x32x64, one 16-block per issue, fp32 rescale"),
              ("gemm_kernel<5,", "W4A8 (MXFP8 x MXFP4): fp8 x fp4 scaled MFMA 32x32x64, native E8M0 scales"),
              ("gemm_kernel<0,", "BF16 NT: bf16 MFMA 32x32x16")]


def ab_run(args):
    """The gate+up GEMM of the 8k-update step (65536 routed rows, 128
    experts, 2F = 1536, K = 2048) in the four ways this library can run it,
    three launches each, for rocprofv3 counter and trace runs: W4A4 by exact
    fp16 expansion (the shipped design), W4A4 by scale factoring onto the
    fp4 scaled MFMA, W4A8 on the scaled MFMA, and BF16."""
    import torch
    from nvfp4_quantized_moe_token_amd import moe_layer, ops
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = build_inputs("moe_8k_update", torch, dev)
    d = inp["d"]
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    wq_gu = moe_layer.quantize_expert_weights(inp["w_gu"])
    wx_gu = moe_layer.quantize_expert_weights_mx(inp["w_gu"])
    m = ops.moe_permute_nvfp4(inp["ids"], E, inp["x"], want_x_perm=True)
    pm = ops.moe_permute_mx(inp["ids"], E, inp["x"])
    y = torch.empty(T * k, 2 * F, dtype=torch.bfloat16, device=dev)
    w4 = (m["q"], m["scales"], m["gscale"], wq_gu["q"], wq_gu["s"], wq_gu["g"], m["offsets"])
    runs = [lambda: ops.grouped_gemm_w4a4(*w4, out=y),
            lambda: ops.grouped_gemm_w4a4_scaled_mfma(*w4, out=y),
            lambda: ops.grouped_gemm_w4a8(pm["q"], pm["scales"], wx_gu["q"], wx_gu["s"], pm["offsets"], out=y),
            lambda: ops.grouped_gemm_bf16(ops.NT, m["x_perm"], inp["w_gu"], m["offsets"], out=y)]
    for fn in runs:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
    log("ab run done")


def ab_summary(trace_dir, pmc_dir):
    """Per design of the gate+up GEMM (ab_run): average launch time from a
    kernel-trace run, and the counters of a --pmc run (averaged over the
    launches): VALU and LDS instructions per MFMA instruction, the MFMA
    unit's busy fraction of SIMD cycles, LDS bank-conflict cycles."""
    import csv
    T, k, D, F = 8192, 8, 2048, 768
    flops = 2.0 * T * k * 2 * F * D
    dur = {}
    for p in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)):
        with open(p) as f:
            for r in csv.DictReader(f):
                n = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("nvfp4moe::", "")
                for key, _ in AB_KERNELS:
                    if key in n.replace(" ", ""):
                        dur.setdefault(key, []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    vals = {}
    for p in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(p) as f:
            for r in csv.DictReader(f):
                n = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("nvfp4moe::", "").replace(" ", "")
                for key, _ in AB_KERNELS:
                    if key in n:
                        c = vals.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), {})
                        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["# The gate+up GEMM of the 8k-update step (65536 routed rows, 128 experts, N = 1536, K = 2048;",
             "# %.1f GFLOP) run four ways; time: average of 3 launches from a kernel-trace run; counters: one" % (flops / 1e9),
             "# --pmc run, averaged over the 3 launches.  valu/mfma and lds/mfma: SQ_INSTS_VALU, SQ_INSTS_LDS per",
             "# SQ_INSTS_MFMA; mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs);",
             "# valu_active: SQ_ACTIVE_INST_VALU x 4 / (GRBM_GUI_ACTIVE / 8 x 1024) (wave-cycles on VALU per SIMD cycle);",
             "# lds_conflict: SQ_LDS_BANK_CONFLICT cycles per launch.",
             "# commands ($REPO: the repository, $OUT: any output directory): cd /tmp && export TMPDIR=/tmp &&",
             "#   rocprofv3 --kernel-trace --output-format csv -d $OUT/ab_kt -o run -- python $REPO/bench.py --ab-run;",
             "#   rocprofv3 --pmc %s --output-format csv -d $OUT/ab_pmc -o run --" % " ".join(AB_COUNTERS),
             "#   python $REPO/bench.py --ab-run; then python $REPO/bench.py --ab-summary $OUT/ab_kt $OUT/ab_pmc",
             "sources %s" % source_digest(),
             "%-16s %9s %8s %8s %9s %9s %10s %10s %13s  %s" % ("kernel", "us", "TFLOP/s", "of_bf16", "valu/mfma",
                                                             "lds/mfma", "mfma_busy", "valu_act", "lds_conflict",
                                                             "design")]
    for key, desc in AB_KERNELS:
        ts = dur.get(key, [])
        us = sum(ts) / len(ts) / 1e3 if ts else float("nan")
        cs = list(vals.get(key, {}).values())
        avg = {c: sum(v.get(c, 0.0) for v in cs) / max(len(cs), 1) for c in AB_COUNTERS}
        mf = avg["SQ_INSTS_MFMA"] or float("nan")
        cyc = avg["GRBM_GUI_ACTIVE"] / 8.0 * 1024
        tf = flops / (us * 1e-6) / 1e12 if ts else float("nan")
        lines.append("%-16s %9.1f %8.1f %7.1f%% %9.2f %9.2f %9.1f%% %9.1f%% %13.0f  %s" % (
            key.rstrip(","), us, tf, 100 * tf / PEAK_BF16_TFLOPS, avg["SQ_INSTS_VALU"] / mf, avg["SQ_INSTS_LDS"] / mf,
            100 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / cyc if cyc else float("nan"),
            100 * avg["SQ_ACTIVE_INST_VALU"] * 4 / cyc if cyc else float("nan"), avg["SQ_LDS_BANK_CONFLICT"], desc))
    print("\n".join(lines))


def bench_dense(args):
    """One JSON line for the dense workload: `value` is the W4A4 GEMM's
    TFLOP/s (see dense_side)."""
    import torch
    torch.cuda.set_device(torch.device("cuda:0"))
    r = dense_side(args)
    w4 = r["w4a4"]
    res = {
        "metric": "W4A4 MoE grouped-GEMM TFLOP/s + % MI355X MFMA peak; quantize GB/s",
        "value": w4["achieved"], "unit": "TFLOP/s", "n_gpus": 1, "steps": r["reps"], "warmup": 1,
        "ms_per_step": w4["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 mfma, fp32 acc", "data": "synthetic",
        "config": {"workload": "qwen3_4b_up", "M": r["M"], "N": r["N"], "K": r["K"], "parallelism": "none (1 GPU)"},
        "w4a4_gemm": {**w4, "speedup_vs_bf16": r["w4a4_speedup_vs_bf16"]},
        "bf16_gemm": r["bf16"],
        "quantize_x": r["quantize_x"],
        "quantize_w": r["quantize_w"],
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe_8k_update",
                    choices=["moe_8k_update", "moe_4k", "moe_16k_skew", "qwen3_4b_up"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-w4a8", action="store_true", help="skip the W4A8 (MXFP8 x MXFP4) side measurement")
    ap.add_argument("--no-nvfp4-backward", action="store_true", help="skip the NVFP4 backward side measurement")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense qwen3_4b_up W4A4 vs BF16 GEMM side measurement")
    ap.add_argument("--overlap", action="store_true",
                    help="weight-gradient GEMMs on a second stream (per-op times then overlap)")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short run for rocprofv3 --pmc: steps only, then a 1 GiB calibration copy")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="FETCH_SIZE and WRITE_SIZE run directories, optionally a GRBM_GUI_ACTIVE one")
    ap.add_argument("--kernel-stats-summary", metavar="DIR")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="per-op wave, load-path, L2 and LDS counters from several --pmc-run counter runs")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="per-op executed MFMA FLOPs and MFMA busy fraction from a --pmc-run counter run")
    ap.add_argument("--ab-run", action="store_true",
                    help="the gate+up GEMM run four ways (W4A4 A/B designs, W4A8, BF16), for rocprofv3")
    ap.add_argument("--ab-summary", nargs=2, metavar=("TRACE_DIR", "PMC_DIR"))
    ap.add_argument("--dispatch-summary", nargs=2, metavar=("DIR", "KERNEL"),
                    help="per-launch durations of one kernel in a kernel-trace run, by grid size")
    args = ap.parse_args()
    if args.ab_summary:
        ab_summary(*args.ab_summary)
        return
    if args.ab_run:
        ab_run(args)
        return
    if args.dispatch_summary:
        dispatch_summary(*args.dispatch_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.kernel_stats_summary:
        kernel_stats_summary(args.kernel_stats_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(sharding is described, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload == "qwen3_4b_up":
        bench_dense(args)
        return

    import torch
    from nvfp4_quantized_moe_token_amd import moe_layer, ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating", args.workload)
    inp = build_inputs(args.workload, torch, dev)
    d = inp["d"]
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    backward = args.workload == "moe_8k_update"

    # Expert weight quantization (each expert's amax and its NVFP4 encoding
    # from one read of the weights): once per optimizer step, outside the
    # step.  One untimed call, then the median of 5; bytes are one read of
    # the bf16 weights and one write of codes and scales.
    wq_gu = moe_layer.quantize_expert_weights(inp["w_gu"])
    wq_dn = moe_layer.quantize_expert_weights(inp["w_dn"])
    torch.cuda.synchronize()
    wq_times = []
    for _ in range(5):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        wq_gu = moe_layer.quantize_expert_weights(inp["w_gu"])
        wq_dn = moe_layer.quantize_expert_weights(inp["w_dn"])
        ev1.record()
        torch.cuda.synchronize()
        wq_times.append(ev0.elapsed_time(ev1))
    wq_ms = sorted(wq_times)[2]
    wq_bytes = (E * 2 * F * D + E * D * F) * (2 + 0.5625)

    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=backward)
    meta_box = {}
    seq = step_ops(ops, inp, wq_gu, wq_dn, buf, meta_box, backward)
    wstream = torch.cuda.Stream() if (args.overlap and backward) else None
    # Python's garbage collector is paused from here to the end of the timed
    # steps: a full collection in the middle of a step stalls the launching
    # thread for tens of milliseconds, and the GPU idles once it has drained
    # what was queued.  The collection that precedes the pause runs before
    # the warmup, so the GPU is back at its working clock when timing starts
    # (an idle gap just before the timed region cost ~3% in measurements).
    gc.collect()
    gc.disable()
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        run_step(torch, seq, wstream, False)
    torch.cuda.synchronize()

    if args.pmc_run:
        mark = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(args.steps):
            for i, (_, fn) in enumerate(seq):
                mark.fill_(i)
                fn()
            mark.fill_(len(seq))
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc run done")
        return

    # Timed steps; every op is bracketed by HIP events on its launch stream.
    log("timed steps", args.steps, "(weight gradients on a second stream)" if wstream is not None else "")
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        marks.append(run_step(torch, seq, wstream, True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    ms_per_step = wall * 1e3 / args.steps
    per_op = {}
    for evs in marks:
        for n, e0, e1 in evs:
            per_op.setdefault(n, []).append(e0.elapsed_time(e1))
    per_op = {n: sum(v) / len(v) for n, v in per_op.items()}

    # The same serial step captured once into a HIP graph and replayed as
    # many times: the launch gaps between its kernels shrink.  Reported beside
    # the eager step time, which the per-op events above belong to.
    graph_ms = None
    if wstream is None:
        gstream = torch.cuda.Stream()
        gstream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gstream):
            for _, fn in seq:
                fn()
        torch.cuda.current_stream().wait_stream(gstream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in seq:
                fn()
        gc.disable()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        gc.enable()

    # The plain W4A4 gate+up GEMM (bf16 Y1, no epilogue) and the BF16 grouped
    # GEMM on the same shape and routing, each timed alone; the latter and
    # the standalone quantize below read the bf16 X_perm, written here once
    # (the forward-only workloads do not keep it).
    offs = meta_box["m"]["offsets"]
    ops.moe_permute_nvfp4(inp["ids"], E, inp["x"], x_perm=buf.x_perm, want_x_perm=True, amax_out=buf.amax[0:1],
                          q=buf.a1_q, scales=buf.a1_s, gscale=buf.a1_g, workspace=buf.ws)
    y1w = torch.empty_like(buf.y1)
    y1b = torch.empty_like(buf.y1)
    side = {
        "w4a4_gate_up": lambda: ops.grouped_gemm_w4a4(buf.a1_q, buf.a1_s, buf.a1_g, wq_gu["q"], wq_gu["s"],
                                                      wq_gu["g"], offs, out=y1w),
        "bf16_nt_gate_up_baseline": lambda: ops.grouped_gemm_bf16(ops.NT, buf.x_perm, inp["w_gu"], offs, out=y1b),
        # the same W4A4 product by scale factoring onto the fp4 scaled MFMA
        "w4a4_gate_up_scaled_mfma": lambda: ops.grouped_gemm_w4a4_scaled_mfma(
            buf.a1_q, buf.a1_s, buf.a1_g, wq_gu["q"], wq_gu["s"], wq_gu["g"], offs, out=y1w),
    }
    per_op_extra = {}
    nrep = max(5, min(args.steps, 20))
    for name, fn in side.items():
        for _ in range(3):
            fn()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(nrep):
            fn()
        b1.record()
        torch.cuda.synchronize()
        per_op_extra[name] = b0.elapsed_time(b1) / nrep

    # Standalone NVFP4 quantize of the permuted activations (R x D bf16,
    # larger than the 256 MB Infinity Cache), cache flushed by a read of a
    # 512 MiB buffer before each repetition; median.  The flush runs on the
    # GPU while the quantize is enqueued, so the events see no launch gap.
    flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    qts = []
    for _ in range(7):
        torch.cuda.synchronize()
        flush.sum()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        ops.nvfp4_quantize(buf.x_perm, amax_in=buf.amax[0:1], q=buf.a1_q, scales=buf.a1_s, gscale=buf.a1_g)
        q1.record()
        torch.cuda.synchronize()
        qts.append(q0.elapsed_time(q1))
    per_op_extra["quantize_x_perm_cold"] = sorted(qts)[len(qts) // 2]
    # The same at the size of the 16384-token workload's X_perm (131072 x D),
    # on a seeded N(0,1) bf16 tensor: the size the quantizer's GB/s is quoted at.
    g16 = torch.Generator(device=dev)
    g16.manual_seed(0)
    x16 = torch.randn(16384 * k, D, device=dev, generator=g16).to(torch.bfloat16)
    a16 = x16.abs().amax().float().reshape(1)
    q16 = torch.empty(16384 * k, D // 2, dtype=torch.uint8, device=dev)
    s16 = torch.empty(16384 * k, D // 16, dtype=torch.uint8, device=dev)
    g16s = torch.empty(1, dtype=torch.float32, device=dev)
    qts = []
    for _ in range(7):
        torch.cuda.synchronize()
        flush.sum()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        ops.nvfp4_quantize(x16, amax_in=a16, q=q16, scales=s16, gscale=g16s)
        q1.record()
        torch.cuda.synchronize()
        qts.append(q0.elapsed_time(q1))
    del flush, x16, q16, s16
    per_op_extra["quantize_x_perm_16k_cold"] = sorted(qts)[len(qts) // 2]

    R = T * k
    f1, f2 = gemm_flops(R, D, F)
    step_flops = (f1 + f2) * (3 if backward else 1)
    tflops = step_flops / (ms_per_step * 1e-3) / 1e12
    # The committed counter summaries were taken on the moe_8k_update step;
    # other workloads get none of their fields.
    profiled = (T, k, E, D, F) == (8192, 8, 128, 2048, 768) and backward
    traffic = load_traffic() if profiled else {}
    mfma = load_mfma() if profiled else {}
    kernels = {}
    for name, ms in list(per_op.items()) + list(per_op_extra.items()):
        fl, by = op_work(name, T, k, E, D, F, backward)
        ent = {"ms": round(ms, 4)}
        if fl:
            ent["tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
            ent["frac_bf16_mfma_peak"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
            if name.startswith("w4a4"):
                ent["frac_fp4_mfma_peak"] = round(ent["tflops"] / PEAK_FP4_TFLOPS, 4)
        ent["gbs"] = round(by / (ms * 1e-3) / 1e9, 1)
        ent["frac_hbm_peak"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
        tr = traffic.get(name, {})
        if "fetch" in tr:
            ent["hbm_bytes_measured"] = tr["fetch"] + tr["write"]
            ent["hbm_bytes_algorithmic"] = by
        if "clock_ghz" in tr:
            ent["sustained_clock_ghz"] = tr["clock_ghz"]
            if fl:
                ent["frac_bf16_peak_at_sustained_clock"] = round(
                    ent["tflops"] / (PEAK_BF16_TFLOPS * tr["clock_ghz"] / PEAK_CLOCK_GHZ), 4)
        if name in mfma:
            # rocprofv3 counters (profiles/): MFMA FLOPs executed (padding
            # included) and the MFMA unit's busy fraction of SIMD cycles
            ent["mfma_executed_gflop_counter"] = mfma[name]["executed_gflop"]
            ent["mfma_busy_counter"] = mfma[name]["mfma_busy"]
        kernels[name] = ent

    def traffic_bytes(names):
        tr = [traffic.get(o, {}) for o in names]
        if not all("fetch" in t for t in tr):
            return None
        return round(sum(t["fetch"] + t["write"] for t in tr) / len(names))

    def clock_fields(names, ach):
        """Sustained clock of the ops (time-weighted) and the fraction of the
        bf16 MFMA peak scaled to that clock."""
        tr = [traffic.get(o, {}) for o in names]
        if not names or not all("clock_ghz" in t for t in tr):
            return {}
        w = [per_op.get(o, per_op_extra.get(o, 0.0)) for o in names]
        clk = sum(t["clock_ghz"] * wi for t, wi in zip(tr, w)) / sum(w)
        return {"sustained_clock_ghz": round(clk, 3),
                "frac_at_sustained_clock": round(ach / (PEAK_BF16_TFLOPS * clk / PEAK_CLOCK_GHZ), 4)}

    def roofline_of(name):
        ms = per_op[name] if name in per_op else per_op_extra[name]
        fl, by = op_work(name, T, k, E, D, F, backward)
        tr_bytes = traffic_bytes([name])
        if fl:
            ach = fl / (ms * 1e-3) / 1e12
            return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": tr_bytes,
                    "algorithmic_bytes": by, "ms": round(ms, 4), **clock_fields([name], ach)}
        ach = by / (ms * 1e-3) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": tr_bytes, "ms": round(ms, 4)}

    def roofline_of_kernel(kname):
        """Roofline of one kernel over its launches in a step: algorithmic
        work per launch / its average launch duration, both from the HIP
        events around its launches inside the timed steps (on the stream it
        runs on).  A GEMM is reported against the 16-bit MFMA peak -- the
        contraction it runs -- with its HBM rate beside it (`hbm_view`);
        its arithmetic intensity and the ridge point (bf16 MFMA peak / HBM
        peak) are given so the reader can see which ceiling is nearer."""
        names = [o for o in STEP_OPS if KERNEL_OF_OP.get(o) == kname and o in per_op]
        n = len(names)
        ms = sum(per_op[o] for o in names) / n
        fl = sum(op_work(o, T, k, E, D, F, backward)[0] for o in names) / n
        by = sum(op_work(o, T, k, E, D, F, backward)[1] for o in names) / n
        tfl = fl / (ms * 1e-3) / 1e12
        gbs = by / (ms * 1e-3) / 1e9
        tr = traffic_bytes(names)
        out = {"kernel": kname, "ops": names, "bound": "mfma", "achieved": round(tfl, 1),
               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tfl / PEAK_BF16_TFLOPS, 4),
               "traffic": tr, "traffic_source": os.path.relpath(TRAFFIC_FILE, ROOT) if tr is not None else None,
               "algorithmic_flops": round(fl), "algorithmic_bytes": round(by), "avg_launch_ms": round(ms, 4),
               "flop_per_byte": round(fl / by, 1), "ridge_flop_per_byte": round(RIDGE, 1),
               "hbm_view": {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4)},
               **clock_fields(names, tfl)}
        if all(o in mfma for o in names):
            # time-weighted MFMA busy fraction of the kernel's launches, from
            # the committed counter summary of the same kernel sources
            out["mfma_busy_counter"] = round(sum(mfma[o]["mfma_busy"] * per_op[o] for o in names) /
                                             sum(per_op[o] for o in names), 4)
            out["mfma_busy_source"] = os.path.relpath(MFMA_FILE, ROOT)
        return out

    # Dominant kernel: the largest share of the step's time.
    per_kernel = {}
    for o, ms in per_op.items():
        per_kernel[KERNEL_OF_OP.get(o, o)] = per_kernel.get(KERNEL_OF_OP.get(o, o), 0.0) + ms
    dominant = max(per_kernel, key=per_kernel.get)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()

    w4 = kernels["w4a4_gate_up"]
    bl = kernels["bf16_nt_gate_up_baseline"]
    # The metric: the W4A4 grouped GEMMs of the step (gate+up with its SiLU
    # epilogue, and down), their algorithmic FLOPs over their summed time.
    w4_ops = ["w4a4_gate_up_silu", "w4a4_down"]
    w4_ms = sum(per_op[o] for o in w4_ops)
    w4_tflops = (f1 + f2) / (w4_ms * 1e-3) / 1e12
    dense = dense_side(args) if not args.no_dense else None
    nvbwd = None
    if backward and not args.no_nvfp4_backward:
        log("nvfp4 backward variant")
        nvbwd = nvfp4_backward_side(torch, ops, moe_layer, inp, wq_gu, wq_dn, buf, meta_box, T, k, E, D, F, nrep)
        bwd_names = ["gather_dy", "bf16_nn_down", "silu_gate_bwd", "bf16_tn_down", "bf16_nn_gate_up",
                     "unpermute_dx", "bf16_tn_gate_up"]
        nvbwd["bf16_backward_ms_in_step"] = round(sum(per_op[n] for n in bwd_names), 4)
        nvbwd["bf16_backward_gemm_ms_in_step"] = round(sum(per_op[n] for n in bwd_names if n.startswith("bf16_")), 4)
    log("delayed amax of H")
    delayed = delayed_amax_side(torch, ops, moe_layer, inp, wq_gu, wq_dn, T, k, E, D, F, nrep, backward)
    fwd_names = ["permute_quantize_x", "w4a4_gate_up_silu", "quantize_h", "w4a4_down", "unpermute"]
    delayed["forward_ms_amax_computed"] = round(sum(per_op[n] for n in fwd_names), 4)
    w4a8 = None
    if not args.no_w4a8:
        log("w4a8 variant")
        w4a8 = w4a8_side(torch, ops, moe_layer, inp, T, k, E, D, F, nrep)
        w4a8["speedup_gate_up_vs_w4a4"] = round(w4["ms"] / w4a8["ops"]["w4a8_gate_up"]["ms"], 3)
        w4a8["speedup_gate_up_vs_bf16"] = round(bl["ms"] / w4a8["ops"]["w4a8_gate_up"]["ms"], 3)
        w4a8["speedup_gemms_vs_w4a4_in_step"] = round(w4_ms / w4a8["gemm_ms"], 3)
    res = {
        "metric": "W4A4 MoE grouped-GEMM TFLOP/s + % MI355X MFMA peak; quantize GB/s",
        "value": round(w4_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16+bf16 mfma, fp32 acc" if backward else "fp16 mfma, fp32 acc",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "d_model": D, "experts": E, "top_k": k, "ffn": F,
                   "step": "fwd W4A4 + bwd BF16" if backward else "fwd W4A4", "parallelism": "none (1 GPU)",
                   "wgrad_stream": wstream is not None},
        "value_definition": "W4A4 grouped GEMMs of the step (gate+up with the SiLU-gate epilogue, and down): "
                            "%.1f GFLOP over their summed in-step time, HIP events" % ((f1 + f2) / 1e9),
        "w4a4_in_step": {"ops": w4_ops, "ms": round(w4_ms, 4), "tflops": round(w4_tflops, 1),
                         "frac_bf16_mfma_peak": round(w4_tflops / PEAK_BF16_TFLOPS, 4),
                         "frac_fp4_mfma_peak": round(w4_tflops / PEAK_FP4_TFLOPS, 4)},
        "step": {"ms": round(ms_per_step, 4), "gflop": round(step_flops / 1e9, 1), "tflops": round(tflops, 2),
                 "frac_bf16_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                 "tokens_per_s": round(T / (ms_per_step * 1e-3), 1)},
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 4), "tflops": round(step_flops / (graph_ms * 1e-3) / 1e12, 2),
            "tokens_per_s": round(T / (graph_ms * 1e-3), 1)},
        "roofline": roofline_of_kernel(dominant) if dominant in KERNEL_OF_OP.values() else roofline_of(dominant),
        "w4a4_gemm": {**roofline_of("w4a4_gate_up"), "frac_fp4_peak": w4.get("frac_fp4_mfma_peak"),
                      "bf16_same_shape_tflops": bl.get("tflops"),
                      "speedup_vs_bf16": round(bl["ms"] / w4["ms"], 3),
                      "scaled_mfma_design_tflops": kernels["w4a4_gate_up_scaled_mfma"].get("tflops"),
                      "speedup_vs_scaled_mfma_design": round(kernels["w4a4_gate_up_scaled_mfma"]["ms"] / w4["ms"], 3)},
        "dense_qwen3_4b_up": dense,
        "w4a8": w4a8,
        "forward_delayed_amax_h": delayed,
        "nvfp4_backward": nvbwd,
        "quantize": dict(roofline_of("quantize_x_perm_cold"), amax="reused (amax_in from the permute)"),
        "quantize_16k": dict(roofline_of("quantize_x_perm_16k_cold"), amax="reused (amax_in)"),
        "permute_quantize": dict(roofline_of("permute_quantize_x"), amax="computed (fused into the metadata pass)"),
        "cpu_baseline": cpu,
        "kernels": kernels,
        "weight_quantize": {"ms": round(wq_ms, 4), "gbs": round(wq_bytes / (wq_ms * 1e-3) / 1e9, 1),
                            "kernel": "nvfp4_quantize_onepass (per-expert amax and encoding from one read)",
                            "note": "both projections; gbs: one read of the bf16 weights + NVFP4 codes and "
                                    "scales written"},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
