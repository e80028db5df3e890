"""Benchmark of the NVFP4 token-wise MoE hot path on one MI355X.

A step is one pass of the whole path over one batch: the MoE layer forward
on the NVFP4 token-wise path (permute + amax, quantize, grouped W4A4 GEMM
gate+up, SiLU gate + amax, requantize, grouped W4A4 GEMM down, unpermute)
followed by its BF16 backward (weighted gather, grouped NN/TN GEMMs for both
projections, SiLU-gate backward, unpermute).  Default workload: the
Qwen3-30B-A3B-shaped full update at 8192 tokens (d_model 2048, 128 experts,
top-8, FFN 768), synthetic seeded inputs, inputs resident in HBM.  Expert
weight quantization runs once per optimizer step and is timed separately.

Prints one JSON line (rank 0, N = 1).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16/fp16 MFMA, 256 CU x 2.4 GHz
PEAK_FP4_TFLOPS = 10066.0   # dense fp4 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemm_flops(R, D, F):
    """Algorithmic FLOPs of the two expert projections for R routed rows."""
    return 2.0 * R * (2 * F) * D, 2.0 * R * D * F


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


class Timeline:
    """Per-op HIP events on the current stream (the stream the ops launch on)."""

    def __init__(self, torch, enabled):
        self.torch, self.enabled, self.ev = torch, enabled, []

    def mark(self, name):
        if not self.enabled:
            return None
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.ev.append((name, e))
        return e

    def durations(self):
        out = {}
        for (n0, e0), (n1, e1) in zip(self.ev[:-1], self.ev[1:]):
            if n0 == "__end__":
                continue
            out.setdefault(n0, []).append(e0.elapsed_time(e1))
        return out


def run_step(torch, ops, inp, wq_gu, wq_dn, buf, tl, backward=True):
    E = buf.E
    tl.mark("moe_permute")
    meta = ops.moe_permute(inp["ids"], E, x=inp["x"], x_perm=buf.x_perm, amax_out=buf.amax[0:1], workspace=buf.ws)
    tl.mark("quantize_x")
    ops.nvfp4_quantize(buf.x_perm, amax_in=buf.amax[0:1], q=buf.a1_q, scales=buf.a1_s, gscale=buf.a1_g)
    tl.mark("w4a4_gate_up")
    ops.grouped_gemm_w4a4(buf.a1_q, buf.a1_s, buf.a1_g, wq_gu["q"], wq_gu["s"], wq_gu["g"], meta["offsets"],
                          out=buf.y1)
    tl.mark("silu_gate_fwd")
    ops.silu_gate_fwd(buf.y1, h=buf.h, amax_out=buf.amax[1:2])
    tl.mark("quantize_h")
    ops.nvfp4_quantize(buf.h, amax_in=buf.amax[1:2], q=buf.a2_q, scales=buf.a2_s, gscale=buf.a2_g)
    tl.mark("w4a4_down")
    ops.grouped_gemm_w4a4(buf.a2_q, buf.a2_s, buf.a2_g, wq_dn["q"], wq_dn["s"], wq_dn["g"], meta["offsets"],
                          out=buf.y2)
    tl.mark("unpermute")
    ops.moe_unpermute(buf.y2, meta["dest"], buf.T, buf.k, topk_w=inp["tw"], out=buf.out)
    if backward:
        off = meta["offsets"]
        tl.mark("gather_dy")
        ops.moe_gather(inp["dy"], meta["src"], buf.k, topk_w=inp["tw"], out=buf.dy2)
        tl.mark("bf16_nn_down")
        ops.grouped_gemm_bf16(ops.NN, buf.dy2, inp["w_dn"], off, out=buf.dh)
        tl.mark("bf16_tn_down")
        ops.grouped_gemm_bf16(ops.TN, buf.dy2, buf.h, off, out=buf.dw_dn)
        tl.mark("silu_gate_bwd")
        ops.silu_gate_bwd(buf.y1, buf.dh, dy1=buf.dy1)
        tl.mark("bf16_nn_gate_up")
        ops.grouped_gemm_bf16(ops.NN, buf.dy1, inp["w_gu"], off, out=buf.dx_perm)
        tl.mark("bf16_tn_gate_up")
        ops.grouped_gemm_bf16(ops.TN, buf.dy1, buf.x_perm, off, out=buf.dw_gu)
        tl.mark("unpermute_dx")
        ops.moe_unpermute(buf.dx_perm, meta["dest"], buf.T, buf.k, topk_w=None, out=buf.dx)
    tl.mark("__end__")
    return meta


def kernel_work(name, T, k, D, F):
    """(flops, algorithmic bytes) of one launch of each op of the step."""
    R = T * k
    f1, f2 = gemm_flops(R, D, F)
    nv = lambda rows, cols: rows * cols * (0.5 + 1.0 / 16)  # noqa: E731  NVFP4 bytes
    table = {
        # metadata + gather (bf16 rows read once per assignment, written once)
        "moe_permute": (0.0, R * D * 2 * 2 + R * 4 * 3),
        "quantize_x": (0.0, R * D * 2 + nv(R, D)),
        "w4a4_gate_up": (f1, nv(R, D) + nv(128 * 2 * F, D) + R * 2 * F * 2),
        "silu_gate_fwd": (0.0, R * 2 * F * 2 + R * F * 2),
        "quantize_h": (0.0, R * F * 2 + nv(R, F)),
        "w4a4_down": (f2, nv(R, F) + nv(128 * D, F) + R * D * 2),
        "unpermute": (0.0, R * D * 2 + T * D * 2),
        "gather_dy": (0.0, R * D * 2 + R * D * 2),
        "bf16_nn_down": (f2, R * D * 2 + 128 * D * F * 2 + R * F * 2),
        "bf16_tn_down": (f2, R * D * 2 + R * F * 2 + 128 * D * F * 4),
        "silu_gate_bwd": (0.0, R * 2 * F * 2 + R * F * 2 + R * 2 * F * 2),
        "bf16_nn_gate_up": (f1, R * 2 * F * 2 + 128 * 2 * F * D * 2 + R * D * 2),
        "bf16_tn_gate_up": (f1, R * 2 * F * 2 + R * D * 2 + 128 * 2 * F * D * 4),
        "unpermute_dx": (0.0, R * D * 2 + T * D * 2),
    }
    return table[name]


def cpu_baseline(seconds_hint=True):
    """The oracle, as it stands, on a bounded sample of the same workload:
    512 tokens routed top-8 over 8 experts (every expert gets 512 rows, the
    per-expert GEMM shape of the full update), forward + BF16 backward.
    Expert weight quantization happens before the timer, as on the GPU."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    T, k, E, D, F = 512, 8, 8, 2048, 768
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
                sample="forward+backward of 512 tokens x top-8 over 8 experts (512 rows per expert), "
                       "d_model 2048, FFN 768; %.1f s" % dt, seconds=round(dt, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe_8k_update",
                    choices=["moe_8k_update", "moe_4k", "moe_16k_skew"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true", help="skip per-op HIP events (for profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(sharding is described, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from nvfp4_quantized_moe_token_amd import moe_layer, ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating", args.workload)
    inp = build_inputs(args.workload, torch, dev)
    d = inp["d"]
    T, k, E, D, F = d["T"], d["k"], d["E"], d["D"], d["F"]
    backward = args.workload == "moe_8k_update"

    # Expert weight quantization: once per optimizer step, outside the step.
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    wq_gu = moe_layer.quantize_expert_weights(inp["w_gu"])
    wq_dn = moe_layer.quantize_expert_weights(inp["w_dn"])
    ev1.record()
    torch.cuda.synchronize()
    wq_ms = ev0.elapsed_time(ev1)
    wq_bytes = (E * 2 * F * D + E * D * F) * (2 + 0.5625)

    buf = moe_layer.Buffers(T, k, E, D, F, dev, backward=backward)
    off_tl = Timeline(torch, False)
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        run_step(torch, ops, inp, wq_gu, wq_dn, buf, off_tl, backward)
    torch.cuda.synchronize()

    log("timed steps", args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(torch, ops, inp, wq_gu, wq_dn, buf, off_tl, backward)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-op durations from HIP events in separate instrumented steps.
    per_op = {}
    if not args.no_events:
        tl = Timeline(torch, True)
        for _ in range(max(3, min(args.steps, 10))):
            run_step(torch, ops, inp, wq_gu, wq_dn, buf, tl, backward)
        torch.cuda.synchronize()
        for name, v in tl.durations().items():
            per_op[name] = sum(v) / len(v)

    R = T * k
    f1, f2 = gemm_flops(R, D, F)
    step_flops = (f1 + f2) * (3 if backward else 1)
    tflops = step_flops / (ms_per_step * 1e-3) / 1e12
    kernels = {}
    for name, ms in per_op.items():
        fl, by = kernel_work(name, T, k, D, F)
        ent = {"ms": round(ms, 4)}
        if fl:
            ent["tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
            ent["frac_bf16_mfma_peak"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
            if name.startswith("w4a4"):
                ent["frac_fp4_mfma_peak"] = round(ent["tflops"] / PEAK_FP4_TFLOPS, 4)
        ent["gbs"] = round(by / (ms * 1e-3) / 1e9, 1)
        ent["frac_hbm_peak"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = ent

    roofline = None
    if per_op:
        dom = max(per_op, key=per_op.get)
        fl, by = kernel_work(dom, T, k, D, F)
        if fl:
            ach = fl / (per_op[dom] * 1e-3) / 1e12
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
        else:
            ach = by / (per_op[dom] * 1e-3) / 1e9
            roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()

    res = {
        "metric": "W4A4 MoE grouped-GEMM TFLOP/s + % MI355X MFMA peak; quantize GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4-w4a4 fwd (fp16 MFMA, fp32 acc) + bf16 bwd" if backward else "nvfp4-w4a4 (fp16 MFMA, fp32 acc)",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "d_model": D, "experts": E, "top_k": k, "ffn": F,
                   "step": "fwd W4A4 + bwd BF16" if backward else "fwd W4A4", "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "step_gflop": round(step_flops / 1e9, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "weight_quantize": {"ms": round(wq_ms, 4), "gbs": round(wq_bytes / (wq_ms * 1e-3) / 1e9, 1)},
    }
    if "w4a4_gate_up" in kernels:
        res["w4a4_gemm_tflops"] = kernels["w4a4_gate_up"].get("tflops")
    if "quantize_x" in kernels:
        res["quantize_gbs"] = kernels["quantize_x"]["gbs"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
