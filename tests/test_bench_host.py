"""Host-side logic of bench.py that needs no GPU: the rocprofv3 summaries
(kernel statistics, per-launch durations, PMC traffic per op) read from
small synthetic CSV files, and the refusal of more than one GPU."""

import csv
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_dispatch_summary_groups_by_grid(tmp_path, capsys):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    k = "void nvfp4moe::quantize_kernel<256, true>(HIP_vector_type<unsigned int, 4u> const*, long)"
    rows = [[k, 0, 10000, 256, 1, 1], [k, 0, 30000, 256, 1, 1], [k, 0, 20000, 256, 1, 1],
            [k, 0, 50000, 1024, 1, 1], ["other_kernel(int)", 0, 99000, 256, 1, 1]]
    _write(str(tmp_path / "run" / "kt_kernel_trace.csv"), hdr, rows)
    bench.dispatch_summary(str(tmp_path), "quantize_kernel")
    out = [l for l in capsys.readouterr().out.splitlines() if not l.startswith(("#", "sources "))]
    assert len(out) == 3                                    # header + two grid sizes
    first = out[1].split()
    assert first[0] == "quantize_kernel<256,true>" and first[1] == "256" and first[2] == "3"
    assert float(first[3]) == 20.0 and float(first[4]) == 10.0 and float(first[5]) == 30.0
    assert out[2].split()[1] == "1024" and float(out[2].split()[3]) == 50.0


def test_kernel_stats_summary_sorts_by_total(tmp_path, capsys):
    hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"]
    _write(str(tmp_path / "kt_kernel_stats.csv"), hdr,
           [["small", 2, 2000, 1000, 900, 1100, 10.0], ["big", 1, 18000, 18000, 18000, 18000, 90.0]])
    bench.kernel_stats_summary(str(tmp_path))
    lines = capsys.readouterr().out.splitlines()
    assert any(l.startswith("# command") for l in lines)           # names the command that made it
    assert ("sources " + bench.source_digest()) in lines
    out = [l for l in lines if not l.startswith(("#", "sources "))]
    assert out[1].split()[0] == "big" and out[2].split()[0] == "small"
    assert float(out[1].split()[3]) == 18.0


def _pmc_rows(counter, per_op, calib_kib):
    """One step: a marker before every op and after the last, each op one
    dispatch of per_op[op] KiB, then the calibration copy."""
    rows, i = [], 0
    for _ in range(2):                                       # an earlier step is ignored
        for name in bench.STEP_OPS:
            rows.append([i, "void at::native::FillFunctor<int>", counter, 0.0, 0, 1]); i += 1
            rows.append([i, "kernel_of_" + name, counter, per_op[name], 0, 1000]); i += 1
        rows.append([i, "void at::native::FillFunctor<int>", counter, 0.0, 0, 1]); i += 1
    rows.append([i, "copy_kernel", counter, calib_kib, 0, 1]); i += 1
    return rows


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path, capsys):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    fetch = {n: 100.0 * (j + 1) for j, n in enumerate(bench.STEP_OPS)}
    write = {n: 10.0 * (j + 1) for j, n in enumerate(bench.STEP_OPS)}
    # the copy's fetch counter reads half its bytes, its write counter all of them
    _write(str(tmp_path / "f" / "run_counter_collection.csv"), hdr,
           _pmc_rows("FETCH_SIZE", fetch, bench.CALIB_BYTES / 1024 / 2))
    _write(str(tmp_path / "w" / "run_counter_collection.csv"), hdr,
           _pmc_rows("WRITE_SIZE", write, bench.CALIB_BYTES / 1024))
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"))
    ops = {}
    for line in capsys.readouterr().out.splitlines():
        parts = line.split()
        if parts and parts[0] == "op":
            ops[parts[1]] = (float(parts[3]), float(parts[5]), parts[7])
    assert list(ops) == bench.STEP_OPS
    for j, n in enumerate(bench.STEP_OPS):
        f, w, kn = ops[n]
        assert f == pytest.approx(2 * 1024 * 100.0 * (j + 1)) and w == pytest.approx(1024 * 10.0 * (j + 1))
        assert kn == "kernel_of_" + n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_mfma_summary_counts_executed_flops(tmp_path, capsys):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows, i = [], 0
    T, k, E, D, F = 8192, 8, 128, 2048, 768
    for name in bench.STEP_OPS:
        rows.append([i, "void at::native::FillFunctor<int>", "GRBM_GUI_ACTIVE", 0.0, 0, 1]); i += 1
        alg = bench.op_work(name, T, k, E, D, F)[0]
        if alg:
            # executed = algorithmic + 10%, over 1 ms; MFMA busy half of 1000 cycles on every SIMD
            for cn, v in (("SQ_INSTS_VALU_MFMA_MOPS_F16", alg * 1.1 / 512), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0),
                          ("SQ_VALU_MFMA_BUSY_CYCLES", 500.0 * 1024), ("GRBM_GUI_ACTIVE", 1000.0 * 8)):
                rows.append([i, "gemm_" + name, cn, v, 0, 1_000_000])
            i += 1
        else:
            rows.append([i, "elementwise_" + name, "SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0, 0, 1000]); i += 1
    rows.append([i, "void at::native::FillFunctor<int>", "GRBM_GUI_ACTIVE", 0.0, 0, 1])
    _write(str(tmp_path / "m" / "run_counter_collection.csv"), hdr, rows)
    bench.mfma_summary(str(tmp_path / "m"))
    ops = [l.split() for l in capsys.readouterr().out.splitlines() if l and not l.startswith(("#", "sources", "op "))]
    gemm_ops = [n for n in bench.STEP_OPS if bench.op_work(n, T, k, E, D, F)[0]]
    assert [o[0] for o in ops] == gemm_ops
    for o in ops:
        assert float(o[3]) == pytest.approx(1.1, abs=1e-3)      # executed / algorithmic
        assert float(o[4]) == pytest.approx(1000.0)             # us
        assert o[7] == "50.0%"                                  # MFMA busy


def test_committed_mfma_summary_parses():
    """The committed MFMA summary lists the step's GEMM ops with their busy
    fractions; load_mfma returns them when the sources fingerprint matches."""
    path = os.path.join(ROOT, "profiles", "mfma_moe_8k_update.txt")
    lines = open(path).read().splitlines()
    assert any(l.startswith("sources ") for l in lines)
    rows = [l.split() for l in lines if l.split() and l.split()[0] in bench.STEP_OPS]
    assert {r[0] for r in rows} >= {"w4a4_gate_up_silu", "w4a4_down", "bf16_tn_gate_up", "bf16_nn_gate_up"}
    for r in rows:
        assert 0.0 < float(r[7].rstrip("%")) < 100.0
        assert 1.0 <= float(r[3]) < 1.2                 # executed / algorithmic: padding only
    m = bench.load_mfma()
    assert m == {} or set(m) == {r[0] for r in rows}
