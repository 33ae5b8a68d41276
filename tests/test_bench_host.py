"""Host-side logic of bench.py (no GPU): the counter summaries built from
rocprofv3 --pmc output, and the one-GPU guard."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_pmc(d, rows, trace=()):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(trace)


def test_traffic_from_divides_by_the_copy_calibration(tmp_path):
    kib = bench.COPY_BYTES / 1024
    fwd = "void mz::fwd_mfma_kernel<mz::BF16, 128, 2, 1>(mz::FwdParams)"
    rot = "void mz::k_rotate16_kernel<mz::BF16, false>(mz::FwdParams)"
    # the copy reads half its bytes on FETCH_SIZE, all of them on WRITE_SIZE
    _write_pmc(tmp_path / "f", [["__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2],
                                [fwd, "FETCH_SIZE", 1000.0], [fwd, "FETCH_SIZE", 3000.0],
                                [rot, "FETCH_SIZE", 500.0]])
    _write_pmc(tmp_path / "w", [["__amd_rocclr_copyBuffer", "WRITE_SIZE", kib],
                                [fwd, "WRITE_SIZE", 10.0], [rot, "WRITE_SIZE", 20.0]])
    out = bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))
    assert out["fetch_size_factor"] == 0.5 and out["write_size_factor"] == 1.0
    assert out["fwd_mfma_kernel"]["fetch_size_bytes"] == 2000 * 1024 * 2
    assert out["fwd_mfma_kernel"]["write_size_bytes"] == 10 * 1024
    assert out["fwd_mfma_kernel"]["bytes"] == 2000 * 1024 * 2 + 10 * 1024
    assert out["k_rotate16_kernel"]["bytes"] == 500 * 1024 * 2 + 20 * 1024
    assert "decode_mfma_kernel" not in out


def test_traffic_from_needs_the_copy_kernel(tmp_path):
    _write_pmc(tmp_path / "f", [["mz::fwd_mfma_kernel", "FETCH_SIZE", 1.0]])
    _write_pmc(tmp_path / "w", [["mz::fwd_mfma_kernel", "WRITE_SIZE", 1.0]])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))


def test_counters_from_derived_figures(tmp_path):
    fwd = "void mz::fwd_mfma_kernel<mz::BF16, 128, 2, 1>(mz::FwdParams)"
    gui_per_xcd = 100_000.0
    rows = [
        # two dispatches: means are taken per counter
        [fwd, "GRBM_GUI_ACTIVE", gui_per_xcd * bench.XCDS],
        [fwd, "GRBM_GUI_ACTIVE", gui_per_xcd * bench.XCDS],
        [fwd, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * gui_per_xcd * bench.SIMDS],
        [fwd, "SQ_VALU_MFMA_BUSY_CYCLES", 0.35 * gui_per_xcd * bench.SIMDS],
        [fwd, "SQ_LDS_IDX_ACTIVE", 1000.0], [fwd, "SQ_LDS_IDX_ACTIVE", 1000.0],
        [fwd, "SQ_LDS_BANK_CONFLICT", 10.0], [fwd, "SQ_LDS_BANK_CONFLICT", 30.0],
        [fwd, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6], [fwd, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6],
    ]
    trace = [[fwd, 0, 40_000], [fwd, 100_000, 160_000]]  # 50 us mean
    _write_pmc(tmp_path / "c", rows, trace)
    e = bench.counters_from(str(tmp_path / "c"))["fwd_mfma_kernel"]
    assert e["dispatches"] == 2
    assert e["mfma_busy_pct"] == pytest.approx(30.0)
    assert e["lds_bank_conflict_pct"] == pytest.approx(2.0)
    assert e["mfma_gflop"] == pytest.approx(1e6 * 512 / 1e9, abs=1e-3)
    assert e["avg_duration_us"] == pytest.approx(50.0)
    assert e["gui_cycles_per_ns"] == pytest.approx(gui_per_xcd / 50_000, abs=1e-3)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
