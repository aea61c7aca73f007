"""bench.py --summarize on fabricated rocprofv3 CSVs (no GPU): GEMM
dispatches are matched to shapes through the launch log, warm-up calls are
dropped, casts and copies are ignored, and HBM bytes are the counters scaled
by the plain-copy calibration."""

from __future__ import annotations

import csv
import json
import os

import pytest

import bench

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
              "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
CTR_COLS = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
K0 = "void fg::gemm_fp8_big_kernel<fg::BigCfg<256, 256, 4, 2>, 2, false>(fg::GemmParams)"
K1 = "void fg::gemm_fp8_big_kernel<fg::BigCfg<256, 224, 4, 2>, 2, false>(fg::GemmParams)"
CAST = "void fg::cast_per_token_kernel<false, float, 8>(float const*, long)"


def _write_trace(d, seq):
    """seq: list of (kernel, duration_ns); writes the trace CSV."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(TRACE_COLS)
        t = 1000
        for i, (k, dur) in enumerate(seq, 1):
            w.writerow(["KERNEL_DISPATCH", "Agent 1", 1, i, k, t, t + dur, 256, 1, 1])
            t += dur + 500


def _write_ctr(d, seq, name):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(CTR_COLS)
        for i, (k, v) in enumerate(seq, 1):
            w.writerow([i, i, 256, k, name, v, 0, 1000])


def test_summary_matches_dispatches_to_shapes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "prof"
    # log: 1 warm step, a warm per-shape block, then timed calls in per-shape blocks
    log = [(0, "warm"), (1, "warm"), (0, "warm"), (0, "timed"), (0, "timed"), (1, "timed"), (1, "timed"), (1, "timed")]
    durs = {0: 100_000, 1: 60_000}
    kern = {0: K0, 1: K1}
    gemm = [(kern[i], durs[i] if ph == "timed" else 999_000) for i, ph in log]
    _write_trace(d / "trace", [(CAST, 5000)] + gemm)
    (d / "trace" / "launch_log.json").write_text(json.dumps(log))
    fetch = {0: 200_000.0, 1: 100_000.0}  # KiB
    write = {0: 1000.0, 1: 3000.0}
    for key, name, val in (("fetch", "FETCH_SIZE", fetch), ("write", "WRITE_SIZE", write)):
        _write_ctr(d / key, [(CAST, 1.0)] + [(kern[i], val[i] if ph == "timed" else 9e9) for i, ph in log], name)
        (d / key / "launch_log.json").write_text(json.dumps(log))
    copy = "__amd_rocclr_copyBuffer"
    _write_ctr(d / "copyf", [(copy, (1 << 30) / 1024 / 2.0), (copy, 10.0)], "FETCH_SIZE")
    _write_ctr(d / "copyw", [(copy, (1 << 30) / 1024)], "WRITE_SIZE")
    bench.summarize(str(d), "masked_16x256", 20)
    tj = json.loads((tmp_path / "profiles" / "masked_16x256_traffic.json").read_text())
    assert tj["calibration"]["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert tj["calibration"]["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    s0, s1 = tj["per_shape"]
    assert s0["avg_us"] == pytest.approx(100.0) and s1["avg_us"] == pytest.approx(60.0)
    assert s0["fetch_bytes"] == int(200_000 * 1024 * 2.0) and s1["write_bytes"] == int(3000 * 1024)
    assert tj["hbm_bytes_per_launch"] == int((s0["hbm_bytes"] + s1["hbm_bytes"]) / 2)
    assert "K1" not in s0["kernel"] and "256, 224" in s1["kernel"]
    md = (tmp_path / "profiles" / "masked_16x256_summary.md").read_text()
    assert "16x256x4096x7168" in md and "16x256x7168x2048" in md


def test_summary_rejects_a_log_that_does_not_match(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "prof"
    _write_trace(d / "trace", [(K0, 100)] * 3)
    (d / "trace" / "launch_log.json").write_text(json.dumps([[0, "timed"]] * 2))
    with pytest.raises(SystemExit, match="logged GEMM calls"):
        bench.summarize(str(d), "masked_16x256", 20)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU only: --gpus 2, or a launcher's WORLD_SIZE of
    2, ends with a message before any device work."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           timeout=300, env=dict(os.environ, **env), cwd=root)
        assert r.returncode != 0
        assert "one GPU" in r.stdout
