"""bench.py's contract on the CPU: a run on more than one GPU is refused with
a message (before anything touches a GPU), and the CPU baseline -- the oracle
timed on a bounded sample of the step -- reports the fields the result line
carries."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_fields():
    import bench
    import workloads as W
    from oracle import banded
    cb = bench.cpu_baseline(np, W, rows=256)
    assert {"value", "unit", "cores", "kind", "sample", "single_core_value", "cpu_model"} <= set(cb)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] == banded.default_threads()
    assert cb["value"] > 0 and cb["single_core_value"] > 0 and "rows 0..255" in cb["sample"]
    assert "identical outputs" in cb["sample"]


def test_profile_figures_follow_the_kernel_sources(tmp_path, monkeypatch):
    """A counter figure is reported only while the kernel sources hash to
    the value stored with it; otherwise, or without the file, it is None."""
    import json
    import bench
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "valu.json").write_text(json.dumps(
        {"kernels": {"quant_row_sr": {"valu_issue_share": 0.8, "valu_lane_instr_per_launch": 1_572_864_000,
                                      "source_hash": "abc"}}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "abc")
    assert bench.valu_issue_share_for("quant_row_sr") == 0.8
    assert bench.valu_issue_share_for("quant_col_sr") is None
    assert bench.traffic_for("quant_row_sr") is None  # no traffic.json here
    # VALU view: 1.572864e9 lane-instructions in 0.05 ms = 31.46 T/s of the 39.32 T/s issue peak
    v = bench.valu_view("quant_row_sr", 0.05)
    assert v["achieved"] == 31.46 and v["peak"] == 39.32 and abs(v["frac"] - 0.8) < 1e-3
    assert bench.valu_view("quant_col_sr", 0.05) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "def")
    assert bench.valu_issue_share_for("quant_row_sr") is None
    assert bench.valu_view("quant_row_sr", 0.05) is None
