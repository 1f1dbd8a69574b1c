"""The benchmark's contract: one JSON line with the required fields, measured
on one GPU.

CPU: a request for more than one GPU exits with a message before touching a
GPU; the algorithmic bytes per call are the ones the method moves (read the
bf16 row, write one code byte, or half a byte for E2M1, per element and one
scale byte per 32-element block; the two-pass path also writes and reads its
bf16 intermediate). GPU: a short run prints one line whose fields are
consistent with each other.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_per_call():
    T, D = 8192, 4096
    # read 2D bytes, write D codes and D/32 scales per row: 3.03125 D
    assert bench.fused_bytes(T, D) == 101_711_872 == int(T * D * 3.03125)
    assert bench.fused_bytes(T, D, "e2m1") == int(T * D * 2.53125)
    # RMSNorm reads x, writes y; MXCast reads y, writes codes and scales: 7.03125 D
    assert bench.two_pass_bytes(T, D) == 235_929_600 == int(T * D * 7.03125)


@pytest.mark.gpu
def test_short_run_prints_one_consistent_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "30",
                        "--warmup", "5", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 30 and d["warmup"] == 5
    assert d["config"]["workload"] == "llama3_8b_preattn"
    nbytes = d["config"]["algorithmic_bytes_per_step"]
    assert nbytes == bench.fused_bytes(8192, 4096)
    # value is the whole-job GB/s of the timed steps
    assert abs(d["value"] - nbytes / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.2 < rf["frac"] < 1.0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
