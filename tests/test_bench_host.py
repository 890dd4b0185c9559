"""Host logic of bench.py, without a GPU: the one-GPU guard, the roofline
arithmetic, and the CPU-baseline leg (the oracle) on a small workload."""
import os
import subprocess
import sys

import pytest

import synth
import transformer_lm_pretraining_train_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_lm_head_roofline_arithmetic():
    cfg = g.config_for(synth.workload("gpt2_124m"))
    r = bench.lm_head_roofline(cfg, 4, 4 * 1.5)  # four launches of 1.5 ms
    M, N, K = 16384, 50304, 768
    assert r["achieved"] == pytest.approx(2 * M * N * K / 1.5e-3 / 1e12, rel=1e-4)
    assert r["peak"] == 2516.6 and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["avg_launch_us"] == 1500.0 and r["launches_timed"] == 4
    assert r["algorithmic_bytes"] == 2 * (M * K + N * K + M * N)
    if r["traffic"] is not None:  # counters taken on this GEMM source
        assert r["traffic"] > r["algorithmic_bytes"]


def test_cpu_baseline_reports_the_oracle():
    c = bench.cpu_baseline(synth.workload("tiny"), 1)
    assert c["kind"] == "oracle" and c["unit"] == "tokens/s"
    assert c["value"] > 0 and c["cores"] >= 1 and c["sample"].startswith("tiny:")
