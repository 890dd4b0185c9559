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


def test_wgrad_roofline_arithmetic():
    """Two GPT-2 124M layers' weight gradients per launch (12 layers, six
    launches per micro-step): 2 x 2 x 16384 x 12 x 768^2 = 463.9 GFLOP per
    launch; bytes: the bf16 operands (16 C columns per token per layer) and
    the fp32 gradients read and written.  350M: one layer per launch."""
    cfg = g.config_for(synth.workload("gpt2_124m"))
    r = bench.wgrad_roofline(cfg, 12, 12 * 0.5, 2)  # two micro-steps, twelve launches of 0.5 ms
    M, C = 16384, 768
    flops = 2 * 2 * M * 12 * C * C
    assert r["flops_per_launch"] == flops and abs(flops - 463.9e9) < 0.1e9
    assert r["achieved"] == pytest.approx(flops / 0.5e-3 / 1e12, rel=1e-4)
    assert r["peak"] == 2516.6 and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["avg_launch_us"] == 500.0 and r["launches_timed"] == 12
    assert r["algorithmic_bytes"] == 2 * (2 * M * 16 * C + 8 * 12 * C * C)
    if r["traffic"] is not None:  # counters taken on this GEMM source
        assert r["traffic"] > 0
    c350 = g.config_for(synth.workload("gpt2_350m"))
    r = bench.wgrad_roofline(c350, 48, 48 * 0.5, 2)  # 24 layers, one per launch
    assert r["flops_per_launch"] == 2 * 16384 * 12 * 1024 ** 2 and r["traffic"] is None


def test_other_kernels_arithmetic():
    cfg = g.config_for(synth.workload("gpt2_124m"))
    o = bench.other_kernels(cfg, {"ln_fwd": (25, 25 * 0.010), "lm_head_fwd": (1, 1.2)})
    M, C = 16384, 768
    assert o["ln_fwd"]["bytes_per_launch"] == (4 * C + 8) * M
    assert o["ln_fwd"]["achieved"] == pytest.approx((4 * C + 8) * M / 10e-6 / 1e9, rel=1e-4)
    assert o["lm_head_fwd"]["achieved"] == pytest.approx(2 * M * 50304 * C / 1.2e-3 / 1e12,
                                                         rel=1e-4)


def test_cpu_baseline_reports_the_oracle():
    c = bench.cpu_baseline(synth.workload("tiny"), 1)
    assert c["kind"] == "oracle" and c["unit"] == "tokens/s"
    assert c["value"] > 0 and c["cores"] >= 1 and c["sample"].startswith("tiny:")
    assert "cpu_model" in c and "blas" in c
