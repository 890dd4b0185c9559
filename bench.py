"""Benchmark: GPT-2 training steps on one MI355X through libgpt2.so.

A step is zero_grad, k micro-steps of forward + backward (B x T tokens each,
inputs already resident in HBM), then global-norm clip + AdamW.  Prints one
JSON line with whole-job tokens/s, ms/step, MFU (6 N + 6 L T C flops per
token against the bf16 dense MFMA peak), a roofline entry for the dominant
kernel (every launch of it inside the timed steps bracketed by HIP event
pairs on the library's stream), the same figures for the other main kernels
(from one extra step each, outside the timed region) and the CPU oracle's
throughput on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_124m]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "train tokens/sec + MFU, GPT-2 124M bf16 B×T=16×1024, 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0

# HBM traffic of one launch of the dominant kernel (at GPT-2 124M the weight
# gradients of two layers, gemm_big_kernel<256,256,false,false,EPI_ACC_F32>,
# 216 tiles)
# from two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, mean over the timed pairs), each scaled by
# what the same counter reads for a plain device copy of known size.  Valid
# only for the GEMM source it was measured on (first 16 hex digits of its
# sha256); None until measured.  Source: profiles/gpt2_124m_bf16_train_step_counters.md.
WGRAD_TRAFFIC = {"gemm_source_sha256_16": "8e7ff5b44e7aa6a9", "shape": [16384, 768], "fetch_kib": 519386.3,
                 "write_kib": 55296.0, "fetch_factor": 2.0, "write_factor": 1.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--grad-accum", type=int, default=None,
                    help="override k (micro-steps per optimizer step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--fused-head", action="store_true",
                    help="train without stored logits (gpt2_config.fused_head = 1)")
    ap.add_argument("--recompute", type=int, default=0, choices=(0, 1, 2),
                    help="activation recompute (gpt2_config.recompute)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run three plain device-to-device copies of this many MiB "
                         "(the reference dispatches for scaling hardware traffic counters)")
    ap.add_argument("--cpu-sample-batch", type=int, default=3,
                    help="sequences in the oracle's timed sample (about 5 s of CPU work each)")
    return ap.parse_args()


def wgrad_layer_flops(cfg):
    """Algorithmic flops of one layer's weight gradients: dW += dy^T x for
    fc-proj (C x 4C), fc (4C x C), proj (C x C) and qkv (3C x C), K = B*T
    tokens: 2 * B*T * 12 C^2."""
    C, M = cfg.n_embd, cfg.micro_batch * cfg.seq_len
    return 2.0 * M * 12 * C * C


def wgrad_roofline(cfg, n, total_ms, micro_steps):
    """Roofline entry for the dominant kernel of the step: the grouped
    launches of the layers' weight gradients (the four products of one layer
    or of two layers per launch, one 256 x 256 tile per workgroup, fp32
    accumulation into the gradients; at GPT-2 124M two layers per launch, on
    the library's second stream beside the next layer's input-gradient work).
    Every such launch of the timed steps is bracketed by the library's event
    pairs; the flops per launch are the timed layers' flops over the
    launches."""
    import hashlib
    C, M, L = cfg.n_embd, cfg.micro_batch * cfg.seq_len, cfg.n_layer
    n = max(n, 1)
    t = total_ms / 1e3 / n
    layers = L * micro_steps / n  # layers per launch
    flops = wgrad_layer_flops(cfg) * layers
    achieved = flops / t / 1e12
    # per layer: the bf16 operands dy and x of the four products, read once
    # (columns C + 4C, 4C + C, C + C, 3C + C: 16 C per token), and the 12 C^2
    # fp32 gradients, read and written
    alg = int(layers * (2 * M * 16 * C + 8 * 12 * C * C))
    traffic = None
    src = os.path.join(ROOT, "transformer_lm_pretraining_train_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    tr = WGRAD_TRAFFIC
    if tr and sha == tr["gemm_source_sha256_16"] and (M, C) == tuple(tr["shape"]) and layers == 2:
        traffic = int(tr["fetch_kib"] * 1024 * tr["fetch_factor"]
                      + tr["write_kib"] * 1024 * tr["write_factor"])
    return {"kernel": "gemm_big_kernel<256,256,false,false,EPI_ACC_F32> (grouped weight gradients, "
                      f"{layers:g} layer(s) per launch: {4 * layers:g} products, K={M})",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "traffic_unit": "bytes per launch", "algorithmic_bytes": alg,
            "flops_per_launch": flops, "avg_launch_us": round(t * 1e6, 1), "launches_timed": n}


def other_kernels(cfg, n_timed):
    """Algorithmic work per launch of the other main kernels, each timed over
    one extra step: the lm_head forward product (2 M Vp C flops), causal
    attention (4 hd flops per query-key pair forward, 10 hd backward), the
    fused cross-entropy of the forward (one bf16 read of each logit row and
    one bf16 write of its gradient) and AdamW (30 bytes per parameter: read
    p, g, m, v, write p, m, v and the bf16 copy).  The LayerNorm entries
    (forward: bf16 row in and out, fp32 mean and rstd out; backward: bf16 dy,
    x and the incoming residual gradient in, bf16 dx out, fp32 mean and rstd
    in, none incoming for the final LayerNorm) are computed here but not
    timed by main(): an event pair adds several microseconds to a 10-25 us
    launch, so their rates come from the profiler's kernel trace."""
    import transformer_lm_pretraining_train_amd as g
    B, T, H, C, L = cfg.micro_batch, cfg.seq_len, cfg.n_head, cfg.n_embd, cfg.n_layer
    M = B * T
    hd = C // H
    pairs = B * H * T * (T + 1) // 2
    ln_bwd = (2 * L * (8 * C + 8) + (6 * C + 8)) * M / (2 * L + 1)
    work = {"lm_head_fwd": (2.0 * M * cfg.padded_vocab_size * C, "mfma"),
            "attn_fwd": (4.0 * hd * pairs, "mfma"), "attn_bwd": (10.0 * hd * pairs, "mfma"),
            "ce_fwd": (4.0 * M * cfg.padded_vocab_size, "hbm"),
            "ln_fwd": ((4.0 * C + 8) * M, "hbm"), "ln_bwd": (ln_bwd, "hbm"),
            "adamw": (30.0 * g.num_params(cfg), "hbm")}
    out = {}
    for name, (n, ms) in n_timed.items():
        w, bound = work[name]
        t = ms / 1e3 / n
        if bound == "mfma":
            a = w / t / 1e12
            out[name] = {"bound": bound, "achieved": round(a, 2), "unit": "TFLOP/s",
                         "peak": PEAK_BF16_TFLOPS, "frac": round(a / PEAK_BF16_TFLOPS, 4),
                         "avg_launch_us": round(t * 1e6, 1), "launches_timed": n}
        else:
            a = w / t / 1e9
            out[name] = {"bound": bound, "achieved": round(a, 1), "unit": "GB/s",
                         "peak": PEAK_HBM_GBS, "frac": round(a / PEAK_HBM_GBS, 4),
                         "bytes_per_launch": int(w), "avg_launch_us": round(t * 1e6, 1),
                         "launches_timed": n}
    return out


def host_info():
    """CPU model (/proc/cpuinfo) and the BLAS library NumPy runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, blas


def cpu_baseline(wl, B_sample):
    """The CPU oracle (as it stands) on one micro-step of B_sample sequences
    of the workload plus one AdamW over all parameters; tokens/s."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    ocfg = oracle.Config.from_workload(wl)
    layout = oracle.param_layout(ocfg)
    flat = synth.init_params(layout, wl.n_layer, wl.vocab_size, [wl.seed_id, 2])
    stream = synth.token_stream(wl, B_sample * wl.seq_len + 1)
    x, y = synth.micro_batch(stream, 0, B_sample, wl.seq_len)
    m = np.zeros_like(flat)
    v = np.zeros_like(flat)
    t0 = time.perf_counter()
    oracle.train_step(ocfg, flat, m, v, 0, [(x, y)], 6e-4)
    dt = time.perf_counter() - t0
    toks = B_sample * wl.seq_len
    cpu_model, blas = host_info()
    return {"value": round(toks / dt, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "blas": blas,
            "sample": f"{wl.name}: one micro-step of B={B_sample} x T={wl.seq_len} tokens "
                      f"(fwd + bwd) plus one clip + AdamW over all parameters, fp32 NumPy; "
                      f"{dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): data parallelism "
              "over several GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import transformer_lm_pretraining_train_amd as g

    wl = synth.workload(args.workload)
    if args.grad_accum:
        wl = wl.replace(grad_accum=args.grad_accum)
    cfg = g.config_for(wl, "bf16", fused_head=int(args.fused_head), recompute=args.recompute)
    torch.cuda.set_device(0)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration: three device copies of {n} bytes")
        del src, dst
    stream = torch.cuda.Stream()
    log(f"bench: {wl.name} bf16, B={wl.micro_batch} T={wl.seq_len} k={wl.grad_accum}, "
        f"fused_head={int(args.fused_head)} recompute={args.recompute}")

    with torch.cuda.stream(stream):
        model = g.Model(cfg, stream=stream)
        layout = [(n, o, s) for n, o, s, _ in g.param_layout(cfg)]
        flat = synth.init_params(layout, wl.n_layer, wl.vocab_size, [wl.seed_id, 2])
        model.set_params(torch.from_numpy(flat).cuda())
        toks = synth.token_stream(wl, wl.tokens_per_step + 1)
        batches = []
        for mi in range(wl.grad_accum):
            x, y = synth.micro_batch(toks, mi, wl.micro_batch, wl.seq_len)
            batches.append((torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()))
        losses = torch.zeros(wl.grad_accum, device="cuda")
        norm = torch.zeros(1, device="cuda")
    stream.synchronize()

    def step(s):
        lr = 6e-4 * min(1.0, s / 700)  # warm-up part of the schedule
        model.zero_grad()
        for mi, (x, y) in enumerate(batches):
            model.forward(x, y, losses[mi:mi + 1])
            model.backward()
        model.clip_and_adamw(lr, norm_out=norm)  # waits for the stream

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s + 1)
            log(f"warmup step {s + 1}: loss {losses.mean().item():.4f} norm {norm.item():.4f}")
        stream.synchronize()
        if not args.no_roofline:
            model.set_kernel_timer("wgrad", args.steps * wl.grad_accum * wl.n_layer)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for s in range(args.steps):
            step(args.warmup + s + 1)
        ev1.record(stream)
        stream.synchronize()
        wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    log(f"timed {args.steps} steps: wall {wall:.3f} s, events {gpu_s:.3f} s; "
        f"last loss {losses.mean().item():.4f} norm {norm.item():.4f}")
    ms = wall / args.steps * 1e3
    tps = wl.tokens_per_step * args.steps / wall
    fpt = g.flops_per_token(cfg)
    mfu = fpt * tps / (PEAK_BF16_TFLOPS * 1e12)

    roof = others = None
    if not args.no_roofline:
        roof = wgrad_roofline(cfg, *model.read_kernel_timer(), args.steps * wl.grad_accum)
        log(f"roofline: {roof}")
        # one more step per timed kernel, outside the timed region
        timed = {}
        names = ["attn_fwd", "attn_bwd", "adamw"]
        if not args.fused_head:
            names += ["lm_head_fwd", "ce_fwd"]
        with torch.cuda.stream(stream):
            for s, name in enumerate(names):
                model.set_kernel_timer(name, 4096)
                step(args.warmup + args.steps + s + 1)
                timed[name] = model.read_kernel_timer()
            model.set_kernel_timer("none")
        others = other_kernels(cfg, timed)
        log(f"other kernels: {others}")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, args.cpu_sample_batch)
        log(f"cpu baseline: {cpu}")
    out = {
        "metric": METRIC, "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (Zipf token stream, GPT-2 random init)",
        "config": {"workload": wl.name, "n_layer": wl.n_layer, "n_head": wl.n_head,
                   "n_embd": wl.n_embd, "vocab": wl.vocab_size,
                   "padded_vocab": wl.padded_vocab_size, "micro_batch": wl.micro_batch,
                   "seq_len": wl.seq_len, "grad_accum": wl.grad_accum,
                   "tokens_per_step": wl.tokens_per_step, "parallelism": "single-gpu",
                   "fused_head": int(args.fused_head), "recompute": args.recompute},
        "mfu": round(mfu, 4), "flops_per_token": fpt,
        "roofline": roof, "other_kernels": others, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
