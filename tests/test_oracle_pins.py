"""Pins of the oracle's building blocks and optimizer against closed forms,
textbook definitions, library routines and the numbers the pages print."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


# ---------------------------------------------------------------- layout
def test_parameter_count_matches_training_log(golden):
    d = golden["d48_run"]
    cfg = oracle.Config(d["n_layer"], d["n_head"], d["n_embd"], d["seq_len"], 50257,
                        d["padded_vocab_size"])
    n = oracle.num_params(cfg)
    assert n == d["num_parameters"]
    assert 2 * n == d["param_bytes_bf16"]
    assert (2 * n) // 2 ** 20 == d["param_mib"]
    assert (4 * n // d["num_processes"]) // 2 ** 20 == d["optimizer_state_shard_mib"]
    assert d["total_batch_size"] // (d["micro_batch"] * d["seq_len"] * d["num_processes"]) \
        == d["grad_accum_steps"]


def test_layout_is_dense_and_ordered():
    cfg = oracle.Config(3, 2, 16, 8, 11, 16)
    lay = oracle.param_layout(cfg)
    off = 0
    for _, o, s in lay:
        assert o == off
        off += int(np.prod(s))
    assert off == oracle.num_params(cfg)
    m = oracle.decay_mask(cfg)
    assert m.sum() == sum(int(np.prod(s)) for _, _, s in lay if len(s) == 2)


# ---------------------------------------------------------------- LR schedule
def test_lr_warmup_matches_training_log(golden):
    d = golden["d48_run"]
    for step, lr in d["lr_by_step"]:
        got = oracle.lr_schedule(step, d["max_lr"], d["warmup_iters"], 32000)
        assert f"{got:.2e}" == f"{lr:.2e}", (step, got, lr)


def test_lr_cosine_endpoints():
    mx = 6e-4
    assert oracle.lr_schedule(700, mx, 700, 32000) == pytest.approx(mx)
    assert oracle.lr_schedule(32000, mx, 700, 32000) == pytest.approx(0.1 * mx)
    mid = (700 + 32000) / 2
    assert oracle.lr_schedule(mid, mx, 700, 32000) == pytest.approx(0.55 * mx)
    vals = [oracle.lr_schedule(s, mx, 700, 32000) for s in range(700, 32001, 997)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


# ---------------------------------------------------------------- LayerNorm
def test_layernorm_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3 + 1
    w = np.ones(33)
    b = np.zeros(33)
    y, mean, rstd = oracle.layernorm_forward(x, w, b, 1e-5)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    # a constant row maps to exactly the shift
    c = np.full((1, 33), 2.5)
    bb = rng.standard_normal(33)
    yc, _, _ = oracle.layernorm_forward(c, rng.standard_normal(33), bb, 1e-5)
    assert np.array_equal(yc[0], bb)


def test_layernorm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 48))
    w = rng.standard_normal(48)
    b = rng.standard_normal(48)
    y, _, _ = oracle.layernorm_forward(x, w, b, 1e-5)
    yt = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), torch.from_numpy(w),
                                        torch.from_numpy(b), eps=1e-5)
    assert np.allclose(y, yt.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- GELU
def test_gelu_textbook_values():
    assert oracle.gelu(np.float64(0.0)) == 0.0
    assert oracle.gelu_grad(np.float64(0.0)) == 0.5
    big = np.array([10.0, 20.0])
    assert np.allclose(oracle.gelu(big), big, rtol=1e-12)
    assert np.allclose(oracle.gelu(-big), 0.0, atol=1e-12)
    # the tanh form approximates x * Phi(x) to within 5e-4 everywhere
    xs = np.linspace(-6, 6, 2001)
    exact = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    assert np.max(np.abs(oracle.gelu(xs) - exact)) < 5e-4
    # derivative against central differences
    h = 1e-6
    fd = (oracle.gelu(xs + h) - oracle.gelu(xs - h)) / (2 * h)
    assert np.max(np.abs(fd - oracle.gelu_grad(xs))) < 1e-8


# ---------------------------------------------------------------- attention
def test_attention_single_position_returns_v():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((2, 3, 1, 8)) for _ in range(3))
    o, p = oracle.causal_attention_forward(q, k, v)
    assert np.array_equal(o, v)
    assert np.all(p == 1.0)


def test_attention_zero_query_is_prefix_mean():
    rng = np.random.default_rng(3)
    T = 9
    q = np.zeros((1, 2, T, 4))
    k = rng.standard_normal((1, 2, T, 4))
    v = rng.standard_normal((1, 2, T, 4))
    o, p = oracle.causal_attention_forward(q, k, v)
    for t in range(T):
        assert np.allclose(o[0, :, t], v[0, :, :t + 1].mean(axis=1), rtol=1e-13, atol=1e-14)
    assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-14)
    assert np.all(np.triu(p[0, 0], 1) == 0)


def test_attention_brute_force_loops():
    """Pure-Python loops over (i, j) for a small case."""
    rng = np.random.default_rng(4)
    T, hd = 5, 3
    q, k, v = (rng.standard_normal((1, 1, T, hd)) for _ in range(3))
    o, _ = oracle.causal_attention_forward(q, k, v)
    for i in range(T):
        s = [sum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(hd)) / math.sqrt(hd)
             for j in range(i + 1)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        for d in range(hd):
            ref = sum(e[j] / z * v[0, 0, j, d] for j in range(i + 1))
            assert abs(o[0, 0, i, d] - ref) < 1e-13


# ---------------------------------------------------------------- cross-entropy
def test_cross_entropy_zero_logits_is_ln_v():
    V, Vp = 65, 128
    z = np.zeros((6, Vp))
    loss, losses, probs = oracle.cross_entropy_forward(z, np.arange(6), V)
    assert loss == pytest.approx(math.log(V), rel=1e-15)
    assert np.all(probs[:, V:] == 0)


def test_cross_entropy_rows_sum_to_one_fp32():
    rng = np.random.default_rng(5)
    V, Vp = 50257, 50304
    z = (rng.standard_normal((4, Vp)) * 3).astype(np.float32)
    z[:, V:] = 1e4  # padded columns must be ignored whatever they hold
    _, losses, probs = oracle.cross_entropy_forward(z, np.array([0, 1, 50256, 7]), V)
    assert np.all(np.abs(probs.sum(axis=1, dtype=np.float64) - 1) <= 1e-6)
    assert np.all(probs[:, V:] == 0)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z[:, :V]).double(),
                                            torch.tensor([0, 1, 50256, 7]), reduction="none")
    assert np.allclose(losses, ref.numpy(), rtol=1e-5)


# ---------------------------------------------------------------- clip + AdamW
def test_clip_closed_form():
    rng = np.random.default_rng(6)
    g = rng.standard_normal(1000)
    n = oracle.global_norm(g)
    assert n == pytest.approx(np.linalg.norm(g), rel=1e-14)
    s = oracle.clip_scale(n, 1.0)
    assert oracle.global_norm(g * s) == pytest.approx(1.0, rel=1e-12)
    small = g / (10 * n)
    assert oracle.clip_scale(oracle.global_norm(small), 1.0) == 1.0
    # the library routine adds 1e-6 to the norm; the difference is below 1e-6 rel.
    gt = torch.from_numpy(g.copy())
    gt_param = torch.zeros_like(gt, requires_grad=True)
    gt_param.grad = gt
    torch.nn.utils.clip_grad_norm_([gt_param], 1.0)
    assert np.allclose(gt_param.grad.numpy(), g * s, rtol=2e-6)


def test_adamw_first_step_closed_form():
    """At t = 1, mhat = g and vhat = g^2, so the update is
    -lr * (g / (|g| + eps) + wd * p * mask)."""
    rng = np.random.default_rng(7)
    p = rng.standard_normal(500)
    g = rng.standard_normal(500)
    mask = (np.arange(500) % 3 != 0).astype(np.float64)
    lr, wd, eps = 6e-4, 0.1, 1e-8
    p1, m, v = oracle.adamw_update(p.copy(), g, np.zeros(500), np.zeros(500), 1, lr, 0.9, 0.95,
                                   eps, wd, mask)
    ref = p - lr * (g / (np.abs(g) + eps) + wd * p * mask)
    assert np.allclose(p1, ref, rtol=1e-12, atol=1e-16)
    assert np.allclose(m, 0.1 * g, rtol=1e-14)
    assert np.allclose(v, 0.05 * g * g, rtol=1e-14)
    # lr = 0 leaves p unchanged; g = 0 with fresh state shrinks 2-D params by (1 - lr wd)
    p0, _, _ = oracle.adamw_update(p.copy(), g, np.zeros(500), np.zeros(500), 1, 0.0, 0.9, 0.95,
                                   eps, wd, mask)
    assert np.array_equal(p0, p)
    pz, _, _ = oracle.adamw_update(p.copy(), np.zeros(500), np.zeros(500), np.zeros(500), 1, lr,
                                   0.9, 0.95, eps, wd, mask)
    assert np.allclose(pz, p * (1 - lr * wd * mask), rtol=1e-15)


def test_adamw_matches_torch_optimizer():
    """Three steps against torch.optim.AdamW with decay on the 2-D group only."""
    rng = np.random.default_rng(8)
    w2 = rng.standard_normal((6, 5))
    w1 = rng.standard_normal(7)
    grads = [(rng.standard_normal((6, 5)), rng.standard_normal(7)) for _ in range(3)]
    tw2 = torch.tensor(w2, requires_grad=True)
    tw1 = torch.tensor(w1, requires_grad=True)
    opt = torch.optim.AdamW([{"params": [tw2], "weight_decay": 0.1},
                             {"params": [tw1], "weight_decay": 0.0}],
                            lr=1e-3, betas=(0.9, 0.95), eps=1e-8)
    p = np.concatenate([w2.ravel(), w1])
    mask = np.concatenate([np.ones(30), np.zeros(7)])
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for t, (g2, g1) in enumerate(grads, start=1):
        tw2.grad = torch.tensor(g2)
        tw1.grad = torch.tensor(g1)
        opt.step()
        oracle.adamw_update(p, np.concatenate([g2.ravel(), g1]), m, v, t, 1e-3, 0.9, 0.95, 1e-8,
                            0.1, mask)
    ref = np.concatenate([tw2.detach().numpy().ravel(), tw1.detach().numpy()])
    assert np.allclose(p, ref, rtol=1e-12, atol=1e-15)


def test_train_step_skips_nothing_and_counts():
    cfg = oracle.Config(2, 2, 16, 8, 11, 16)
    layout = oracle.param_layout(cfg)
    flat = synth.init_params(layout, 2, 11, [9, 2])
    m = np.zeros_like(flat)
    v = np.zeros_like(flat)
    rng = np.random.default_rng(9)
    batches = [(rng.integers(0, 11, (2, 8)).astype(np.int32),
                rng.integers(0, 11, (2, 8)).astype(np.int32)) for _ in range(2)]
    before = flat.copy()
    out = oracle.train_step(cfg, flat, m, v, 0, batches, lr=1e-3)
    assert out["t"] == 1
    assert out["norm"] > 0
    # padded wte rows: zero gradient and zero value, so they stay exactly zero
    W = oracle.unflatten(cfg, flat)["wte"]
    assert np.all(W[11:] == 0)
    assert not np.array_equal(before, flat)


# ---------------------------------------------------------------- synthetic inputs
def test_init_statistics():
    cfg = oracle.Config(4, 4, 256, 64, 500, 512)
    layout = oracle.param_layout(cfg)
    flat = synth.init_params(layout, 4, 500, [1, 2])
    P = oracle.unflatten(cfg, flat)
    assert np.std(P["h0.qkv_w"]) == pytest.approx(0.02, rel=0.02)
    assert np.std(P["h1.fc_w"]) == pytest.approx(0.02, rel=0.02)
    assert np.std(P["h2.proj_w"]) == pytest.approx(0.02 / math.sqrt(8), rel=0.03)
    assert np.std(P["h3.fcp_w"]) == pytest.approx(0.02 / math.sqrt(8), rel=0.03)
    assert np.all(P["wte"][500:] == 0)
    assert np.all(P["h0.ln1_w"] == 1) and np.all(P["lnf_b"] == 0) and np.all(P["h0.qkv_b"] == 0)


def test_zipf_token_stream():
    wl = synth.workload("small")
    s = synth.token_stream(wl, 200000)
    assert s.min() >= 0 and s.max() < 65
    w = np.arange(1, 66, dtype=np.float64) ** -1.1
    p0 = 1 / w.sum()
    assert np.mean(s == 0) == pytest.approx(p0, abs=0.005)
    assert 0.2 < p0 < 0.3
    big = synth.workload("gpt2_124m")
    s2 = synth.token_stream(big, 100000)
    assert s2.max() < 50257
    assert 0.08 < np.mean(s2 == 0) < 0.14
    x, y = synth.micro_batch(s2, 1, 4, 16)
    assert np.array_equal(x.ravel()[1:], y.ravel()[:-1])
    assert x[0, 0] == s2[64]
