"""Pins of the oracle's forward and backward against things other than itself:
central finite differences (fp64), an independent torch CPU autograd model
built from torch.nn.functional primitives, and invariants the method fixes
(causality, accumulation, tying, vocabulary padding)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def tiny_cfg(Vp=16, L=2, C=16, H=2, T=8, V=11):
    return oracle.Config(n_layer=L, n_head=H, n_embd=C, block_size=T, vocab_size=V,
                         padded_vocab_size=Vp)


def make_state(cfg, dtype=np.float64, seed=7, perturbed=True):
    layout = oracle.param_layout(cfg)
    flat = synth.init_params(layout, cfg.n_layer, cfg.vocab_size, seed=[seed, 2])
    if perturbed:
        flat = synth.perturb_affine(layout, flat, seed=[seed, 3])
    # larger weights than the GPT-2 init so every term carries signal
    rng = np.random.default_rng([seed, 4])
    flat = flat.astype(np.float64)
    for name, off, shape in layout:
        if len(shape) == 2:
            n = int(np.prod(shape))
            flat[off:off + n] *= 5.0
            if name == "wte":
                flat[off + cfg.vocab_size * shape[1]: off + n] = 0.0
    return flat.astype(dtype), rng


def tokens_for(cfg, B, T, seed=11):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, cfg.vocab_size, size=(B, T)).astype(np.int32)
    y = rng.integers(0, cfg.vocab_size, size=(B, T)).astype(np.int32)
    return x, y


def loss_of(cfg, flat, x, y):
    loss, _ = oracle.forward(cfg, oracle.unflatten(cfg, flat), x, y)
    return loss


def test_finite_differences_per_tensor():
    """Central differences in fp64 along a random direction inside each tensor."""
    cfg = tiny_cfg()
    flat, rng = make_state(cfg)
    x, y = tokens_for(cfg, 2, 8)
    g, _ = oracle.accumulate_grads(cfg, flat, [(x, y)])
    h = 1e-6
    for name, off, shape in oracle.param_layout(cfg):
        n = int(np.prod(shape))
        d = np.zeros_like(flat)
        d[off:off + n] = rng.standard_normal(n)
        if name == "wte":  # padded rows never reach the loss
            d[off + cfg.vocab_size * cfg.n_embd: off + n] = 0
        fd = (loss_of(cfg, flat + h * d, x, y) - loss_of(cfg, flat - h * d, x, y)) / (2 * h)
        an = float(np.dot(g, d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)) + 1e-9, (name, fd, an)


def test_finite_differences_tiny_workload_sampled():
    """The tiny workload (4 layers, C=64, hd=16, T=64, V=65) in fp64, three
    random whole-vector directions."""
    wl = synth.workload("tiny")
    cfg = oracle.Config.from_workload(wl)
    layout = oracle.param_layout(cfg)
    flat = synth.init_params(layout, cfg.n_layer, cfg.vocab_size, [wl.seed_id, 2])
    flat = synth.perturb_affine(layout, flat, [wl.seed_id, 3]).astype(np.float64)
    stream = synth.token_stream(wl, 2 * 64 + 1)
    x, y = synth.micro_batch(stream, 0, 2, 64)
    g, _ = oracle.accumulate_grads(cfg, flat, [(x, y)])
    rng = np.random.default_rng(5)
    h = 1e-6
    for _ in range(3):
        d = rng.standard_normal(flat.shape)
        fd = (loss_of(cfg, flat + h * d, x, y) - loss_of(cfg, flat - h * d, x, y)) / (2 * h)
        an = float(np.dot(g, d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def torch_reference_loss(cfg, flat_t, x, y):
    """Independent GPT-2 forward from torch.nn.functional primitives."""
    P = {n: flat_t[o:o + int(np.prod(s))].view(*s) for n, o, s in oracle.param_layout(cfg)}
    B, T = x.shape
    C, H = cfg.n_embd, cfg.n_head
    xt = torch.from_numpy(x.astype(np.int64))
    h = F.embedding(xt, P["wte"]) + P["wpe"][:T]
    for l in range(cfg.n_layer):
        p = f"h{l}."
        a = F.layer_norm(h, (C,), P[p + "ln1_w"], P[p + "ln1_b"], eps=cfg.ln_eps)
        q, k, v = F.linear(a, P[p + "qkv_w"], P[p + "qkv_b"]).split(C, dim=-1)
        q, k, v = (t.reshape(B, T, H, C // H).transpose(1, 2) for t in (q, k, v))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        o = o.transpose(1, 2).reshape(B, T, C)
        h = h + F.linear(o, P[p + "proj_w"], P[p + "proj_b"])
        a = F.layer_norm(h, (C,), P[p + "ln2_w"], P[p + "ln2_b"], eps=cfg.ln_eps)
        a = F.gelu(F.linear(a, P[p + "fc_w"], P[p + "fc_b"]), approximate="tanh")
        h = h + F.linear(a, P[p + "fcp_w"], P[p + "fcp_b"])
    h = F.layer_norm(h, (C,), P["lnf_w"], P["lnf_b"], eps=cfg.ln_eps)
    logits = F.linear(h, P["wte"])[..., :cfg.vocab_size]
    return F.cross_entropy(logits.reshape(-1, cfg.vocab_size),
                           torch.from_numpy(y.astype(np.int64)).reshape(-1))


@pytest.mark.parametrize("Vp", [11, 16])
def test_matches_torch_autograd(Vp):
    cfg = tiny_cfg(Vp=Vp, L=3, C=32, H=4, T=12)
    flat, _ = make_state(cfg)
    x, y = tokens_for(cfg, 3, 12)
    g, losses = oracle.accumulate_grads(cfg, flat, [(x, y)])
    ft = torch.from_numpy(flat.copy()).requires_grad_(True)
    lt = torch_reference_loss(cfg, ft, x, y)
    lt.backward()
    assert abs(losses[0] - lt.item()) <= 1e-12 * abs(lt.item())
    gt = ft.grad.numpy()
    for name, off, shape in oracle.param_layout(cfg):
        n = int(np.prod(shape))
        a, b = g[off:off + n], gt[off:off + n]
        assert np.linalg.norm(a - b) <= 1e-10 * max(np.linalg.norm(b), 1e-30), name


def test_causal_invariance_bitwise():
    """Changing token t+1 leaves every logit at positions <= t bit-identical."""
    cfg = tiny_cfg(L=2, C=32, H=4, T=16, V=23, Vp=23)
    for dtype in (np.float32, np.float64):
        flat, _ = make_state(cfg, dtype=dtype)
        P = oracle.unflatten(cfg, flat)
        x, _ = tokens_for(cfg, 2, 16)
        t = 6
        x2 = x.copy()
        x2[:, t + 1:] = (x2[:, t + 1:] + 5) % cfg.vocab_size
        _, c1 = oracle.forward(cfg, P, x)
        _, c2 = oracle.forward(cfg, P, x2)
        l1 = c1["logits"].reshape(2, 16, -1)
        l2 = c2["logits"].reshape(2, 16, -1)
        assert np.array_equal(l1[:, :t + 1], l2[:, :t + 1])
        assert not np.array_equal(l1[:, t + 1], l2[:, t + 1])


def test_accumulation_equals_full_batch():
    """k micro-batches with seed 1/(M k) equal one batch holding all of them."""
    cfg = tiny_cfg(L=2, C=32, H=4, T=8, V=13, Vp=16)
    for dtype, tol in ((np.float64, 1e-12), (np.float32, 1e-5)):
        flat, _ = make_state(cfg, dtype=dtype)
        x, y = tokens_for(cfg, 8, 8)
        g_full, _ = oracle.accumulate_grads(cfg, flat, [(x, y)])
        batches = [(x[i:i + 2], y[i:i + 2]) for i in range(0, 8, 2)]
        g_acc, losses = oracle.accumulate_grads(cfg, flat, batches)
        assert np.linalg.norm(g_acc - g_full) <= tol * np.linalg.norm(g_full)
        full_loss = loss_of(cfg, flat, x, y)
        assert abs(np.mean(losses) - full_loss) <= tol * full_loss


def test_tied_head_gradient_is_sum_of_untied_parts():
    cfg = tiny_cfg(L=2, C=16, H=2, T=8, V=11, Vp=16)
    flat, _ = make_state(cfg)
    P = oracle.unflatten(cfg, flat)
    x, y = tokens_for(cfg, 2, 8)
    g_tied, _ = oracle.accumulate_grads(cfg, flat, [(x, y)])
    # untied: a separate copy of wte drives the head
    head = P["wte"].copy()
    head_grad = np.zeros_like(head)
    gu = np.zeros_like(flat)
    G = oracle.unflatten(cfg, gu)
    _, cache = oracle.forward(cfg, P, x, y, lm_head=head)
    oracle.backward(cfg, P, cache, G, seed=1.0 / x.size, lm_head=head, lm_head_grad=head_grad)
    Gt = oracle.unflatten(cfg, g_tied)
    assert np.allclose(Gt["wte"], G["wte"] + head_grad, rtol=1e-12, atol=1e-15)
    assert np.abs(G["wte"]).sum() > 0 and np.abs(head_grad).sum() > 0


def test_vocab_padding_changes_nothing_but_shape():
    """Padding V=65 to Vp=128 reproduces the unpadded loss and gradients on
    the first 65 rows; padded rows get exactly zero gradient."""
    c65 = oracle.Config(2, 4, 64, 16, 65, 65)
    c128 = oracle.Config(2, 4, 64, 16, 65, 128)
    f65, _ = make_state(c65)
    P65 = oracle.unflatten(c65, f65)
    f128 = np.zeros(oracle.num_params(c128))
    P128 = oracle.unflatten(c128, f128)
    for n in P65:
        if n == "wte":
            P128[n][:65] = P65[n]
        else:
            P128[n][...] = P65[n]
    x, y = tokens_for(c65, 2, 16)
    g65, l65 = oracle.accumulate_grads(c65, f65, [(x, y)])
    g128, l128 = oracle.accumulate_grads(c128, f128, [(x, y)])
    assert abs(l65[0] - l128[0]) <= 1e-13 * l65[0]
    G65, G128 = oracle.unflatten(c65, g65), oracle.unflatten(c128, g128)
    for n in G65:
        b = G128[n][:65] if n == "wte" else G128[n]
        assert np.allclose(G65[n], b, rtol=1e-11, atol=1e-14), n
    assert np.all(G128["wte"][65:] == 0)


def test_initial_loss_close_to_ln_vocab(golden):
    """At GPT-2 init the loss is about ln V (10.82 for V = 50257, printed on
    the nanoGPT page); with the final LayerNorm at unit scale the logits are
    ~N(0, 0.02^2 C), which adds about 0.02^2 C / 2."""
    g = golden["init_loss"]
    V = g["vocab_size"]
    assert abs(math.log(V) - g["loss"]) < 0.01
    cfg = oracle.Config(2, 12, 768, 64, V, 50304)
    layout = oracle.param_layout(cfg)
    flat = synth.init_params(layout, cfg.n_layer, V, seed=[3, 2])
    wl = synth.workload("gpt2_124m")
    stream = synth.token_stream(wl, 4 * 64 + 1)
    x, y = synth.micro_batch(stream, 0, 4, 64)
    loss = loss_of(cfg, flat, x, y)
    closed = math.log(V) + 0.5 * 0.02 ** 2 * 768
    assert abs(loss - g["loss"]) <= 0.4
    assert abs(loss - closed) <= 0.1, (loss, closed)


def test_train_step_matches_torch_clip_and_adamw():
    """oracle.train_step as a whole -- k micro-steps of accumulated gradients,
    the global-norm clip applied to the gradient before AdamW's moments, the
    step count t advancing from 1, weight decay on 2-D tensors only ([wiki]
    training recipe) -- against the torch autograd model above followed by
    torch.nn.utils.clip_grad_norm_ and torch.optim.AdamW with a decayed 2-D
    group and an undecayed 1-D group.  Two optimizer steps of two micro-steps
    each, with a gradient norm far above the threshold so that the clip
    scales every step (at t = 1 Adam's update is ~sign(g) whatever the
    scale, so m and v carry the evidence; the second step needs the scales
    of both).  The norm is ~4e4, which makes the library routine's +1e-6 in
    the clip denominator a 2e-11 relative change."""
    cfg = tiny_cfg(Vp=16, L=2, C=16, H=2, T=8, V=11)
    flat, _ = make_state(cfg)
    oracle.unflatten(cfg, flat)["lnf_w"][:] *= 1e4
    steps = []
    for s in range(2):
        steps.append([tokens_for(cfg, 2, 8, seed=100 + 10 * s + i) for i in range(2)])
    lr, clip = 1e-3, 1.0

    # oracle
    p, m, v, t = flat.copy(), np.zeros_like(flat), np.zeros_like(flat), 0
    norms = []
    for batches in steps:
        out = oracle.train_step(cfg, p, m, v, t, batches, lr, grad_clip=clip)
        t = out["t"]
        norms.append(out["norm"])
    assert t == 2
    assert min(norms) > 1e4 * clip  # the clip bites on both steps

    # torch: one leaf per tensor, AdamW groups by dimensionality
    layout = oracle.param_layout(cfg)
    leaves = [torch.tensor(flat[o:o + int(np.prod(s))].reshape(s).copy(), requires_grad=True)
              for _, o, s in layout]
    opt = torch.optim.AdamW([{"params": [q for q in leaves if q.dim() == 2], "weight_decay": 0.1},
                             {"params": [q for q in leaves if q.dim() == 1], "weight_decay": 0.0}],
                            lr=lr, betas=(0.9, 0.95), eps=1e-8)
    for batches in steps:
        opt.zero_grad()
        ft = torch.cat([q.reshape(-1) for q in leaves])
        loss = sum(torch_reference_loss(cfg, ft, x, y) for x, y in batches) / len(batches)
        loss.backward()
        torch.nn.utils.clip_grad_norm_(leaves, clip)
        opt.step()

    def flat_of(ts):
        return np.concatenate([q.detach().numpy().ravel() for q in ts])

    tp = flat_of(leaves)
    tm = flat_of([opt.state[q]["exp_avg"] for q in leaves])
    tv = flat_of([opt.state[q]["exp_avg_sq"] for q in leaves])
    assert all(int(opt.state[q]["step"]) == 2 for q in leaves)
    for name, o, s in layout:
        n = int(np.prod(s))
        sl = slice(o, o + n)
        for mine, ref, what in ((m, tm, "m"), (v, tv, "v"), (p - flat, tp - flat, "delta p")):
            a, b = mine[sl], ref[sl]
            assert np.linalg.norm(a - b) <= 1e-10 * max(np.linalg.norm(b), 1e-300), (name, what)
