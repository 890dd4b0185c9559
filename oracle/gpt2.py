"""CPU oracle for one GPT-2 pretraining step -- TEST INFRASTRUCTURE ONLY.

A plain, slow NumPy implementation of what the GPU library computes:
forward, backward, global-norm gradient clipping and AdamW for the
decoder-only GPT-2 transformer.  It works in whatever float dtype the
parameters arrive in (float32 for parity, float64 for finite differences).
Attention materialises the full T x T score matrix and the loss is the
textbook mean cross-entropy; nothing here is blocked, fused or reordered.

Only the tests, the smoke entry and the benchmark's CPU-baseline leg may use
this module.  The GPU library shares no code with it.

Pages cited (by title and section; "the pages" are the web pages this
method is taken from):

* [rgzn1] news post on Karpathy's 4-hour "reproduce GPT-2 124M" lecture,
  rgzn1.com -- lecture outline: 12 layers, 768 channels, wte 50257 x 768.
* [qntz] "From 0 to 1 build GPT" post, qntz.me -- section "building the
  Transformer": multi-head self-attention via matmul + softmax, MLP,
  residual connections, LayerNorm; section "nanoGPT": loss 10.82 at init.
* [wiki] "Let's reproduce GPT-2 (124M)" notes, nolimitkun wiki -- section
  GPU optimisation ladder (vocab padding 50257 -> 50304) and section
  training recipe (AdamW 0.9/0.95/1e-8, global clip 1.0, cosine to 10 % with
  warm-up, weight decay 0.1 on 2-D params only, residual init 1/sqrt(2N),
  wte/lm_head tying, loss divided by the accumulation count).
* [dszhyy] llm.c GPT-2 1.5B post, dszhyy.com -- GPT2Config block
  (layer_norm_epsilon 1e-5, initializer_range 0.02), flags section (GELU,
  weight decay on 2-D weights), setup section (the training log: parameter
  count, learning-rate warm-up values).

Readings where the pages are silent are listed next to the code they
affect: tanh-form GELU, biased LayerNorm variance with eps inside the square
root, attention scale 1/sqrt(head_dim) with position i seeing j <= i,
qkv columns ordered [q | k | v] with heads contiguous inside each, linear
weights stored (out, in), padded logits treated as -inf.

Every function here is pinned by tests/test_oracle_*.py (finite
differences, torch CPU autograd, closed forms, the pages' printed numbers).
"""
from __future__ import annotations

import math

import numpy as np

GELU_K = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


# --------------------------------------------------------------------------
# parameter layout
# --------------------------------------------------------------------------
def param_layout(cfg):
    """Flat parameter order: list of ``(name, offset, shape)``.

    wte (Vp, C), wpe (block_size, C), then per layer ln1 gain/shift, qkv
    weight (3C, C) and bias, attention output projection (C, C) and bias,
    ln2 gain/shift, fc weight (4C, C) and bias, fc projection (C, 4C) and
    bias; last the final LayerNorm gain/shift.  lm_head is wte (tied,
    [wiki] training recipe), so it has no entry.
    """
    C, L = cfg.n_embd, cfg.n_layer
    shapes = [("wte", (cfg.padded_vocab_size, C)), ("wpe", (cfg.block_size, C))]
    for l in range(L):
        p = f"h{l}."
        shapes += [
            (p + "ln1_w", (C,)), (p + "ln1_b", (C,)),
            (p + "qkv_w", (3 * C, C)), (p + "qkv_b", (3 * C,)),
            (p + "proj_w", (C, C)), (p + "proj_b", (C,)),
            (p + "ln2_w", (C,)), (p + "ln2_b", (C,)),
            (p + "fc_w", (4 * C, C)), (p + "fc_b", (4 * C,)),
            (p + "fcp_w", (C, 4 * C)), (p + "fcp_b", (C,)),
        ]
    shapes += [("lnf_w", (C,)), ("lnf_b", (C,))]
    out, off = [], 0
    for name, shape in shapes:
        out.append((name, off, shape))
        off += int(np.prod(shape))
    return out


def num_params(cfg) -> int:
    return sum(int(np.prod(s)) for _, _, s in param_layout(cfg))


def unflatten(cfg, flat):
    """Dict name -> view into ``flat`` (no copy)."""
    return {n: flat[o: o + int(np.prod(s))].reshape(s) for n, o, s in param_layout(cfg)}


def decay_mask(cfg, dtype=np.float32):
    """1 for elements of 2-D tensors (weight decay applies), else 0
    ([wiki] training recipe; [dszhyy] flags section, ``-c 0.1``)."""
    m = np.zeros(num_params(cfg), dtype=dtype)
    for _, off, shape in param_layout(cfg):
        if len(shape) == 2:
            m[off: off + int(np.prod(shape))] = 1
    return m


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def layernorm_forward(x, w, b, eps):
    """Per row: mean, biased variance, rstd = 1/sqrt(var + eps),
    y = w * (x - mean) * rstd + b.  eps = 1e-5 ([dszhyy] GPT2Config)."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    y = (x - mean) * rstd * w + b
    return y, mean[..., 0], rstd[..., 0]


def layernorm_backward(dy, x, w, mean, rstd):
    """Gradients of layernorm_forward: (dx, dw, db)."""
    xhat = (x - mean[..., None]) * rstd[..., None]
    dw = (dy * xhat).reshape(-1, x.shape[-1]).sum(axis=0)
    db = dy.reshape(-1, x.shape[-1]).sum(axis=0)
    g = dy * w
    dx = rstd[..., None] * (g - g.mean(axis=-1, keepdims=True)
                            - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dx, dw, db


def gelu(h):
    """GELU, tanh form (Hendrycks & Gimpel):
    0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3)))."""
    return 0.5 * h * (1.0 + np.tanh(GELU_K * (h + GELU_A * h ** 3)))


def gelu_grad(h):
    """d gelu / d h for the tanh form."""
    t = np.tanh(GELU_K * (h + GELU_A * h ** 3))
    return 0.5 * (1.0 + t) + 0.5 * h * (1.0 - t * t) * GELU_K * (1.0 + 3.0 * GELU_A * h * h)


def split_heads(qkv, B, T, H):
    """qkv (B*T, 3C) with columns [q | k | v], head h at columns
    h*hd .. (h+1)*hd of each third -> q, k, v as (B, H, T, hd)."""
    C = qkv.shape[-1] // 3
    hd = C // H
    parts = []
    for i in range(3):
        t = qkv[:, i * C:(i + 1) * C].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        parts.append(t)
    return parts


def merge_heads(o):
    B, H, T, hd = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B * T, H * hd)


def causal_attention_forward(q, k, v):
    """Scaled dot-product self-attention with a causal mask
    ([qntz] building the Transformer: matmul + softmax): S = q k^T / sqrt(hd),
    S[i, j] = -inf for j > i, P = softmax over j, O = P v.
    Returns (O, P); P is materialised in full."""
    hd = q.shape[-1]
    T = q.shape[-2]
    s = (q @ np.swapaxes(k, -1, -2)) * (1.0 / math.sqrt(hd))
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v, p


def causal_attention_backward(do, q, k, v, p):
    """Gradients of causal_attention_forward: (dq, dk, dv).
    Softmax backward in its textbook form dS = P * (dP - rowsum(dP * P))."""
    hd = q.shape[-1]
    scale = 1.0 / math.sqrt(hd)
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq, dk, dv


def cross_entropy_forward(logits, targets, vocab_size):
    """Mean cross-entropy over rows; logits columns >= vocab_size (vocab
    padding, [wiki] GPU optimisation ladder) are excluded, i.e. treated as
    -inf, so their probability is exactly 0.  Returns (mean loss, per-row
    losses, probabilities over all padded columns)."""
    z = logits[:, :vocab_size]
    zmax = z.max(axis=1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1))
    rows = np.arange(z.shape[0])
    losses = lse - z[rows, targets]
    probs = np.zeros_like(logits)
    probs[:, :vocab_size] = np.exp(z - lse[:, None])
    return losses.mean(), losses, probs


# --------------------------------------------------------------------------
# model forward / backward
# --------------------------------------------------------------------------
def forward(cfg, params, tokens, targets=None, lm_head=None):
    """Forward pass on tokens (B, T).

    x0 = wte[tok] + wpe[t]; per layer (pre-LN): x += proj(attn(ln1(x)));
    x += fcp(gelu(fc(ln2(x)))); then lnf and logits = lnf(x) wte^T (tied
    head, [wiki] training recipe) over the padded vocabulary.
    ``lm_head`` replaces wte in the head only (untied variant, for tests).
    Returns (mean loss or None, cache dict).
    """
    B, T = tokens.shape
    H, eps = cfg.n_head, cfg.ln_eps
    P = params
    tok = tokens.reshape(-1)
    x = P["wte"][tok] + np.tile(P["wpe"][:T], (B, 1))
    cache = {"tokens": tok, "B": B, "T": T, "x0": x, "layers": []}
    for l in range(cfg.n_layer):
        p = f"h{l}."
        c = {"x_in": x}
        ln1, c["m1"], c["r1"] = layernorm_forward(x, P[p + "ln1_w"], P[p + "ln1_b"], eps)
        qkv = ln1 @ P[p + "qkv_w"].T + P[p + "qkv_b"]
        q, k, v = split_heads(qkv, B, T, H)
        o, probs = causal_attention_forward(q, k, v)
        atty = merge_heads(o)
        x2 = x + atty @ P[p + "proj_w"].T + P[p + "proj_b"]
        ln2, c["m2"], c["r2"] = layernorm_forward(x2, P[p + "ln2_w"], P[p + "ln2_b"], eps)
        h = ln2 @ P[p + "fc_w"].T + P[p + "fc_b"]
        g = gelu(h)
        x3 = x2 + g @ P[p + "fcp_w"].T + P[p + "fcp_b"]
        c.update(ln1=ln1, qkv=qkv, q=q, k=k, v=v, probs=probs, atty=atty, x2=x2,
                 ln2=ln2, h=h, g=g)
        cache["layers"].append(c)
        x = x3
    lnf, cache["mf"], cache["rf"] = layernorm_forward(x, P["lnf_w"], P["lnf_b"], eps)
    head = P["wte"] if lm_head is None else lm_head
    logits = lnf @ head.T
    cache.update(x_final=x, lnf=lnf, logits=logits)
    loss = None
    if targets is not None:
        tgt = targets.reshape(-1)
        loss, losses, probs = cross_entropy_forward(logits, tgt, cfg.vocab_size)
        cache.update(targets=tgt, losses=losses, ce_probs=probs)
    return loss, cache


def backward(cfg, params, cache, grads, seed, lm_head=None, lm_head_grad=None):
    """Accumulate d(seed * sum_rows loss_row)/d params into ``grads``.

    With seed = 1 / (B*T*k) this is the gradient of (mean loss) / k, the
    per-micro-step contribution under k-step accumulation ([wiki] training
    recipe: the loss must be divided by the accumulation count).
    ``grads`` is a dict of arrays shaped like the params (added to in place).
    """
    P, G = params, grads
    H = cfg.n_head
    B, T = cache["B"], cache["T"]
    M = B * T
    # softmax + cross-entropy: dz = seed * (p - onehot(target)); padded
    # columns have p = 0 and therefore dz = 0.
    dz = cache["ce_probs"].copy()
    dz[np.arange(M), cache["targets"]] -= 1.0
    dz *= seed
    head = P["wte"] if lm_head is None else lm_head
    if lm_head is None:
        G["wte"] += dz.T @ cache["lnf"]
    else:
        lm_head_grad += dz.T @ cache["lnf"]
    dlnf = dz @ head
    dx, dw, db = layernorm_backward(dlnf, cache["x_final"], P["lnf_w"], cache["mf"], cache["rf"])
    G["lnf_w"] += dw
    G["lnf_b"] += db
    for l in reversed(range(cfg.n_layer)):
        p = f"h{l}."
        c = cache["layers"][l]
        # x3 = x2 + g fcp_w^T + fcp_b
        G[p + "fcp_w"] += dx.T @ c["g"]
        G[p + "fcp_b"] += dx.sum(axis=0)
        dg = dx @ P[p + "fcp_w"]
        dh = dg * gelu_grad(c["h"])
        G[p + "fc_w"] += dh.T @ c["ln2"]
        G[p + "fc_b"] += dh.sum(axis=0)
        dln2 = dh @ P[p + "fc_w"]
        dxl, dw, db = layernorm_backward(dln2, c["x2"], P[p + "ln2_w"], c["m2"], c["r2"])
        G[p + "ln2_w"] += dw
        G[p + "ln2_b"] += db
        dx2 = dx + dxl
        # x2 = x + atty proj_w^T + proj_b
        G[p + "proj_w"] += dx2.T @ c["atty"]
        G[p + "proj_b"] += dx2.sum(axis=0)
        datty = dx2 @ P[p + "proj_w"]
        do = datty.reshape(B, T, H, -1).transpose(0, 2, 1, 3)
        dq, dk, dv = causal_attention_backward(do, c["q"], c["k"], c["v"], c["probs"])
        dqkv = np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv)], axis=1)
        G[p + "qkv_w"] += dqkv.T @ c["ln1"]
        G[p + "qkv_b"] += dqkv.sum(axis=0)
        dln1 = dqkv @ P[p + "qkv_w"]
        dxl, dw, db = layernorm_backward(dln1, c["x_in"], P[p + "ln1_w"], c["m1"], c["r1"])
        G[p + "ln1_w"] += dw
        G[p + "ln1_b"] += db
        dx = dx2 + dxl
    # embedding: scatter-add into the token rows, sum over the batch for wpe
    np.add.at(G["wte"], cache["tokens"], dx)
    G["wpe"][:T] += dx.reshape(B, T, -1).sum(axis=0)
    return G


# --------------------------------------------------------------------------
# optimizer
# --------------------------------------------------------------------------
def global_norm(g):
    """Euclidean norm of the whole gradient vector (accumulated in fp64)."""
    g64 = np.asarray(g, dtype=np.float64)
    return float(np.sqrt(np.dot(g64, g64)))


def clip_scale(norm, max_norm):
    """Global clip ([wiki] training recipe, threshold 1.0): the gradient is
    multiplied by min(1, max_norm / norm)."""
    return min(1.0, max_norm / norm) if norm > 0 else 1.0


def adamw_update(p, g, m, v, t, lr, beta1, beta2, eps, weight_decay, mask):
    """One AdamW step at 1-indexed step ``t`` (decoupled weight decay,
    Loshchilov & Hutter), in place on p, m, v:
    m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
    mhat = m / (1 - b1^t);  vhat = v / (1 - b2^t);
    p -= lr * (mhat / (sqrt(vhat) + eps) + wd * mask * p).
    Hyper-parameters per [wiki] training recipe: 0.9, 0.95, 1e-8, wd 0.1."""
    dt = p.dtype
    b1, b2 = dt.type(beta1), dt.type(beta2)
    m *= b1
    m += (dt.type(1) - b1) * g
    v *= b2
    v += (dt.type(1) - b2) * g * g
    mhat = m / dt.type(1.0 - beta1 ** t)
    vhat = v / dt.type(1.0 - beta2 ** t)
    p -= dt.type(lr) * (mhat / (np.sqrt(vhat) + dt.type(eps)) + dt.type(weight_decay) * mask * p)
    return p, m, v


def lr_schedule(step, max_lr, warmup, total, min_ratio=0.1):
    """Learning rate at 1-indexed ``step``: linear warm-up max_lr*step/warmup,
    then cosine decay to min_ratio*max_lr at ``total`` ([wiki] training
    recipe; [dszhyy] flags section ``-l 0.0006 -q 0.1 -u 700``; the warm-up
    values in the [dszhyy] setup-section log pin the 1-indexing)."""
    min_lr = min_ratio * max_lr
    if step <= warmup:
        return max_lr * step / warmup
    if step >= total:
        return min_lr
    ratio = (step - warmup) / (total - warmup)
    return min_lr + 0.5 * (1.0 + math.cos(math.pi * ratio)) * (max_lr - min_lr)


# --------------------------------------------------------------------------
# one optimizer step
# --------------------------------------------------------------------------
def accumulate_grads(cfg, flat_params, batches, observe=None):
    """Sum over k micro-batches of the gradient of (mean loss)/k.
    Returns (flat grads, list of per-micro-batch mean losses).  ``observe``,
    if given, is called with each micro-batch's forward cache (read-only use:
    per-position losses, logits) before its backward."""
    k = len(batches)
    P = unflatten(cfg, flat_params)
    gflat = np.zeros_like(flat_params)
    G = unflatten(cfg, gflat)
    losses = []
    for x, y in batches:
        loss, cache = forward(cfg, P, x, y)
        if observe is not None:
            observe(cache)
        backward(cfg, P, cache, G, seed=1.0 / (x.size * k))
        losses.append(float(loss))
        del cache
    return gflat, losses


def train_step(cfg, flat_params, m, v, t, batches, lr, beta1=0.9, beta2=0.95, eps=1e-8,
               weight_decay=0.1, grad_clip=1.0, observe=None):
    """zero_grad, k x (forward + backward), global norm, clip, AdamW.

    Updates ``flat_params``, ``m``, ``v`` in place and returns a dict with the
    new step count, the mean loss over micro-batches, the pre-clip norm, the
    clip scale and the (unclipped) accumulated gradient.  ``observe`` as for
    accumulate_grads.
    """
    gflat, losses = accumulate_grads(cfg, flat_params, batches, observe)
    norm = global_norm(gflat)
    s = clip_scale(norm, grad_clip)
    g = gflat * flat_params.dtype.type(s)
    t = t + 1
    adamw_update(flat_params, g, m, v, t, lr, beta1, beta2, eps, weight_decay,
                 decay_mask(cfg, flat_params.dtype))
    return {"t": t, "loss": float(np.mean(losses)), "losses": losses, "norm": norm,
            "scale": s, "grads": gflat}
