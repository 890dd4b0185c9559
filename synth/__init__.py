"""Seeded synthetic inputs for the GPT-2 training step.

This module is shared by the tests, the benchmark and the smoke entry.  It
draws the inputs that both the GPU library and the CPU oracle consume --
token streams, micro-batch slices and the initial parameter vector -- and
holds none of the training step's arithmetic.

Sources for the workload shapes (the pages are cited by title and section):

* GPT-2 124M is 12 layers of 768 channels with a 50257 x 768 token table
  (news post "Karpathy 4-hour GPT-2 lecture", rgzn1.com, lecture outline).
* The vocabulary is padded from 50257 to 50304 (page "Let's reproduce GPT-2
  (124M)", section GPU optimisation ladder, "nice numbers").
* Init: N(0, 0.02) weights (GPT2Config ``initializer_range``, dszhyy.com
  page, deployment section); residual projections scaled by 1/sqrt(2 L)
  ("Let's reproduce GPT-2 (124M)", training recipe section).
* The training data (FineWeb-EDU) is not available; a Zipf unigram stream of
  the same vocabulary stands in for it.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "token_stream",
    "micro_batch",
    "init_params",
    "perturb_affine",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic training configuration (shape, batch, token law, seeds)."""

    name: str
    seed_id: int
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    vocab_size: int
    padded_vocab_size: int
    micro_batch: int
    seq_len: int
    grad_accum: int
    token_law: str  # "uniform" or "zipf"
    zipf_s: float
    gpu_dtype: str  # compute dtype the GPU path runs this workload in

    @property
    def tokens_per_micro_step(self) -> int:
        return self.micro_batch * self.seq_len

    @property
    def tokens_per_step(self) -> int:
        return self.micro_batch * self.seq_len * self.grad_accum

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 4, 64, 64, 65, 65, 8, 64, 1, "uniform", 0.0, "fp32"),
    "small": Workload("small", 2, 6, 6, 384, 256, 65, 65, 16, 256, 4, "zipf", 1.1, "bf16"),
    "gpt2_124m": Workload("gpt2_124m", 3, 12, 12, 768, 1024, 50257, 50304, 16, 1024, 32,
                          "zipf", 1.05, "bf16"),
    "gpt2_350m": Workload("gpt2_350m", 4, 24, 16, 1024, 1024, 50257, 50304, 16, 1024, 32,
                          "zipf", 1.05, "bf16"),
    "gpt2_1558m": Workload("gpt2_1558m", 5, 48, 25, 1600, 1024, 50257, 50304, 16, 1024, 32,
                           "zipf", 1.05, "bf16"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def token_stream(wl: Workload, n: int, seed=None) -> np.ndarray:
    """``n`` int32 token ids in [0, vocab_size), seeded by ``[seed_id, 1]``.

    "uniform": every id equally likely.  "zipf": p(id) proportional to
    (id + 1) ** -s, drawn by inverting the fp64 cumulative distribution.
    """
    rng = np.random.default_rng([wl.seed_id, 1] if seed is None else seed)
    V = wl.vocab_size
    if wl.token_law == "uniform":
        return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)
    if wl.token_law == "zipf":
        w = np.arange(1, V + 1, dtype=np.float64) ** (-wl.zipf_s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(n)
        ids = np.searchsorted(cdf, u, side="right")
        return np.minimum(ids, V - 1).astype(np.int32)
    raise ValueError(f"unknown token law {wl.token_law!r}")


def micro_batch(stream: np.ndarray, m: int, B: int, T: int):
    """Micro-batch ``m`` of a token stream: ``B*T + 1`` consecutive ids, split
    into inputs ``x = buf[:-1]`` and targets ``y = buf[1:]`` (next token),
    each reshaped to (B, T)."""
    buf = stream[m * B * T: (m + 1) * B * T + 1]
    if buf.shape[0] != B * T + 1:
        raise ValueError("token stream too short for this micro-batch")
    x = np.ascontiguousarray(buf[:-1].reshape(B, T), dtype=np.int32)
    y = np.ascontiguousarray(buf[1:].reshape(B, T), dtype=np.int32)
    return x, y


def _is_residual_projection(name: str) -> bool:
    return name.endswith(".proj_w") or name.endswith(".fcp_w")


def init_params(layout, n_layer: int, vocab_size: int, seed, std: float = 0.02) -> np.ndarray:
    """GPT-2 style initial parameters as one flat float32 vector.

    ``layout`` is a sequence of ``(name, offset, shape)`` in flat order.
    2-D weights ~ N(0, std^2); the attention and MLP output projections
    (names ``*.proj_w``, ``*.fcp_w``) are scaled by 1/sqrt(2 * n_layer);
    biases and LayerNorm shifts are 0, LayerNorm gains are 1; rows of
    ``wte`` at or beyond ``vocab_size`` (vocabulary padding) are 0.
    """
    rng = np.random.default_rng(seed)
    total = max(off + int(np.prod(shape)) for _, off, shape in layout)
    flat = np.zeros(total, dtype=np.float32)
    for name, off, shape in layout:
        n = int(np.prod(shape))
        view = flat[off: off + n].reshape(shape)
        base = name.split(".")[-1]
        if len(shape) == 2:
            w = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
            if _is_residual_projection(name):
                w *= np.float32(1.0 / math.sqrt(2 * n_layer))
            if name == "wte" and shape[0] > vocab_size:
                w[vocab_size:] = 0.0
            view[...] = w
        elif base.endswith("_w") and base.startswith("ln"):
            view[...] = 1.0
        else:
            view[...] = 0.0
    return flat


def perturb_affine(layout, flat: np.ndarray, seed, std: float = 0.02) -> np.ndarray:
    """Copy of ``flat`` with biases ~ N(0, std^2), LayerNorm gains
    1 + N(0, 0.1^2) and shifts ~ N(0, std^2), so that bias and affine terms
    are exercised instead of being hidden behind zeros and ones."""
    rng = np.random.default_rng(seed)
    out = flat.copy()
    for name, off, shape in layout:
        if len(shape) != 1:
            continue
        n = int(np.prod(shape))
        base = name.split(".")[-1]
        if base.startswith("ln") and base.endswith("_w"):
            out[off: off + n] = 1.0 + 0.1 * rng.standard_normal(n).astype(np.float32)
        else:
            out[off: off + n] = std * rng.standard_normal(n).astype(np.float32)
    return out
