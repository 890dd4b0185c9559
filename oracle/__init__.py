"""CPU oracle for the GPT-2 training step -- TEST INFRASTRUCTURE ONLY.

Plain NumPy reference that the GPU library is checked against.  Only the
test suite, the smoke entry point and the benchmark's CPU-baseline leg may
import it; the GPU library never does, and shares no code with it.

Every function is pinned by CPU tests against something other than itself
(finite differences, torch CPU autograd, closed forms, the pages' printed
numbers).  Parity unpinned: none.
"""
from .gpt2 import *  # noqa: F401,F403
from . import gpt2  # noqa: F401


class Config:
    """Model shape for the oracle."""

    def __init__(self, n_layer, n_head, n_embd, block_size, vocab_size,
                 padded_vocab_size=None, ln_eps=1e-5):
        self.n_layer = n_layer
        self.n_head = n_head
        self.n_embd = n_embd
        self.block_size = block_size
        self.vocab_size = vocab_size
        self.padded_vocab_size = padded_vocab_size or vocab_size
        self.ln_eps = ln_eps

    @classmethod
    def from_workload(cls, wl, **kw):
        c = cls(wl.n_layer, wl.n_head, wl.n_embd, wl.block_size, wl.vocab_size,
                wl.padded_vocab_size)
        for k, v in kw.items():
            setattr(c, k, v)
        return c
