"""Python binding of libgpt2.so -- one GPT-2 pretraining step on an MI355X.

Argument marshalling only: every step of forward, backward, clipping and
AdamW runs in the library's HIP kernels.  PyTorch provides device memory
(one workspace tensor plus the caller's inputs and outputs) and the HIP
stream.  Loading fails loudly when the library has not been built; there is
no fallback.

The names mirror the C ABI in include/gpt2.h and include/gpt2_kernels.h.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GPT2Config", "TensorInfo", "GPT2Error", "lib", "library_path", "Model", "ZScore",
    "param_layout",
    "num_params", "workspace_bytes", "gemm", "gemm_colsum_ok", "gemm_workspace_bytes",
    "gemm_acc_group", "gemm_acc_group_workspace_bytes", "attention_forward", "attention_backward",
    "attention_colsum_ok",
    "attention_backward_scratch_bytes", "flops_per_token", "config_for",
    "GPT2_FP32", "GPT2_BF16", "EPI",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libgpt2.so")

GPT2_FP32, GPT2_BF16 = 0, 1
ERRORS = {0: "OK", -1: "EINVAL", -2: "EWORKSPACE", -3: "ESTATE", -4: "ETOKEN",
          -5: "ENONFINITE", -6: "EHIP"}
EPI = {"store": 0, "bias": 1, "bias_resid": 2, "bias_gelu": 3, "gelu_bwd": 4, "acc_f32": 5}
DBG = {"logits": 0, "losses": 1, "argmax": 2, "ln1": 3, "qkv": 4, "atty": 5, "res2": 6,
       "fch": 7, "res3": 8, "lnf": 9, "att_lse": 10, "encoded": 11}
TIMER = {"none": 0, "lm_head_fwd": 1, "attn_fwd": 2, "attn_bwd": 3, "ce_fwd": 4, "adamw": 5,
         "wgrad": 6, "ln_fwd": 7, "ln_bwd": 8}


class GPT2Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layer", "n_head", "n_embd", "block_size", "vocab_size", "padded_vocab_size",
        "micro_batch", "seq_len", "grad_accum_steps", "dtype", "deterministic")] + [
        ("ln_eps", ctypes.c_float), ("recompute", ctypes.c_int32), ("fused_head", ctypes.c_int32)]

    def __repr__(self):
        return "GPT2Config(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class TensorInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("offset", ctypes.c_int64), ("ndim", ctypes.c_int32),
                ("decay", ctypes.c_int32), ("shape", ctypes.c_int64 * 2)]


class GPT2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgpt2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m transformer_lm_pretraining_train_amd.build`")
        L = ctypes.CDLL(library_path)
        P, I, I64, SZ, F, D = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                               ctypes.c_float, ctypes.c_double)
        CFG = ctypes.POINTER(GPT2Config)
        sig = {
            "gpt2_workspace_bytes": (SZ, [CFG]),
            "gpt2_num_params": (I64, [CFG]),
            "gpt2_param_layout": (I, [CFG, ctypes.POINTER(TensorInfo), I]),
            "gpt2_create": (I, [CFG, P, SZ, P, ctypes.POINTER(P)]),
            "gpt2_destroy": (I, [P]),
            "gpt2_set_params": (I, [P, P]),
            "gpt2_get_params": (I, [P, P]),
            "gpt2_get_grads": (I, [P, P]),
            "gpt2_set_grads": (I, [P, P]),
            "gpt2_get_opt_state": (I, [P, P, P, ctypes.POINTER(I64)]),
            "gpt2_set_opt_state": (I, [P, P, P, I64]),
            "gpt2_forward": (I, [P, P, P, P]),
            "gpt2_backward": (I, [P]),
            "gpt2_zero_grad": (I, [P]),
            "gpt2_clip_and_adamw": (I, [P, F, F, F, F, F, F, P]),
            "gpt2_sync": (I, [P]),
            "gpt2_debug_read": (I, [P, I, I, P, SZ]),
            "gpt2_set_kernel_timer": (I, [P, I, I]),
            "gpt2_read_kernel_timer": (I, [P, ctypes.POINTER(I), ctypes.POINTER(ctypes.c_double)]),
            "gpt2_last_error": (ctypes.c_char_p, []),
            "gpt2_forward_loss": (I, [P, P, P, P]),
            "gpt2_zscore_create": (I, [I, ctypes.POINTER(P)]),
            "gpt2_zscore_update": (I, [P, D, ctypes.POINTER(D)]),
            "gpt2_zscore_destroy": (I, [P]),
            "gpt2_zscore_get_state": (I, [P, P, I, ctypes.POINTER(I), ctypes.POINTER(I)]),
            "gpt2_zscore_set_state": (I, [P, P, I]),
            "gpt2_grad_norm": (I, [P, F, ctypes.POINTER(F)]),
            "gpt2_adamw_update": (I, [P, F, F, F, F, F]),
            "gpt2_guarded_step": (I, [P, P, P, F, F, F, F, F, F, F, F, F, ctypes.POINTER(F),
                                      ctypes.POINTER(D), ctypes.POINTER(D), ctypes.POINTER(I)]),
            "gpt2_skip_counts": (I, [P, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
            "gpt2_save_state": (I, [P, ctypes.c_char_p]),
            "gpt2_load_state": (I, [P, ctypes.c_char_p]),
            "gpt2k_gemm": (I, [I, I, I, I, I, I, P, I64, P, I64, I, P, I64, P, P, I64, P, I64, P,
                               I64, P, SZ, P]),
            "gpt2k_gemm_colsum_ok": (I, [I, I, I, I, I, I, I64, I64, I]),
            "gpt2k_gemm_colsum": (I, [I, I, I, I, I, I, P, I64, P, I64, I, P, I64, P, P, I64, P,
                                      I64, P, I64, P, I64, P, SZ, P]),
            "gpt2k_gemm_workspace_bytes": (SZ, [I, I, I, I, I]),
            "gpt2k_gemm_acc_group_workspace_bytes": (SZ, [I, I, P, P, I, P, P]),
            "gpt2k_gemm_acc_group": (I, [I, I, P, P, I, P, P, P, P, P, P, P, SZ, P]),
            "gpt2k_attention_forward": (I, [I, P, P, P, I, I, I, I, P]),
            "gpt2k_attention_backward_scratch_bytes": (SZ, [I, I, I]),
            "gpt2k_attention_backward": (I, [I, P, P, P, P, P, I, I, I, I, P, P]),
            "gpt2k_attention_colsum_ok": (I, [I, I]),
            "gpt2k_attention_backward_colsum": (I, [I, P, P, P, P, P, I, I, I, I, P, P, P]),
            "gpt2k_attention_backward_noalloc": (I, [I, P, P, P, P, P, I, I, I, I, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise GPT2Error(rc, lib().gpt2_last_error().decode())
    return rc


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def config_for(wl, dtype=None, **overrides) -> GPT2Config:
    """GPT2Config for a synthetic workload (see the ``synth`` module)."""
    dt = {"fp32": GPT2_FP32, "bf16": GPT2_BF16}[dtype or wl.gpu_dtype]
    c = GPT2Config(wl.n_layer, wl.n_head, wl.n_embd, wl.block_size, wl.vocab_size,
                   wl.padded_vocab_size, wl.micro_batch, wl.seq_len, wl.grad_accum, dt, 0, 1e-5)
    for k, v in overrides.items():
        setattr(c, k, v)
    return c


def workspace_bytes(cfg: GPT2Config) -> int:
    n = lib().gpt2_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise GPT2Error(-1, lib().gpt2_last_error().decode())
    return n


def num_params(cfg: GPT2Config) -> int:
    n = lib().gpt2_num_params(ctypes.byref(cfg))
    if n < 0:
        raise GPT2Error(-1, lib().gpt2_last_error().decode())
    return n


def param_layout(cfg: GPT2Config):
    """[(name, offset, shape, decay)] in flat order (host only, no GPU)."""
    n = _check_count(lib().gpt2_param_layout(ctypes.byref(cfg), None, 0))
    arr = (TensorInfo * n)()
    _check_count(lib().gpt2_param_layout(ctypes.byref(cfg), arr, n))
    out = []
    for t in arr:
        shape = (t.shape[0], t.shape[1]) if t.ndim == 2 else (t.shape[0],)
        out.append((t.name.decode(), t.offset, shape, bool(t.decay)))
    return out


def _check_count(rc):
    if rc < 0:
        raise GPT2Error(rc, lib().gpt2_last_error().decode())
    return rc


def flops_per_token(cfg: GPT2Config) -> int:
    """Training FLOPs per token, 6 N + 6 L T C: the convention that
    reproduces the MFU printed in the llm.c 1.5B training log (dszhyy.com
    page, setup section); 6 L T C is the causal attention matmul work of
    forward and backward."""
    return 6 * num_params(cfg) + 6 * cfg.n_layer * cfg.seq_len * cfg.n_embd


class Model:
    """One model on the current HIP device, over a torch-allocated workspace."""

    def __init__(self, cfg: GPT2Config, stream=None):
        import torch
        self.cfg = cfg
        self.torch_stream = stream if stream is not None else torch.cuda.current_stream()
        self.nbytes = workspace_bytes(cfg)
        self.workspace = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        self.n_params = num_params(cfg)
        h = ctypes.c_void_p()
        _check(lib().gpt2_create(ctypes.byref(cfg), _ptr(self.workspace), self.nbytes,
                                 _stream(self.torch_stream), ctypes.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- state
    def _vec(self):
        import torch
        return torch.empty(self.n_params, dtype=torch.float32, device="cuda")

    def set_params(self, flat):
        _check(lib().gpt2_set_params(self.h, _ptr(flat)))

    def get_params(self, out=None):
        out = self._vec() if out is None else out
        _check(lib().gpt2_get_params(self.h, _ptr(out)))
        return out

    def get_grads(self, out=None):
        out = self._vec() if out is None else out
        _check(lib().gpt2_get_grads(self.h, _ptr(out)))
        return out

    def set_grads(self, flat):
        _check(lib().gpt2_set_grads(self.h, _ptr(flat)))

    def get_opt_state(self):
        m, v = self._vec(), self._vec()
        step = ctypes.c_int64()
        _check(lib().gpt2_get_opt_state(self.h, _ptr(m), _ptr(v), ctypes.byref(step)))
        return m, v, step.value

    def set_opt_state(self, m, v, step):
        _check(lib().gpt2_set_opt_state(self.h, _ptr(m), _ptr(v), step))

    # ---- the step
    def forward(self, tokens, targets=None, loss_out=None):
        _check(lib().gpt2_forward(self.h, _ptr(tokens), _ptr(targets), _ptr(loss_out)))
        return loss_out

    def forward_loss(self, tokens, targets, loss_out=None):
        """The loss alone, without materialising the logits (gpt2_forward_loss)."""
        _check(lib().gpt2_forward_loss(self.h, _ptr(tokens), _ptr(targets), _ptr(loss_out)))
        return loss_out

    def backward(self):
        _check(lib().gpt2_backward(self.h))

    def zero_grad(self):
        _check(lib().gpt2_zero_grad(self.h))

    def clip_and_adamw(self, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                       grad_clip=1.0, norm_out=None):
        _check(lib().gpt2_clip_and_adamw(self.h, lr, beta1, beta2, eps, weight_decay, grad_clip,
                                         _ptr(norm_out)))
        return norm_out

    def sync(self):
        _check(lib().gpt2_sync(self.h))

    # ---- training-loop robustness (see gpt2.h)
    def grad_norm(self, grad_clip=1.0):
        n = ctypes.c_float()
        _check(lib().gpt2_grad_norm(self.h, grad_clip, ctypes.byref(n)))
        return n.value

    def adamw_update(self, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
        _check(lib().gpt2_adamw_update(self.h, lr, beta1, beta2, eps, weight_decay))

    def guarded_step(self, loss, lr, loss_z=None, norm_z=None, z_max_loss=5.0, z_max_norm=5.0,
                     beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_clip=1.0):
        """Returns dict(norm, z_loss, z_norm, skipped); a non-finite norm raises
        GPT2Error (ENONFINITE) after counting the skip."""
        n, zl, zn, sk = ctypes.c_float(), ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
        _check(lib().gpt2_guarded_step(
            self.h, loss_z.h if loss_z is not None else None,
            norm_z.h if norm_z is not None else None, float(loss), z_max_loss, z_max_norm, lr,
            beta1, beta2, eps, weight_decay, grad_clip, ctypes.byref(n), ctypes.byref(zl),
            ctypes.byref(zn), ctypes.byref(sk)))
        return {"norm": n.value, "z_loss": zl.value, "z_norm": zn.value, "skipped": bool(sk.value)}

    def skip_counts(self):
        a, b = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().gpt2_skip_counts(self.h, ctypes.byref(a), ctypes.byref(b)))
        return {"nonfinite": a.value, "outlier": b.value}

    def save_state(self, path):
        _check(lib().gpt2_save_state(self.h, os.fsencode(path)))

    def load_state(self, path):
        _check(lib().gpt2_load_state(self.h, os.fsencode(path)))

    def set_kernel_timer(self, name, max_launches=4096):
        """Bracket every launch of one step (TIMER key) with a HIP event pair."""
        _check(lib().gpt2_set_kernel_timer(self.h, TIMER[name], max_launches))

    def read_kernel_timer(self):
        """(launches timed since the last read, their summed duration in ms)."""
        n = ctypes.c_int(0)
        ms = ctypes.c_double(0.0)
        _check(lib().gpt2_read_kernel_timer(self.h, ctypes.byref(n), ctypes.byref(ms)))
        return n.value, ms.value

    def debug_read(self, name, out, layer=0):
        _check(lib().gpt2_debug_read(self.h, DBG[name], layer, _ptr(out),
                                     out.numel() * out.element_size()))
        return out


class ZScore:
    """Rolling z-score over the last ``window`` finite values (gpt2_zscore_*;
    host only)."""

    def __init__(self, window=128):
        h = ctypes.c_void_p()
        _check(lib().gpt2_zscore_create(window, ctypes.byref(h)))
        self.h = h

    def update(self, x):
        z = ctypes.c_double()
        _check(lib().gpt2_zscore_update(self.h, float(x), ctypes.byref(z)))
        return z.value

    def get_state(self):
        """The values held, oldest first (a list of floats)."""
        w, n = ctypes.c_int(), ctypes.c_int()
        _check(lib().gpt2_zscore_get_state(self.h, None, 0, ctypes.byref(w), ctypes.byref(n)))
        buf = (ctypes.c_double * max(n.value, 1))()
        _check(lib().gpt2_zscore_get_state(self.h, buf, n.value, None, None))
        return list(buf[:n.value])

    def set_state(self, values):
        buf = (ctypes.c_double * max(len(values), 1))(*values)
        _check(lib().gpt2_zscore_set_state(self.h, buf, len(values)))

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_zscore_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()


# ---- kernel-level entry points
def gemm_workspace_bytes(dtype, M, N, K, epilogue):
    epi = EPI[epilogue] if isinstance(epilogue, str) else epilogue
    return lib().gpt2k_gemm_workspace_bytes(dtype, M, N, K, epi)


def gemm(dtype, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, epilogue, out, ldo, bias=None,
         resid=None, ldr=0, out2=None, ldo2=0, aux=None, ldx=0, ws=None, stream=None,
         colsum=None, ldcs=0):
    """C(m, n) = sum_k A(m, k) B(n, k) + epilogue (see gpt2_kernels.h).  For the
    fp32-accumulating epilogue a split-K workspace is allocated here when
    ``ws`` is None and the product would use one.  ``colsum`` (fp32, 64-row
    block column sums of the output) goes to gpt2k_gemm_colsum."""
    epi = EPI[epilogue] if isinstance(epilogue, str) else epilogue
    if ws is None:
        nb = gemm_workspace_bytes(dtype, M, N, K, epi)
        if nb:
            import torch
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    if colsum is None:
        _check(lib().gpt2k_gemm(dtype, int(a_kmajor), int(b_kmajor), M, N, K, _ptr(A), lda, _ptr(B),
                                ldb, epi, _ptr(out), ldo, _ptr(bias), _ptr(resid), ldr, _ptr(out2),
                                ldo2, _ptr(aux), ldx, _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(lib().gpt2k_gemm_colsum(dtype, int(a_kmajor), int(b_kmajor), M, N, K, _ptr(A), lda,
                                       _ptr(B), ldb, epi, _ptr(out), ldo, _ptr(bias), _ptr(resid),
                                       ldr, _ptr(out2), ldo2, _ptr(aux), ldx, _ptr(colsum), ldcs,
                                       _ptr(ws), nbytes, _stream(stream)))


def gemm_colsum_ok(dtype, a_kmajor, b_kmajor, M, N, K, lda, ldb, epilogue):
    epi = EPI[epilogue] if isinstance(epilogue, str) else epilogue
    return bool(lib().gpt2k_gemm_colsum_ok(dtype, int(a_kmajor), int(b_kmajor), M, N, K, lda, ldb,
                                           epi))


def _arr(ctype, vals):
    a = (ctype * len(vals))(*vals)
    return a, ctypes.cast(a, ctypes.c_void_p)


def gemm_acc_group_workspace_bytes(dtype, Ms, Ns, K, ldas, ldbs):
    n = len(Ms)
    keep = [_arr(ctypes.c_int, Ms), _arr(ctypes.c_int, Ns), _arr(ctypes.c_int64, ldas),
            _arr(ctypes.c_int64, ldbs)]
    return lib().gpt2k_gemm_acc_group_workspace_bytes(dtype, n, keep[0][1], keep[1][1], K,
                                                       keep[2][1], keep[3][1])


def gemm_acc_group(dtype, Ms, Ns, K, As, ldas, Bs, ldbs, outs, ldos, ws=None, stream=None):
    """out_i += A_i^T B_i (m-major A_i, n-major B_i) for up to four products
    sharing K, in one launch where possible (see gpt2_kernels.h).  A split-K
    workspace is allocated here when ``ws`` is None and one is needed."""
    n = len(Ms)
    if ws is None:
        nb = gemm_acc_group_workspace_bytes(dtype, Ms, Ns, K, ldas, ldbs)
        if nb:
            import torch
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    keep = [_arr(ctypes.c_int, Ms), _arr(ctypes.c_int, Ns), _arr(ctypes.c_void_p, [a.data_ptr() for a in As]),
            _arr(ctypes.c_int64, ldas), _arr(ctypes.c_void_p, [b.data_ptr() for b in Bs]),
            _arr(ctypes.c_int64, ldbs), _arr(ctypes.c_void_p, [o.data_ptr() for o in outs]),
            _arr(ctypes.c_int64, ldos)]
    _check(lib().gpt2k_gemm_acc_group(dtype, n, keep[0][1], keep[1][1], K, keep[2][1], keep[3][1],
                                      keep[4][1], keep[5][1], keep[6][1], keep[7][1], _ptr(ws),
                                      nbytes, _stream(stream)))


def attention_forward(dtype, out, lse, qkv, B, T, H, hd, stream=None):
    _check(lib().gpt2k_attention_forward(dtype, _ptr(out), _ptr(lse), _ptr(qkv), B, T, H, hd,
                                         _stream(stream)))


def attention_backward_scratch_bytes(B, T, H):
    return lib().gpt2k_attention_backward_scratch_bytes(B, T, H)


def attention_backward(dtype, dqkv, dout, qkv, out, lse, B, T, H, hd, scratch, stream=None,
                       colsum=None):
    """``colsum``: fp32 (B * ceil(T/128), 3C) column sums of dqkv per 128-row
    block (gpt2k_attention_backward_colsum)."""
    _check(lib().gpt2k_attention_backward_colsum(dtype, _ptr(dqkv), _ptr(dout), _ptr(qkv),
                                                 _ptr(out), _ptr(lse), B, T, H, hd,
                                                 _ptr(scratch), _ptr(colsum), _stream(stream)))


def attention_backward_noalloc(dtype, dqkv, dout, qkv, out, lse, B, T, H, hd, stream=None,
                               colsum=None):
    """gpt2k_attention_backward_noalloc: the attention backward with its
    per-row scratch in the library's fixed device array (no allocation)."""
    _check(lib().gpt2k_attention_backward_noalloc(dtype, _ptr(dqkv), _ptr(dout), _ptr(qkv),
                                                  _ptr(out), _ptr(lse), B, T, H, hd, _ptr(colsum),
                                                  _stream(stream)))


def attention_colsum_ok(dtype, hd):
    return bool(lib().gpt2k_attention_colsum_ok(dtype, hd))
