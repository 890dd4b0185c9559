"""gpt2k_attention_backward_noalloc (the attention backward for callers that
cannot allocate: its scratch in the library's fixed device array) against
the entry point that takes a caller-provided scratch buffer, through the C
ABI: bit-identical dqkv and column sums on two calls in a row, the second
with a smaller input, and a clear error for an input beyond the fixed
array."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import transformer_lm_pretraining_train_amd as g  # noqa: E402
from gpu_util import bf16_round, host, to_dev  # noqa: E402

BF16, FP32 = g.GPT2_BF16, g.GPT2_FP32


def _inputs(dt, B, T, H, hd, seed):
    rng = np.random.default_rng(seed)
    C = H * hd
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    qkv = rng.standard_normal((B * T, 3 * C)).astype(np.float32)
    dout = rng.standard_normal((B * T, C)).astype(np.float32)
    if dt == BF16:
        qkv, dout = bf16_round(qkv), bf16_round(dout)
    d_qkv, d_dout = to_dev(qkv, tdt), to_dev(dout, tdt)
    d_out = torch.empty((B * T, C), dtype=tdt, device="cuda")
    d_lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    g.attention_forward(dt, d_out, d_lse, d_qkv, B, T, H, hd)
    return d_qkv, d_dout, d_out, d_lse


def _both(dt, B, T, H, hd, seed, colsum):
    C = H * hd
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    qkv, dout, out, lse = _inputs(dt, B, T, H, hd, seed)
    ref = torch.full((B * T, 3 * C), float("nan"), dtype=tdt, device="cuda")
    got = torch.full_like(ref, float("nan"))
    nblk = (T + 127) // 128
    cs_ref = cs_got = None
    if colsum:
        cs_ref = torch.full((B * nblk, 3 * C), float("nan"), device="cuda")
        cs_got = torch.full_like(cs_ref, float("nan"))
    scratch = torch.empty(g.attention_backward_scratch_bytes(B, T, H), dtype=torch.uint8,
                          device="cuda")
    g.attention_backward(dt, ref, dout, qkv, out, lse, B, T, H, hd, scratch, colsum=cs_ref)
    g.attention_backward_noalloc(dt, got, dout, qkv, out, lse, B, T, H, hd, colsum=cs_got)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), host(ref))
    if colsum:
        assert np.array_equal(host(cs_got), host(cs_ref))


@pytest.mark.parametrize("dt,hd,colsum", [(BF16, 64, True), (BF16, 64, False), (FP32, 32, False)])
def test_noalloc_attention_backward_matches_scratch_entry_point(dt, hd, colsum):
    """Two calls in a row on one GPU (the fixed array keeps the first call's
    values), the second smaller: B*H*T = 16*12*1024 (the GPT-2 124M shape for
    bf16), then 3*5*200."""
    print(f"noalloc attention backward dt={dt} hd={hd} colsum={colsum}", flush=True)
    if dt == BF16:
        _both(dt, 16, 1024, 12, hd, 1, colsum)
    else:
        _both(dt, 4, 256, 4, hd, 1, colsum)
    _both(dt, 3, 200, 5, hd, 2, colsum)


def test_noalloc_attention_backward_rejects_inputs_beyond_its_array():
    """B*H*T above 2^20 rows is refused before anything runs."""
    B, T, H, hd = 64, 1024, 17, 64  # 1114112 rows of D
    C = H * hd
    # tiny stand-ins: the call must fail on the size check, before any launch
    dummy = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(g.GPT2Error) as ei:
        g.attention_backward_noalloc(BF16, dummy, dummy, dummy, dummy, lse, B, T, H, hd)
    assert ei.value.name == "EINVAL" and "fixed scratch" in str(ei.value)
    assert C > 0
