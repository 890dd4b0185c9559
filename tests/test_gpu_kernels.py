"""GEMM and attention kernels through the kernel-level C ABI, against the
oracle's definitions (plain matmul; the oracle's causal attention) on the
same seeded inputs: small ragged shapes element by element, and the GPT-2
124M shapes on sampled rows / heads."""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import transformer_lm_pretraining_train_amd as g  # noqa: E402
from gpu_util import bf16_round, cosine, host, rel_l2, to_dev  # noqa: E402

FP32, BF16 = g.GPT2_FP32, g.GPT2_BF16


def _store(mat, kmajor, rows, K, ld_extra, rng, pad_value):
    """Lay out logical operand mat (rows x K) in memory: k-major (rows, ld)
    or m-major (K, ld).  Padding holds pad_value."""
    if kmajor:
        ld = ((K + 7) // 8) * 8 + ld_extra
        buf = np.full((rows, ld), pad_value, dtype=np.float32)
        buf[:, :K] = mat
    else:
        ld = ((rows + 7) // 8) * 8 + ld_extra
        buf = np.full((K, ld), pad_value, dtype=np.float32)
        buf[:, :rows] = mat.T
    return buf, ld


def run_gemm(dt, akm, bkm, M, N, K, epi, seed=0, ld_extra=0, pad_value=np.nan):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K)).astype(np.float32)
    if dt == BF16:
        A, B = bf16_round(A), bf16_round(B)
    # NaN padding only where the kernel promises not to read it into an
    # output that is stored: the k tail of k-major operands is masked.
    Abuf, lda = _store(A, akm, M, K, ld_extra, rng, pad_value if akm else 0.0)
    Bbuf, ldb = _store(B, bkm, N, K, ld_extra, rng, pad_value if bkm else 0.0)
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    dA, dB = to_dev(Abuf, tdt), to_dev(Bbuf, tdt)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bias = rng.standard_normal(N).astype(np.float32)
    resid = rng.standard_normal((M, N)).astype(np.float32)
    aux = rng.standard_normal((M, N)).astype(np.float32)
    if dt == BF16:
        resid, aux = bf16_round(resid), bf16_round(aux)
    kw = {}
    if epi == "acc_f32":
        init = rng.standard_normal((M, N)).astype(np.float32)
        out = to_dev(init)
        expect = init + ref
    else:
        out = torch.zeros((M, N), dtype=tdt, device="cuda")
        if epi == "store":
            expect = ref
        elif epi == "bias":
            expect = ref + bias
        elif epi == "bias_resid":
            expect = ref + bias + resid
        elif epi == "bias_gelu":
            expect = ref + bias
            out2 = torch.zeros((M, N), dtype=tdt, device="cuda")
            kw.update(out2=out2, ldo2=N)
        elif epi == "gelu_bwd":
            expect = ref * oracle.gelu_grad(aux.astype(np.float64))
        kw.update(bias=to_dev(bias), resid=to_dev(resid, tdt), ldr=N, aux=to_dev(aux, tdt), ldx=N)
    g.gemm(dt, akm, bkm, M, N, K, dA, lda, dB, ldb, epi, out, N, **kw)
    torch.cuda.synchronize()
    got = host(out)
    res = {"got": got, "expect": expect}
    if epi == "bias_gelu":
        res["got2"] = host(kw["out2"])
        res["expect2"] = oracle.gelu(got.astype(np.float64))
    return res


ORIENT = [(True, True), (True, False), (False, False), (False, True)]
EPIS = ["store", "bias", "bias_resid", "bias_gelu", "gelu_bwd", "acc_f32"]


@pytest.mark.parametrize("dt", [FP32, BF16])
@pytest.mark.parametrize("akm,bkm", ORIENT)
@pytest.mark.parametrize("M,N,K", [(200, 72, 136), (129, 65, 65), (256, 128, 64), (64, 320, 1000),
                                   (300, 200, 136), (777, 1000, 520), (512, 129, 65), (1024, 768, 192)])
def test_gemm_orientations_ragged(dt, akm, bkm, M, N, K):
    print(f"gemm dt={dt} akm={akm} bkm={bkm} M={M} N={N} K={K}", flush=True)
    r = run_gemm(dt, akm, bkm, M, N, K, "store", seed=M + N + K, ld_extra=8)
    assert np.all(np.isfinite(r["got"]))
    tol = 1e-5 if dt == FP32 else 4e-3
    assert rel_l2(r["got"], r["expect"]) < tol


@pytest.mark.parametrize("dt", [FP32, BF16])
@pytest.mark.parametrize("epi", EPIS)
def test_gemm_epilogues(dt, epi):
    print(f"gemm epilogue dt={dt} {epi}", flush=True)
    akm, bkm = (False, False) if epi == "acc_f32" else (True, True)
    r = run_gemm(dt, akm, bkm, 150, 136, 200, epi, seed=3)
    tol = 1e-5 if dt == FP32 or epi == "acc_f32" else 4e-3
    assert rel_l2(r["got"], r["expect"]) < tol
    # the same epilogue on the large-tile kernels (M >= 256), ragged edges
    r = run_gemm(dt, akm, bkm, 520, 392, 200, epi, seed=4)
    tol = 1e-5 if dt == FP32 or epi == "acc_f32" else 4e-3
    assert rel_l2(r["got"], r["expect"]) < tol
    if epi == "bias_gelu":
        assert rel_l2(r["got2"], r["expect2"]) < (1e-5 if dt == FP32 else 4e-3)


@pytest.mark.parametrize("epi", ["bias", "bias_resid", "bias_gelu"])
@pytest.mark.parametrize("N,ldo", [(520, 520), (514, 520)])
def test_bias_epilogues_on_192_wide_tiles(epi, N, ldo):
    """The bias epilogues on the 256 x 192 large-tile kernel (the qkv, fc and
    projection products of the model; M = 16384 rows make three 192-wide tile
    columns the cheapest plan for these N), where each lane loads its bias
    once per tile: a last tile column 136 or 130 wide, and for N = 514 a
    last 8-column chunk that reaches past N (element-wise there, 16-byte
    accesses elsewhere, output pitch 520).  All outputs against fp64 of the
    bf16-rounded inputs."""
    M, K = 16384, 136
    print(f"gemm 256x192 {epi} N={N} ldo={ldo}", flush=True)
    rng = np.random.default_rng(N + len(epi))
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    B = bf16_round(rng.standard_normal((N, K)).astype(np.float32))
    bias = rng.standard_normal(N).astype(np.float32)
    resid = bf16_round(rng.standard_normal((M, ldo)).astype(np.float32))
    ref = A.astype(np.float64) @ B.astype(np.float64).T + bias
    if epi == "bias_resid":
        ref = ref + resid[:, :N]
    out = torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device="cuda")
    kw = {"bias": to_dev(bias)}
    if epi == "bias_resid":
        kw.update(resid=to_dev(resid, torch.bfloat16), ldr=ldo)
    if epi == "bias_gelu":
        out2 = torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device="cuda")
        kw.update(out2=out2, ldo2=ldo)
    g.gemm(BF16, True, True, M, N, K, to_dev(A, torch.bfloat16), K, to_dev(B, torch.bfloat16), K,
           epi, out, ldo, **kw)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isnan(got[:, N:])), "columns past N were written"
    got = got[:, :N]
    assert rel_l2(got, ref) < 4e-3
    # the last tile column on its own (ragged edge)
    assert rel_l2(got[:, 384:], ref[:, 384:]) < 4e-3
    if epi == "bias_gelu":
        g2 = host(out2)[:, :N]
        assert rel_l2(g2, oracle.gelu(got.astype(np.float64))) < 4e-3


@pytest.mark.parametrize("akm,bkm", ORIENT)
@pytest.mark.parametrize("K,pad", [(200, 0), (40, 0), (136, 3)])
def test_gemm_store_persistent_256_tiles(akm, bkm, K, pad):
    """Products large enough for the persistent 256 x 256 store kernel (4
    rounds of tiles), ragged in M, N and K, one k-tile (K = 40), and an output
    pitch that is not a multiple of 8 (every store element-wise); 80 sampled
    rows, all columns, against fp64."""
    M, N = 8092, 8132
    ldo = N + pad
    print(f"gemm 256x256 store akm={akm} bkm={bkm} M={M} N={N} K={K} ldo={ldo}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(K + pad)
    kp = (K + 7) // 8 * 8
    A = torch.randn((M, kp) if akm else (K, M + 4), device="cuda", generator=gen).to(torch.bfloat16)
    B = torch.randn((N, kp) if bkm else (K, N + 4), device="cuda", generator=gen).to(torch.bfloat16)
    if akm:
        A[:, K:] = float("nan")  # the k tail past K must not reach the output
    if bkm:
        B[:, K:] = float("nan")
    out = torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device="cuda")
    g.gemm(BF16, akm, bkm, M, N, K, A, A.shape[1], B, B.shape[1], "store", out, ldo)
    torch.cuda.synchronize()
    rows = np.random.default_rng(K).choice(M, 64, replace=False)
    extra = [0, 255, 256, M // 2, 7935, 7936, M - 1]  # first, tile borders, last (ragged) tile
    rows = np.unique(np.concatenate([rows, np.array(extra)]))
    ridx = torch.from_numpy(rows).cuda()
    Am = (A[ridx, :K] if akm else A[:, ridx].T).float().cpu().numpy().astype(np.float64)
    Bm = (B[:, :K] if bkm else B[:, :N].T).float().cpu().numpy().astype(np.float64)
    ref = Am @ Bm.T
    got = out[ridx].float().cpu().numpy()
    assert np.all(np.isfinite(got[:, :N]))
    assert rel_l2(got[:, :N], ref) < 4e-3
    if pad:
        assert np.all(np.isnan(got[:, N:]))  # the pitch padding is not written


@pytest.mark.parametrize("akm,bkm,M,N,K", [
    (True, True, 16384, 2304, 768),     # qkv forward
    (True, True, 16384, 3072, 768),     # fc forward
    (True, True, 16384, 768, 3072),     # fc projection forward
    (True, True, 16384, 50304, 768),    # lm_head forward
    (True, False, 16384, 768, 50304),   # lm_head input gradient
    (False, False, 3072, 768, 16384),   # fc weight gradient
    (False, False, 50304, 768, 16384),  # wte gradient from the head
    (True, True, 16384, 4096, 1024),    # 350M fc forward
    (True, True, 16384, 1024, 4096),    # 350M fc projection forward (K = 4096)
    (True, False, 16384, 1024, 4096),   # 350M fc input gradient (K = 4096)
    (False, False, 1024, 4096, 16384),  # 350M fc projection weight gradient
])
def test_gemm_gpt2_124m_shapes_sampled(akm, bkm, M, N, K):
    """bf16 GEMM at the 124M shapes and the 350M MLP shapes; 64 sampled
    output rows against fp64."""
    print(f"gemm 124M akm={akm} bkm={bkm} M={M} N={N} K={K}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(M ^ N ^ K)
    A = torch.randn((M, K) if akm else (K, M), device="cuda", generator=gen).to(torch.bfloat16)
    B = torch.randn((N, K) if bkm else (K, N), device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    g.gemm(BF16, akm, bkm, M, N, K, A, A.shape[1], B, B.shape[1], "store", out, N)
    torch.cuda.synchronize()
    rows = np.random.default_rng(M ^ N ^ K).choice(M, 64, replace=False)
    # the first, middle and last rows, and (wte gradient) both sides of the
    # row split that runs the tail of the tile grid with split-K
    extra = [0, M // 2, M - 1] + ([43519, 43520, 50303 - 256] if M == 50304 else [])
    rows = np.unique(np.concatenate([rows, np.array(extra)]))
    ridx = torch.from_numpy(rows).cuda()
    Am = (A[ridx] if akm else A[:, ridx].T).float().cpu().numpy().astype(np.float64)
    Bm = (B if bkm else B.T).float().cpu().numpy().astype(np.float64)
    ref = Am @ Bm.T
    got = out[ridx].float().cpu().numpy()
    assert rel_l2(got, ref) < 4e-3
    if not akm:
        # weight-gradient form: fp32 accumulation into an existing gradient
        # (split over K when the output grid is small)
        init = torch.randn((M, N), device="cuda", generator=gen)
        acc = init.clone()
        g.gemm(BF16, akm, bkm, M, N, K, A, A.shape[1], B, B.shape[1], "acc_f32", acc, N)
        torch.cuda.synchronize()
        ref2 = init[ridx].cpu().numpy().astype(np.float64) + ref
        assert rel_l2(acc[ridx].cpu().numpy(), ref2) < 1e-5


@pytest.mark.parametrize("M,N,K,ldo", [(1000, 3072, 768, 3072), (16384, 3072, 768, 3072),
                                      (520, 1001, 200, 1001)])
def test_gelu_backward_column_sums(M, N, K, ldo):
    """The GELU-backward product's column sums per 64-row block (the fc bias
    gradient's first stage) equal the fp64 sums of the output it stores, and
    that output is bit-identical to the product's without them: full size,
    a ragged last row block, and a ragged odd width (element-wise stores)."""
    rng = np.random.default_rng(M + N)
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    B = bf16_round(0.05 * rng.standard_normal((N, K)).astype(np.float32))
    aux = bf16_round(rng.standard_normal((M, N)).astype(np.float32))
    Abuf, lda = _store(A, True, M, K, 0, rng, 0.0)
    Bbuf, ldb = _store(B, False, N, K, 0, rng, 0.0)
    dA, dB = to_dev(Abuf, torch.bfloat16), to_dev(Bbuf, torch.bfloat16)
    daux = to_dev(aux, torch.bfloat16)
    assert g.gemm_colsum_ok(BF16, True, False, M, N, K, lda, ldb, "gelu_bwd")
    nb, ldcs = (M + 63) // 64, N + N % 2
    cs = torch.full((nb, ldcs), float("nan"), device="cuda")
    plain = torch.zeros((M, ldo), dtype=torch.bfloat16, device="cuda")
    fused = torch.zeros_like(plain)
    g.gemm(BF16, True, False, M, N, K, dA, lda, dB, ldb, "gelu_bwd", plain, ldo, aux=daux, ldx=N)
    g.gemm(BF16, True, False, M, N, K, dA, lda, dB, ldb, "gelu_bwd", fused, ldo, aux=daux, ldx=N,
           colsum=cs, ldcs=ldcs)
    torch.cuda.synchronize()
    out = host(fused)[:, :N]
    assert np.array_equal(out, host(plain)[:, :N])
    rows = np.zeros((nb * 64, N))
    rows[:M] = out
    expect = rows.reshape(nb, 64, N).sum(axis=1)
    got = host(cs)[:, :N]
    np.testing.assert_allclose(got, expect, rtol=1e-5, atol=1e-6 * np.abs(out).max())
    # the output itself: the product's definition on sampled rows
    idx = rng.choice(M, size=min(M, 64), replace=False)
    ref = (A[idx].astype(np.float64) @ B.astype(np.float64).T) * oracle.gelu_grad(
        aux[idx].astype(np.float64))
    assert rel_l2(out[idx], ref) < 1e-2


@pytest.mark.parametrize("M,N", [(768, 3072), (3072, 768), (768, 768), (2304, 768)])
def test_gemm_weight_gradient_split_k(M, N):
    """The four per-layer weight-gradient products at the 124M shapes
    (K = B*T = 16384), fp32-accumulated, full output against fp64."""
    K = 16384
    print(f"gemm dW M={M} N={N} K={K} ws={g.gemm_workspace_bytes(BF16, M, N, K, 'acc_f32')}",
          flush=True)
    gen = torch.Generator(device="cuda").manual_seed(M + N)
    A = torch.randn((K, M), device="cuda", generator=gen).to(torch.bfloat16)
    B = torch.randn((K, N), device="cuda", generator=gen).to(torch.bfloat16)
    init = torch.randn((M, N), device="cuda", generator=gen)
    out = init.clone()
    g.gemm(BF16, False, False, M, N, K, A, M, B, N, "acc_f32", out, N)
    ref = init.double() + A.double().T @ B.double()
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy(), ref.cpu().numpy()) < 1e-5


def _acc_group_case(dt, shapes, K, seed, ws="auto"):
    """out_i = init_i + A_i^T B_i through gemm_acc_group; A_i (K, M_i), B_i
    (K, N_i) row-major, reference in fp64 on the host."""
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    As, Bs, outs, refs = [], [], [], []
    for M, N in shapes:
        A = rng.standard_normal((K, M)).astype(np.float32)
        B = rng.standard_normal((K, N)).astype(np.float32)
        if dt == BF16:
            A, B = bf16_round(A), bf16_round(B)
        init = rng.standard_normal((M, N)).astype(np.float32)
        As.append(to_dev(A, tdt))
        Bs.append(to_dev(B, tdt))
        outs.append(to_dev(init))
        refs.append(init.astype(np.float64) + A.astype(np.float64).T @ B.astype(np.float64))
    Ms, Ns = [m for m, _ in shapes], [n for _, n in shapes]
    nb = g.gemm_acc_group_workspace_bytes(dt, Ms, Ns, K, Ms, Ns)
    wsb = None
    if ws == "none":
        wsb = torch.empty(8, dtype=torch.uint8, device="cuda")
    print(f"acc group dt={dt} shapes={shapes} K={K} ws={nb} ({ws})", flush=True)
    g.gemm_acc_group(dt, Ms, Ns, K, As, Ms, Bs, Ns, outs, Ns, ws=wsb)
    torch.cuda.synchronize()
    for o, r in zip(outs, refs):
        assert rel_l2(host(o), r) < 1e-5, (o.shape, rel_l2(host(o), r))
    return nb


def test_weight_gradients_of_a_layer_in_one_launch():
    """The four weight-gradient products of a 124M layer (fcp, fc, proj, qkv)
    as one launch, K = 4096 tokens (split in two), full outputs vs fp64."""
    nb = _acc_group_case(BF16, [(768, 3072), (3072, 768), (768, 768), (2304, 768)], 4096, 11)
    assert nb == 2 * 4 * (768 * 3072 * 2 + 768 * 768 + 2304 * 768)


@pytest.mark.parametrize("K", [1000, 2056])
def test_weight_gradient_group_ragged(K):
    """Widths that leave ragged tiles (C = 384) and K with a partial last
    k-tile; K = 1000 runs unsplit, K = 2056 split in two."""
    _acc_group_case(BF16, [(384, 1536), (1536, 384), (384, 384), (1152, 384)], K, 12)


def test_weight_gradients_of_two_layers_in_one_launch():
    """Eight products (two 124M layers): 216 tiles in one round, no K split;
    K = 1000 leaves a partial last k-tile."""
    layer = [(768, 3072), (3072, 768), (768, 768), (2304, 768)]
    nb = _acc_group_case(BF16, layer + layer, 1000, 17)
    assert nb == 0  # no split, no partials


def test_weight_gradients_of_a_350m_layer_in_one_launch():
    """The four weight-gradient products of a GPT-2 350M layer (C = 1024) at
    the full token count K = 16384: 192 tiles, one launch without a K split
    (the way the 350M backward runs each layer, since two layers' 384 tiles
    exceed one round of the CUs); full outputs against fp64."""
    nb = _acc_group_case(BF16, [(1024, 4096), (4096, 1024), (1024, 1024), (3072, 1024)], 16384, 21)
    assert nb == 0


def test_fc_projection_350m_bias_residual_epilogue():
    """The 350M fc-projection forward (M = 16384, N = 1024, K = 4096) with
    its bias + residual epilogue, 64 sampled rows against fp64."""
    M, N, K = 16384, 1024, 4096
    gen = torch.Generator(device="cuda").manual_seed(4096)
    A = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
    B = (0.05 * torch.randn((N, K), device="cuda", generator=gen)).to(torch.bfloat16)
    bias = torch.randn(N, device="cuda", generator=gen)
    resid = torch.randn((M, N), device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    print(f"gemm 350M fc projection bias_resid M={M} N={N} K={K}", flush=True)
    g.gemm(BF16, True, True, M, N, K, A, K, B, K, "bias_resid", out, N, bias=bias, resid=resid,
           ldr=N)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(7).choice(M, 64, replace=False),
                                     np.array([0, M - 1])]))
    ridx = torch.from_numpy(rows).cuda()
    ref = (A[ridx].double() @ B.double().T + bias.double() + resid[ridx].double()).cpu().numpy()
    assert rel_l2(out[ridx].float().cpu().numpy(), ref) < 4e-3


def test_weight_gradient_group_fallbacks():
    """Without workspace, with one or three products, and in fp32 (one
    product per launch) the results are the same products."""
    _acc_group_case(BF16, [(768, 3072), (2304, 768)], 2048, 13, ws="none")
    _acc_group_case(BF16, [(512, 256)], 2048, 14)
    _acc_group_case(BF16, [(256, 128), (512, 512), (304, 136)], 512, 15)
    _acc_group_case(FP32, [(96, 40), (64, 64)], 200, 16)


# ------------------------------------------------------------------ attention
def attention_case(dt, B, T, H, hd, seed):
    rng = np.random.default_rng(seed)
    C = H * hd
    qkv = rng.standard_normal((B * T, 3 * C)).astype(np.float32)
    dout = rng.standard_normal((B * T, C)).astype(np.float32)
    if dt == BF16:
        qkv, dout = bf16_round(qkv), bf16_round(dout)
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    d_qkv = to_dev(qkv, tdt)
    d_out = torch.empty((B * T, C), dtype=tdt, device="cuda")
    d_lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    g.attention_forward(dt, d_out, d_lse, d_qkv, B, T, H, hd)
    d_dout = to_dev(dout, tdt)
    d_dqkv = torch.full((B * T, 3 * C), float("nan"), dtype=tdt, device="cuda")
    scratch = torch.empty(g.attention_backward_scratch_bytes(B, T, H), dtype=torch.uint8,
                          device="cuda")
    g.attention_backward(dt, d_dqkv, d_dout, d_qkv, d_out, d_lse, B, T, H, hd, scratch)
    torch.cuda.synchronize()
    return qkv, dout, host(d_out), host(d_lse), host(d_dqkv)


def oracle_attention(qkv, dout, B, T, H):
    q, k, v = oracle.split_heads(qkv.astype(np.float64), B, T, H)
    o, p = oracle.causal_attention_forward(q, k, v)
    do = dout.astype(np.float64).reshape(B, T, H, -1).transpose(0, 2, 1, 3)
    dq, dk, dv = oracle.causal_attention_backward(do, q, k, v, p)
    dqkv = np.concatenate([oracle.merge_heads(dq), oracle.merge_heads(dk), oracle.merge_heads(dv)], 1)
    hd = q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
    mx = s.max(-1, keepdims=True)
    lse = (mx + np.log(np.exp(s - mx).sum(-1, keepdims=True)))[..., 0]
    return oracle.merge_heads(o), lse, dqkv


@pytest.mark.parametrize("dt", [FP32, BF16])
@pytest.mark.parametrize("B,T,H,hd", [(2, 100, 3, 64), (3, 64, 4, 16), (1, 1, 2, 64), (2, 130, 2, 16),
                                      (1, 257, 2, 64)])
def test_attention_matches_oracle(dt, B, T, H, hd):
    print(f"attention dt={dt} B={B} T={T} H={H} hd={hd}", flush=True)
    qkv, dout, out, lse, dqkv = attention_case(dt, B, T, H, hd, seed=T + hd)
    ro, rlse, rdqkv = oracle_attention(qkv, dout, B, T, H)
    if dt == FP32:
        assert rel_l2(out, ro) < 1e-5
        assert np.max(np.abs(lse - rlse)) < 1e-4
        assert rel_l2(dqkv, rdqkv) < 1e-4
    else:
        assert rel_l2(out, ro) < 1e-2
        assert np.max(np.abs(lse - rlse)) < 2e-2
        C = H * hd
        for part in range(3):
            sl = slice(part * C, (part + 1) * C)
            assert cosine(dqkv[:, sl], rdqkv[:, sl]) > 0.999
            assert rel_l2(dqkv[:, sl], rdqkv[:, sl]) < 3e-2


def test_attention_t1_returns_v():
    """With one position the output is v and lse is the single score."""
    qkv, dout, out, lse, dqkv = attention_case(FP32, 3, 1, 2, 64, seed=5)
    C = 128
    assert np.allclose(out, qkv[:, 2 * C:], rtol=1e-6, atol=1e-6)
    assert np.all(dqkv[:, :2 * C] == 0)  # dq = dk = 0: softmax over one element
    assert np.allclose(dqkv[:, 2 * C:], dout, rtol=1e-6)


def test_attention_gpt2_124m_sampled_heads():
    """bf16 at B=16, T=1024, H=12, hd=64; two (b, h) slices vs the oracle:
    output rel-L2 <= 1e-2, log-sum-exp within 2e-2, dq / dk / dv cosine >=
    0.999 and rel-L2 <= 3e-2 (the bars of the small bf16 cases)."""
    B, T, H, hd = 16, 1024, 12, 64
    print(f"attention 124M bf16 B={B} T={T} H={H}", flush=True)
    qkv, dout, out, lse, dqkv = attention_case(BF16, B, T, H, hd, seed=11)
    C = H * hd
    for b, h in [(0, 0), (13, 7)]:
        rows = slice(b * T, (b + 1) * T)
        cols = np.r_[h * hd:(h + 1) * hd, C + h * hd:C + (h + 1) * hd,
                     2 * C + h * hd:2 * C + (h + 1) * hd]
        sub = qkv[rows][:, cols]
        ro, rlse, rd = oracle_attention(sub, dout[rows][:, h * hd:(h + 1) * hd], 1, T, 1)
        assert rel_l2(out[rows][:, h * hd:(h + 1) * hd], ro) < 1e-2
        assert np.max(np.abs(lse[b, h] - rlse[0, 0])) < 2e-2
        got = dqkv[rows][:, cols]
        for part in range(3):
            sl = slice(part * hd, (part + 1) * hd)
            assert cosine(got[:, sl], rd[:, sl]) > 0.999
            assert rel_l2(got[:, sl], rd[:, sl]) < 3e-2


@pytest.mark.parametrize("B,T,H", [(2, 100, 3), (1, 300, 2), (16, 1024, 12)])
def test_attention_backward_column_sums(B, T, H):
    """The attention backward's column sums of dqkv per 128-row block (the qkv
    bias gradient's first stage) equal the fp64 sums of the dqkv it stores,
    and that dqkv is bit-identical to the backward's without them: ragged T
    (a partial last block, T below one block) and the GPT-2 124M shape."""
    hd, C = 64, H * 64
    assert g.attention_colsum_ok(BF16, hd)
    rng = np.random.default_rng(B * T + H)
    qkv = bf16_round(rng.standard_normal((B * T, 3 * C)).astype(np.float32))
    dout = bf16_round(rng.standard_normal((B * T, C)).astype(np.float32))
    d_qkv, d_dout = to_dev(qkv, torch.bfloat16), to_dev(dout, torch.bfloat16)
    d_out = torch.empty((B * T, C), dtype=torch.bfloat16, device="cuda")
    d_lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    g.attention_forward(BF16, d_out, d_lse, d_qkv, B, T, H, hd)
    scratch = torch.empty(g.attention_backward_scratch_bytes(B, T, H), dtype=torch.uint8,
                          device="cuda")
    nblk = (T + 127) // 128
    cs = torch.full((B * nblk, 3 * C), float("nan"), device="cuda")
    plain = torch.full((B * T, 3 * C), float("nan"), dtype=torch.bfloat16, device="cuda")
    fused = torch.full_like(plain, float("nan"))
    g.attention_backward(BF16, plain, d_dout, d_qkv, d_out, d_lse, B, T, H, hd, scratch)
    g.attention_backward(BF16, fused, d_dout, d_qkv, d_out, d_lse, B, T, H, hd, scratch, colsum=cs)
    torch.cuda.synchronize()
    got_dqkv = host(fused)
    assert np.array_equal(got_dqkv, host(plain))
    rows = np.zeros((B, nblk * 128, 3 * C))
    rows[:, :T] = got_dqkv.reshape(B, T, 3 * C)
    expect = rows.reshape(B * nblk, 128, 3 * C).sum(axis=1)
    np.testing.assert_allclose(host(cs), expect, rtol=1e-5, atol=1e-6 * np.abs(got_dqkv).max())
