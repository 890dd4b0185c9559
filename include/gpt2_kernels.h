/*
 * gpt2_kernels.h -- kernel-level entry points of libgpt2.so, for unit tests
 * and micro-benchmarks of the two matrix-core kernels of the GPT-2 step in
 * isolation.  The training step itself only needs gpt2.h.
 *
 * Conventions as in gpt2.h: dev_* are device pointers owned by the caller;
 * calls enqueue on `hip_stream` (a hipStream_t, NULL = default stream) and
 * return 0 or a negative GPT2_E* code with the message in
 * gpt2_last_error().  Element type: dtype GPT2_FP32 -> float,
 * GPT2_BF16 -> bfloat16 (uint16 storage); bias is always fp32.
 */
#ifndef GPT2_KERNELS_H
#define GPT2_KERNELS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of gpt2k_gemm. */
enum {
  GPT2K_EPI_STORE = 0,      /* out = acc */
  GPT2K_EPI_BIAS = 1,       /* out = acc + bias[n] */
  GPT2K_EPI_BIAS_RESID = 2, /* out = acc + bias[n] + resid[m, n] */
  GPT2K_EPI_BIAS_GELU = 3,  /* out = acc + bias[n]; out2 = gelu_tanh(out) */
  GPT2K_EPI_GELU_BWD = 4,   /* out = acc * gelu_tanh'(aux[m, n]), the derivative rounded to
                               `dtype` first (as the model's forward stores it when it keeps
                               the GELU output); if dev_out2 is not NULL also
                               out2 = gelu_tanh(aux[m, n]) (the activation recompute) */
  GPT2K_EPI_ACC_F32 = 5     /* out (always fp32) += acc */
};

/* C(m, n) = sum_{k < K} A(m, k) B(n, k) for m < M, n < N, then the epilogue,
 * with fp32 accumulation.  The linear layers of the model are this product
 * with W stored (out, in): y = x W^T (A, B k-major), dx = dy W (A k-major,
 * B n-major), dW += dy^T x (A m-major, B n-major).  The linear layers are
 * the qkv, output-projection and MLP products of each block (qntz.me "From 0
 * to 1 build GPT", building the Transformer) and the tied head; their
 * gradients follow from differentiating y = x W^T + b.
 *   a_kmajor != 0: A(m, k) = A[m*lda + k], else A[k*lda + m];
 *   b_kmajor != 0: B(n, k) = B[n*ldb + k], else B[k*ldb + n].
 * Leading dimensions (elements) must be multiples of 8, and each row of A
 * and B must be readable up to round_up(extent, 8) elements.  Output
 * leading dimensions ldo, ldr, ldo2, ldx are in elements.  Pointers not used
 * by the epilogue may be NULL.  For GPT2K_EPI_ACC_F32 the K range may be
 * split over several workgroups whose fp32 partial tiles are summed in a
 * fixed order; that needs gpt2k_gemm_workspace_bytes() of scratch in dev_ws
 * (with less, the product runs unsplit). */
size_t gpt2k_gemm_workspace_bytes(int dtype, int M, int N, int K, int epilogue);
int gpt2k_gemm(int dtype, int a_kmajor, int b_kmajor, int M, int N, int K, const void* dev_A,
               int64_t lda, const void* dev_B, int64_t ldb, int epilogue, void* dev_out,
               int64_t ldo, const float* dev_bias, const void* dev_resid, int64_t ldr,
               void* dev_out2, int64_t ldo2, const void* dev_aux, int64_t ldx, void* dev_ws,
               size_t ws_bytes, void* hip_stream);

/* gpt2k_gemm that also writes per-block column sums of its output, the
 * first stage of a bias gradient (for y = x W^T + b, the gradient of b is
 * the sum of the output gradient over all token rows; the linear layers
 * are those of qntz.me "From 0 to 1 build GPT", building the Transformer):
 *   colsum[b*ldcs + n] = sum over the rows m in [64b, 64b + 64) ∩ [0, M) of
 *   the stored out(m, n), as rounded to `dtype`, for b < ceil(M / 64), n < N,
 * each sum in a fixed order (deterministic).  dev_colsum (fp32, 8-byte
 * aligned, ldcs even and >= N) may be NULL: then this is gpt2k_gemm.  Only
 * products for which gpt2k_gemm_colsum_ok() returns 1 can produce the sums
 * (bf16, GPT2K_EPI_GELU_BWD, a size that runs on the large-tile kernels);
 * for others a non-NULL dev_colsum returns GPT2_EINVAL and nothing runs. */
int gpt2k_gemm_colsum_ok(int dtype, int a_kmajor, int b_kmajor, int M, int N, int K, int64_t lda,
                         int64_t ldb, int epilogue);
int gpt2k_gemm_colsum(int dtype, int a_kmajor, int b_kmajor, int M, int N, int K,
                      const void* dev_A, int64_t lda, const void* dev_B, int64_t ldb, int epilogue,
                      void* dev_out, int64_t ldo, const float* dev_bias, const void* dev_resid,
                      int64_t ldr, void* dev_out2, int64_t ldo2, const void* dev_aux, int64_t ldx,
                      float* dev_colsum, int64_t ldcs, void* dev_ws, size_t ws_bytes,
                      void* hip_stream);

/* Weight gradients of up to eight linear layers over the same K tokens:
 * out_i(m, n) += sum_{k < K} A_i[k*lda_i + m] B_i[k*ldb_i + n] for
 * m < M_i, n < N_i, i < n, 1 <= n <= 8 (dW += dy^T x with dy, x stored
 * row-major: the weight gradient of y = x W^T + b for each linear layer of a
 * block, qntz.me "From 0 to 1 build GPT", building the Transformer).  M, N, lda, ldb, ldo are host arrays of n entries; dev_A,
 * dev_B, dev_out host arrays of n device pointers; out_i is fp32, A_i and
 * B_i are of `dtype`.  In bf16 the products run as one launch whose K is
 * split in a fixed order when gpt2k_gemm_acc_group_workspace_bytes() of
 * scratch is given in dev_ws; otherwise (and in fp32) as gpt2k_gemm calls
 * with GPT2K_EPI_ACC_F32, one per product.  The products' outputs must not
 * overlap each other or their inputs.  Returns GPT2_EINVAL for n outside
 * 1..8, a NULL pointer, negative sizes or pitches not multiples of 8. */
size_t gpt2k_gemm_acc_group_workspace_bytes(int dtype, int n, const int* M, const int* N, int K,
                                            const int64_t* lda, const int64_t* ldb);
int gpt2k_gemm_acc_group(int dtype, int n, const int* M, const int* N, int K,
                         const void* const* dev_A, const int64_t* lda, const void* const* dev_B,
                         const int64_t* ldb, float* const* dev_out, const int64_t* ldo,
                         void* dev_ws, size_t ws_bytes, void* hip_stream);

/* Causal self-attention forward on qkv (B*T, 3C) rows [q | k | v], head h at
 * columns h*hd within each third, C = H*hd: out (B*T, C) = softmax(q k^T /
 * sqrt(hd), j <= i) v per head, lse (B, H, T) fp32 = log sum_j exp(scores)
 * ("Let's reproduce GPT-2 (124M)", GPU optimisation ladder: FlashAttention,
 * which never stores the T x T matrix). */
int gpt2k_attention_forward(int dtype, void* dev_out, float* dev_lse, const void* dev_qkv, int B,
                            int T, int H, int hd, void* hip_stream);

/* Backward of gpt2k_attention_forward: writes dqkv (B*T, 3C) in full from
 * dout (B*T, C), the forward's qkv, out and lse.  dev_scratch must hold
 * gpt2k_attention_backward_scratch_bytes(B, T, H) bytes. */
size_t gpt2k_attention_backward_scratch_bytes(int B, int T, int H);
int gpt2k_attention_backward(int dtype, void* dev_dqkv, const void* dev_dout, const void* dev_qkv,
                             const void* dev_out, const float* dev_lse, int B, int T, int H,
                             int hd, void* dev_scratch, void* hip_stream);

/* gpt2k_attention_backward that also writes per-block column sums of dqkv,
 * the first stage of the qkv bias gradient (the sum of d qkv over all
 * token rows, the bias gradient of the qkv linear layer of qntz.me "From 0
 * to 1 build GPT", building the Transformer):
 *   dev_colsum[(b*ceil(T/128) + i)*3C + c] = sum over t in
 *   [128i, 128i + 128) ∩ [0, T) of the stored dqkv(b*T + t, c)
 * (as rounded to `dtype`; fp32 sums in a fixed order), for every b < B,
 * i < ceil(T/128), c < 3C.  dev_colsum may be NULL (then this is
 * gpt2k_attention_backward); where gpt2k_attention_colsum_ok(dtype, hd) is 0
 * (only bf16 with hd = 64 has them) a non-NULL dev_colsum returns
 * GPT2_EINVAL before anything runs. */
int gpt2k_attention_colsum_ok(int dtype, int hd);
int gpt2k_attention_backward_colsum(int dtype, void* dev_dqkv, const void* dev_dout,
                                    const void* dev_qkv, const void* dev_out,
                                    const float* dev_lse, int B, int T, int H, int hd,
                                    void* dev_scratch, float* dev_colsum, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gpt2k_attention_backward_colsum without the scratch argument.  The
 * per-row values the backward keeps between its two passes live in a fixed
 * device array of 2^20 floats (4 MiB) that the library holds on each GPU it
 * runs on until the process ends; its address is looked up once per device
 * on the first call there.  Allocates nothing (no hipMalloc, no allocating
 * library routine).  Every call on one GPU shares that array: calls that
 * overlap on one GPU (different streams, or host threads) race and must be
 * ordered by the caller.  Nothing in the array needs to start at zero (each
 * call writes every value it reads).  Same arguments, results and errors as
 * gpt2k_attention_backward_colsum, plus GPT2_EINVAL before anything runs
 * when B*H*T > 2^20. */
int gpt2k_attention_backward_noalloc(int dtype, void* dev_dqkv, const void* dev_dout,
                                     const void* dev_qkv, const void* dev_out,
                                     const float* dev_lse, int B, int T, int H, int hd,
                                     float* dev_colsum, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_KERNELS_H */
