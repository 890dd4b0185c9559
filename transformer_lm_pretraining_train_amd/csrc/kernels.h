// Host-side launchers for the gfx950 kernels.  Pointers are device
// pointers; `dt` selects the activation element type (0 = fp32, 1 = bf16).
// Every launcher enqueues on `s` and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

enum DType { F32 = 0, BF16 = 1 };

inline size_t dsize(int dt) { return dt == BF16 ? 2 : 4; }

// ---- embedding
hipError_t encoder_forward(int dt, void* out, const int32_t* tok, const float* wte, const float* wpe,
                           int M, int T, int C, int V, int* err_flag, hipStream_t s);
hipError_t encoder_backward_wpe(int dt, float* dwpe, const void* dx, int B, int T, int C,
                                hipStream_t s);
// dwte[tok[m]] += dx[m], each token's rows summed in position order through a
// counting sort of the positions (no float atomics; ids clamped to [0, V)).
size_t encoder_backward_wte_scratch_bytes(int M, int V, int C);
hipError_t encoder_backward_wte(int dt, float* dwte, const void* dx, const int32_t* tok, int M,
                                int C, int V, void* scratch, hipStream_t s);

// ---- fixed-order column reductions of partial sums
// out_k[c] += sum_{b < nb} partial[b * stride + k * C + c] for c < ncols
// (k = c / C selects out0, out1 or out2; a null out_k is skipped).
struct ColReduce {
  float* out0;
  float* out1;
  float* out2;
  const float* partial;
  int nb, C, stride, ncols;
};
// Several such reductions in as few launches as possible (the LayerNorm and
// bias-gradient column sums of a whole backward pass, deferred to its end).
hipError_t column_reduce_batched(const ColReduce* d, int n, hipStream_t s);

// ---- LayerNorm
hipError_t layernorm_forward(int dt, void* out, float* mean, float* rstd, const void* inp,
                             const float* w, const float* b, int M, int C, float eps, hipStream_t s);
// dres = dx (accumulate false) or dres = dres_in + dx (dres_in null or
// equal to dres: in place); dw, db += column sums of dy*xhat and dy; dsum
// (if not null) += column sums of the new dres.  Two-stage, partials in
// scratch.  With `defer` the partials stay in scratch and their reduction
// is returned in *defer instead of being launched.
size_t layernorm_backward_scratch_bytes(int M, int C);
hipError_t layernorm_backward(int dt, void* dres, const void* dres_in, float* dw, float* db,
                              float* dsum, bool accumulate, const void* dy, const void* inp,
                              const float* mean, const float* rstd, const float* w, int M, int C,
                              void* scratch, hipStream_t s, ColReduce* defer = nullptr);

// ---- bias gradient: db[n] += sum_m dy[m, n] (two-stage, partials in scratch)
size_t bias_grad_scratch_bytes(int M, int N);
hipError_t bias_grad(int dt, float* db, const void* dy, int M, int N, int64_t ldy, void* scratch,
                     hipStream_t s,
                     ColReduce* defer = nullptr);

// ---- cross-entropy over the padded vocabulary (row pitch ldl >= Vp)
hipError_t crossentropy_forward(int dt, float* losses, float* lse, int32_t* argmax,
                                const void* logits, int64_t ldl, const int32_t* targets, int M,
                                int V, int* err_flag, hipStream_t s);
hipError_t mean_loss(float* out, const float* losses, int M, hipStream_t s);
// The forward above plus the logit gradient into dz (same pitch):
// dz = seed * (softmax - onehot) for columns < V, 0 for V..ldl-1.  One read
// of the logits when a row fits the workgroup's registers (bf16: ldl <= 65536).
hipError_t crossentropy_fused(int dt, float* losses, float* lse, int32_t* argmax, void* dz,
                              const void* logits, int64_t ldl, const int32_t* targets, int M,
                              int V, float seed, int* err_flag, hipStream_t s);

// ---- attention (qkv rows of 3C: [q | k | v], head h at h*hd)
hipError_t attention_forward(int dt, void* out, float* lse, const void* qkv, int B, int T, int H,
                             int hd, hipStream_t s);
// dqkv fully written.  scratch: attention_backward_scratch_bytes.  colsum
// (where attention_colsum_ok(), else hipErrorNotSupported; may be null):
// colsum[(b * ceil(T/128) + i) * 3C + c] = sum of the stored dqkv[b*T + t, c]
// over t in [128 i, 128 i + 128) ∩ [0, T), for all 3C columns, in a fixed
// order (the qkv bias gradient's first stage).
size_t attention_backward_scratch_bytes(int B, int T, int H);
bool attention_colsum_ok(int dt, int hd);
inline int attention_colsum_blocks(int B, int T) { return B * ((T + 127) / 128); }
hipError_t attention_backward(int dt, void* dqkv, const void* dout, const void* qkv,
                              const void* out, const float* lse, int B, int T, int H, int hd,
                              void* scratch, hipStream_t s, float* colsum = nullptr);
// The same without a scratch argument: D lives in a fixed device array of
// kNoAllocAttnScratchFloats floats (one per GPU, kept until the process
// ends; calls that overlap on one GPU race on it).  hipErrorInvalidValue
// when B*H*T exceeds it.  Allocates nothing.
constexpr int kNoAllocAttnScratchFloats = 1 << 20;
constexpr int kMaxDevices = 64;
hipError_t attention_backward_noalloc(int dt, void* dqkv, const void* dout, const void* qkv,
                                      const void* out, const float* lse, int B, int T, int H,
                                      int hd, hipStream_t s, float* colsum);

// ---- GEMM: C(m, n) = sum_k A(m, k) B(n, k), then an epilogue.
// a_kmajor: A(m,k) = A[m*lda + k], else A[k*lda + m]; likewise b_kmajor for
// B(n,k) = B[n*ldb + k] or B[k*ldb + n].  Leading dimensions are in
// elements, multiples of 8, and each row must be readable up to
// round_up(extent, 8).
enum EpiMode {
  EPI_STORE = 0,       // out = acc
  EPI_BIAS = 1,        // out = acc + bias[n]
  EPI_BIAS_RESID = 2,  // out = acc + bias[n] + resid[m, n]
  EPI_BIAS_GELU = 3,   // out = acc + bias[n]; out2 = gelu(out); with dgelu out = gelu'(that)
  EPI_GELU_BWD = 4,    // out = acc * T(gelu'(aux[m, n])); out2 (if not null) = gelu(aux[m, n]);
                       // with dgelu aux holds gelu' already: out = acc * aux[m, n]
  EPI_ACC_F32 = 5,     // out (fp32) += acc
  EPI_PARTIAL = 6,     // internal: split-K partial tile, fp32
  EPI_ROWSTATS = 7,    // internal: softmax row statistics, see gemm_rowstats()
  EPI_DLOGITS = 8      // internal: cross-entropy logit gradient, see gemm_dlogits()
};
struct Epilogue {
  int mode;
  void* out;
  int64_t ldo;
  const float* bias;
  const void* resid;
  int64_t ldr;
  void* out2;
  int64_t ldo2;
  const void* aux;
  int64_t ldx;
  // EPI_GELU_BWD only, and only where gemm_colsum_ok(): if not null, also
  // colsum[b * ldcs + n] = sum of the stored out[m, n] (as rounded) over the
  // 64 rows m of block b, for b < gemm_colsum_blocks(M) and n < N: per-block
  // column sums of the output (a bias gradient's first stage), in a fixed
  // order.
  float* colsum;
  int64_t ldcs;
  // GELU derivative stored instead of the pre-activation.  EPI_BIAS_GELU: out
  // receives GELU'(h) of the stored (rounded) pre-activation h in place of h
  // (out2 still GELU(h)).  EPI_GELU_BWD: aux holds that GELU'(h), and out =
  // acc * aux; out2 must be null.  Without the flag EPI_GELU_BWD rounds its
  // GELU'(aux) to the element type before multiplying, so that both ways
  // give the same bits.
  int dgelu;
  // EPI_DLOGITS only: column n of the product is vocabulary entry col0 + n.
  const float* lse;
  const int32_t* targets;
  int col0, vocab;
  float scale;
};
// Split-K (used for fp32-accumulating products with few output tiles and a
// long K) needs gemm_workspace_bytes() of scratch in `ws`.
size_t gemm_workspace_bytes(int dt, int M, int N, int K, int mode);
// persistent = false launches one workgroup per output tile instead of one
// per CU looping over tiles: slower alone, but while another stream's kernel
// holds most CUs the ones left free keep taking tiles.
hipError_t gemm(int dt, bool a_kmajor, bool b_kmajor, int M, int N, int K, const void* A,
                int64_t lda, const void* B, int64_t ldb, const Epilogue& e, hipStream_t s,
                void* ws = nullptr, size_t ws_bytes = 0, bool persistent = true);
// Whether gemm() can produce Epilogue::colsum for this product (it returns
// hipErrorNotSupported for a colsum it cannot produce), and the number of
// 64-row blocks it then writes.
bool gemm_colsum_ok(int dt, bool a_kmajor, bool b_kmajor, int M, int N, int K, int64_t lda,
                    int64_t ldb, int mode);
inline int gemm_colsum_blocks(int M) { return (M + 63) / 64; }
// Softmax statistics of the rows of z = bf16(A B^T) (A, B k-major) without
// storing z -- the loss of the tied head without its logits: for each row m
// and each 128-column group h (columns [128 h, 128 h + 128) ∩ [0, V)),
// stats[m * ld + h] = (max z, sum exp(z - max)) over those columns ((-inf, 0)
// if none), and tgt[m] = z[m, y] with y = target[m] clamped to [0, V).  Only
// bf16 products on the 256 x 256 tiles (gemm_rowstats_ok); ld >=
// gemm_rowstats_cols(N).
bool gemm_rowstats_ok(int dt, int M, int N, int K, int64_t lda, int64_t ldb);
inline int gemm_rowstats_cols(int N) { return 2 * ((N + 255) / 256); }
hipError_t gemm_rowstats(int M, int N, int K, const void* A, int64_t lda, const void* B,
                         int64_t ldb, int V, const int32_t* target, float2* stats, int64_t ld,
                         float* tgt, hipStream_t s);
// loss[m] = log sum_h stats[m, h].s exp(stats[m, h].max - M) + M - tgt[m]
// (M the largest max), combining each row's gemm_rowstats groups in a
// fixed order; lse[m] also written; out-of-range targets set bit 2 of
// err_flag.
hipError_t rowstats_loss(float* losses, float* lse, const float2* stats, int64_t ld, int ncols,
                         const float* tgt, const int32_t* targets, int M, int V, int* err_flag,
                         hipStream_t s);
// The gradient of the mean cross-entropy for one block of vocabulary
// columns without the logits in memory: z = bf16(A B^T) for rows m < M and
// the N columns n of B (B = rows col0 .. col0 + N - 1 of the tied head; A,
// B k-major), then out[m * ldo + n] = bf16(scale * (exp(z - lse[m]) -
// [col0 + n == y])) with y = targets[m] clamped to [0, V), and 0 where
// col0 + n >= V -- what the cross-entropy computes from the stored logits.
// Only bf16 products on the large tiles (gemm_dlogits_ok: also ldo a
// multiple of 8).
bool gemm_dlogits_ok(int dt, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldo);
hipError_t gemm_dlogits(int M, int N, int K, const void* A, int64_t lda, const void* B,
                        int64_t ldb, const float* lse, const int32_t* targets, int col0, int V,
                        float scale, void* out, int64_t ldo, hipStream_t s);
// out (fp32, pitch ldo) += sum_k A[k * lda + m] B[k * ldb + n] for m < M,
// n < N: a weight gradient dW += dy^T x with dy and x stored row-major.
struct AccItem {
  int M, N;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  float* out;
  int64_t ldo;
};
// Up to eight such products with a common K in one launch (bf16), else one
// gemm() each; split-K partials need gemm_acc_group_workspace_bytes() in ws.
// gemm_acc_group_splits: the K split of that launch, 0 if it does not apply.
int gemm_acc_group_splits(int dt, int n, const AccItem* items, int K);
size_t gemm_acc_group_workspace_bytes(int dt, int n, const AccItem* items, int K);
hipError_t gemm_acc_group(int dt, int n, const AccItem* items, int K, void* ws, size_t ws_bytes,
                          hipStream_t s);

// ---- optimizer
struct DecayMap {  // which flat elements belong to 2-D tensors
  int64_t layer0, layer_size, n_layer_end;
  int64_t qkvw0, qkvw1, projw0, projw1, fcw0, fcw1, fcpw0, fcpw1;  // offsets within a layer
};
size_t grad_norm_scratch_bytes();
// writes norm (float) and clip scale min(1, clip/norm) to scratch; if
// norm_out != nullptr also copies the norm there.
hipError_t grad_norm(const float* g, int64_t n, float clip, void* scratch, float* norm_out,
                     hipStream_t s);
const float* grad_norm_result(const void* scratch);  // device pointer: [norm, scale]
hipError_t adamw(float* p, const float* g, float* m, float* v, void* shadow, int64_t n,
                 float lr, float b1, float b2, float eps, float wd, float bc1, float bc2,
                 const float* norm_scale, DecayMap dm, hipStream_t s);
hipError_t fill_f32(float* p, float value, int64_t n, hipStream_t s);
hipError_t fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s);
hipError_t cast_f32_to_bf16(void* dst, const float* src, int64_t n, hipStream_t s);

}  // namespace gk
