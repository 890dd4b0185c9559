// Kernel-level C entry points (gpt2_kernels.h): argument checks, then the
// same launchers the model runtime uses.
#include <cstdio>
#include <string>

#include "../../include/gpt2.h"
#include "../../include/gpt2_kernels.h"
#include "kernels.h"

extern "C" const char* gpt2_last_error(void);
// defined in model.cpp
int gpt2_internal_fail(int code, const char* msg);

using namespace gk;

static int launch_rc(hipError_t e, const char* what) {
  if (e == hipSuccess) return GPT2_OK;
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return gpt2_internal_fail(GPT2_EHIP, m.c_str());
}

extern "C" {

int gpt2k_gemm(int dtype, int a_kmajor, int b_kmajor, int M, int N, int K, const void* A,
               int64_t lda, const void* B, int64_t ldb, int epilogue, void* out, int64_t ldo,
               const float* bias, const void* resid, int64_t ldr, void* out2, int64_t ldo2,
               const void* aux, int64_t ldx, void* ws, size_t ws_bytes, void* stream) {
  return gpt2k_gemm_colsum(dtype, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, epilogue, out, ldo,
                           bias, resid, ldr, out2, ldo2, aux, ldx, nullptr, 0, ws, ws_bytes,
                           stream);
}

int gpt2k_gemm_colsum_ok(int dtype, int a_kmajor, int b_kmajor, int M, int N, int K, int64_t lda,
                         int64_t ldb, int epilogue) {
  return gemm_colsum_ok(dtype, a_kmajor != 0, b_kmajor != 0, M, N, K, lda, ldb, epilogue) ? 1 : 0;
}

int gpt2k_gemm_colsum(int dtype, int a_kmajor, int b_kmajor, int M, int N, int K, const void* A,
                      int64_t lda, const void* B, int64_t ldb, int epilogue, void* out,
                      int64_t ldo, const float* bias, const void* resid, int64_t ldr, void* out2,
                      int64_t ldo2, const void* aux, int64_t ldx, float* colsum, int64_t ldcs,
                      void* ws, size_t ws_bytes, void* stream) {
  if (colsum && !gemm_colsum_ok(dtype, a_kmajor != 0, b_kmajor != 0, M, N, K, lda, ldb, epilogue))
    return gpt2_internal_fail(GPT2_EINVAL, "column sums not available for this product");
  if (colsum && (ldcs < N || ldcs % 2 || reinterpret_cast<uintptr_t>(colsum) % 8))
    return gpt2_internal_fail(GPT2_EINVAL, "ldcs must be even and >= N, colsum 8-byte aligned");
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16)
    return gpt2_internal_fail(GPT2_EINVAL, "dtype must be 0 or 1");
  if (M < 0 || N < 0 || K < 0 || !A || !B || !out)
    return gpt2_internal_fail(GPT2_EINVAL, "bad sizes or NULL operand");
  if (epilogue < EPI_STORE || epilogue > EPI_ACC_F32)
    return gpt2_internal_fail(GPT2_EINVAL, "unknown epilogue");
  if (lda % 8 || ldb % 8) return gpt2_internal_fail(GPT2_EINVAL, "lda, ldb must be multiples of 8");
  if ((epilogue == EPI_BIAS || epilogue == EPI_BIAS_RESID || epilogue == EPI_BIAS_GELU) && !bias)
    return gpt2_internal_fail(GPT2_EINVAL, "epilogue needs bias");
  if (epilogue == EPI_BIAS_RESID && !resid) return gpt2_internal_fail(GPT2_EINVAL, "needs resid");
  if (epilogue == EPI_BIAS_GELU && !out2) return gpt2_internal_fail(GPT2_EINVAL, "needs out2");
  if (epilogue == EPI_GELU_BWD && !aux) return gpt2_internal_fail(GPT2_EINVAL, "needs aux");
  Epilogue e{};
  e.mode = epilogue;
  e.out = out;
  e.ldo = ldo;
  e.bias = bias;
  e.resid = resid;
  e.ldr = ldr;
  e.out2 = out2;
  e.ldo2 = ldo2;
  e.aux = aux;
  e.ldx = ldx;
  e.colsum = colsum;
  e.ldcs = ldcs;
  return launch_rc(gemm(dtype, a_kmajor != 0, b_kmajor != 0, M, N, K, A, lda, B, ldb, e,
                        (hipStream_t)stream, ws, ws_bytes),
                   "gemm");
}

size_t gpt2k_gemm_workspace_bytes(int dtype, int M, int N, int K, int epilogue) {
  return gemm_workspace_bytes(dtype, M, N, K, epilogue);
}

static bool acc_items(int n, const int* M, const int* N, const int64_t* lda, const int64_t* ldb,
                      AccItem* it) {
  if (n < 1 || n > 8 || !M || !N || !lda || !ldb) return false;
  for (int i = 0; i < n; ++i) {
    if (M[i] < 0 || N[i] < 0 || lda[i] % 8 || ldb[i] % 8) return false;
    it[i] = AccItem{M[i], N[i], nullptr, lda[i], nullptr, ldb[i], nullptr, 0};
  }
  return true;
}

size_t gpt2k_gemm_acc_group_workspace_bytes(int dtype, int n, const int* M, const int* N, int K,
                                            const int64_t* lda, const int64_t* ldb) {
  AccItem it[8];
  if (!acc_items(n, M, N, lda, ldb, it) || K < 0) return 0;
  return gemm_acc_group_workspace_bytes(dtype, n, it, K);
}

int gpt2k_gemm_acc_group(int dtype, int n, const int* M, const int* N, int K, const void* const* A,
                         const int64_t* lda, const void* const* B, const int64_t* ldb,
                         float* const* out, const int64_t* ldo, void* ws, size_t ws_bytes,
                         void* stream) {
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16)
    return gpt2_internal_fail(GPT2_EINVAL, "dtype must be 0 or 1");
  AccItem it[8];
  if (!acc_items(n, M, N, lda, ldb, it) || K < 0 || !A || !B || !out || !ldo)
    return gpt2_internal_fail(GPT2_EINVAL, "bad group: n, sizes, pitches or NULL arrays");
  for (int i = 0; i < n; ++i) {
    if (!A[i] || !B[i] || !out[i]) return gpt2_internal_fail(GPT2_EINVAL, "NULL operand");
    it[i].A = A[i];
    it[i].B = B[i];
    it[i].out = out[i];
    it[i].ldo = ldo[i];
  }
  return launch_rc(gemm_acc_group(dtype, n, it, K, ws, ws_bytes, (hipStream_t)stream),
                   "gemm_acc_group");
}

int gpt2k_attention_forward(int dtype, void* out, float* lse, const void* qkv, int B, int T, int H,
                            int hd, void* stream) {
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16)
    return gpt2_internal_fail(GPT2_EINVAL, "dtype must be 0 or 1");
  if (!out || !lse || !qkv || B < 1 || T < 1 || H < 1)
    return gpt2_internal_fail(GPT2_EINVAL, "bad argument");
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return gpt2_internal_fail(GPT2_EINVAL, "head size must be 16, 32, 64 or 128");
  return launch_rc(attention_forward(dtype, out, lse, qkv, B, T, H, hd, (hipStream_t)stream),
                   "attention_forward");
}

size_t gpt2k_attention_backward_scratch_bytes(int B, int T, int H) {
  return attention_backward_scratch_bytes(B, T, H);
}

int gpt2k_attention_backward(int dtype, void* dqkv, const void* dout, const void* qkv,
                             const void* out, const float* lse, int B, int T, int H, int hd,
                             void* scratch, void* stream) {
  return gpt2k_attention_backward_colsum(dtype, dqkv, dout, qkv, out, lse, B, T, H, hd, scratch,
                                         nullptr, stream);
}

int gpt2k_attention_colsum_ok(int dtype, int hd) { return attention_colsum_ok(dtype, hd) ? 1 : 0; }

int gpt2k_attention_backward_colsum(int dtype, void* dqkv, const void* dout, const void* qkv,
                                    const void* out, const float* lse, int B, int T, int H, int hd,
                                    void* scratch, float* colsum, void* stream) {
  if (colsum && !attention_colsum_ok(dtype, hd))
    return gpt2_internal_fail(GPT2_EINVAL, "column sums not available for this dtype / head size");
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16)
    return gpt2_internal_fail(GPT2_EINVAL, "dtype must be 0 or 1");
  if (!dqkv || !dout || !qkv || !out || !lse || !scratch || B < 1 || T < 1 || H < 1)
    return gpt2_internal_fail(GPT2_EINVAL, "bad argument");
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return gpt2_internal_fail(GPT2_EINVAL, "head size must be 16, 32, 64 or 128");
  return launch_rc(attention_backward(dtype, dqkv, dout, qkv, out, lse, B, T, H, hd, scratch,
                                      (hipStream_t)stream, colsum),
                   "attention_backward");
}

int gpt2k_attention_backward_noalloc(int dtype, void* dqkv, const void* dout, const void* qkv,
                                     const void* out, const float* lse, int B, int T, int H,
                                     int hd, float* colsum, void* stream) {
  if (colsum && !attention_colsum_ok(dtype, hd))
    return gpt2_internal_fail(GPT2_EINVAL, "column sums not available for this dtype / head size");
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16)
    return gpt2_internal_fail(GPT2_EINVAL, "dtype must be 0 or 1");
  if (!dqkv || !dout || !qkv || !out || !lse || B < 1 || T < 1 || H < 1)
    return gpt2_internal_fail(GPT2_EINVAL, "bad argument");
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return gpt2_internal_fail(GPT2_EINVAL, "head size must be 16, 32, 64 or 128");
  if ((int64_t)B * H * T > (int64_t)kNoAllocAttnScratchFloats) {
    char msg[160];
    snprintf(msg, sizeof(msg), "B*H*T = %lld exceeds the fixed scratch of %d rows (4 MiB)",
             (long long)B * H * T, kNoAllocAttnScratchFloats);
    return gpt2_internal_fail(GPT2_EINVAL, msg);
  }
  return launch_rc(attention_backward_noalloc(dtype, dqkv, dout, qkv, out, lse, B, T, H, hd,
                                              (hipStream_t)stream, colsum),
                   "attention_backward_noalloc");
}

}  // extern "C"
