// GEMMs of the GPT-2 step on gfx950.
//
//   C(m, n) = sum_k A(m, k) B(n, k), followed by a fused epilogue
//   (bias, residual add, GELU with both outputs, GELU backward, or fp32
//   accumulation into a gradient).
//
// Linear layers store W as (out, in), so the three products of a layer are
//   forward      y  = x W^T        A = x  (k-major), B = W  (k-major)
//   input grad   dx = dy W         A = dy (k-major), B = W  (n-major)
//   weight grad  dW += dy^T x      A = dy (m-major), B = x  (n-major)
// and one kernel template covers all three with compile-time operand
// orientation.  Operand tiles always land in LDS k-contiguous: a k-major
// operand is copied with 16-byte vectors, an m/n-major one is read as
// 4 k-rows x 8 columns per thread and transposed in registers before the
// LDS store, so the MFMA fragment reads are single 16-byte LDS reads.
//
// bf16: v_mfma_f32_32x32x16_bf16, fp32 accumulation.  Workgroup tile
// 128 x 128 x 64, four waves of 64 x 64 (2 x 2 MFMA tiles), next k-tile
// prefetched into registers while the current one is multiplied.
// fp32 (the fp32 parity mode): plain LDS-tiled FMA kernel.
#include "common.h"
#include "kernels.h"

namespace gk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- epilogue
template <int MODE, class T>
__device__ __forceinline__ void epi_apply(const Epilogue& e, int m, int n, float acc) {
  if constexpr (MODE == EPI_STORE) {
    ((T*)e.out)[(int64_t)m * e.ldo + n] = from_f<T>(acc);
  } else if constexpr (MODE == EPI_BIAS) {
    ((T*)e.out)[(int64_t)m * e.ldo + n] = from_f<T>(acc + e.bias[n]);
  } else if constexpr (MODE == EPI_BIAS_RESID) {
    float r = to_f(((const T*)e.resid)[(int64_t)m * e.ldr + n]);
    ((T*)e.out)[(int64_t)m * e.ldo + n] = from_f<T>(acc + e.bias[n] + r);
  } else if constexpr (MODE == EPI_BIAS_GELU) {
    float h = acc + e.bias[n];
    T hq = from_f<T>(h);
    ((T*)e.out)[(int64_t)m * e.ldo + n] = hq;
    // GELU of the stored (rounded) pre-activation, so that the backward,
    // which differentiates at the stored value, is consistent with it.
    ((T*)e.out2)[(int64_t)m * e.ldo2 + n] = from_f<T>(gelu_f(to_f(hq)));
  } else if constexpr (MODE == EPI_GELU_BWD) {
    float h = to_f(((const T*)e.aux)[(int64_t)m * e.ldx + n]);
    ((T*)e.out)[(int64_t)m * e.ldo + n] = from_f<T>(acc * gelu_grad_f(h));
  } else {  // EPI_ACC_F32
    float* o = (float*)e.out + (int64_t)m * e.ldo + n;
    *o += acc;
  }
}

// ================================================================ fp32 SIMT
template <class T> __device__ __forceinline__ float ld_elem(const T* p, int64_t i) { return to_f(p[i]); }

template <int MODE>
__global__ __launch_bounds__(256) void gemm_simt_kernel(bool akm, bool bkm, int M, int N, int K,
                                                        const float* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ B, int64_t ldb,
                                                        Epilogue e) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int el = threadIdx.x + 256 * i;
      int row, kk;
      if (akm) { row = el / 16; kk = el % 16; } else { kk = el / 64; row = el % 64; }
      int m = m0 + row, k = k0 + kk;
      float va = 0.f;
      if (m < M && k < K) va = akm ? A[(int64_t)m * lda + k] : A[(int64_t)k * lda + m];
      As[kk][row] = va;
      if (bkm) { row = el / 16; kk = el % 16; } else { kk = el / 64; row = el % 64; }
      int n = n0 + row;
      k = k0 + kk;
      float vb = 0.f;
      if (n < N && k < K) vb = bkm ? B[(int64_t)n * ldb + k] : B[(int64_t)k * ldb + n];
      Bs[kk][row] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) epi_apply<MODE, float>(e, m, n, acc[i][j]);
    }
}

// ================================================================ bf16 MFMA
constexpr int MF_BM = 128, MF_BN = 128, MF_BK = 64;
constexpr int MF_LDP = MF_BK + 8;  // LDS row pitch (elements): 144 B, 16-byte aligned rows

// Stage of one operand tile (ROWS x 64) held in registers between the
// global load and the LDS store: 4 x 16 bytes per thread.
struct Stage {
  uint4 r[4];
};

// k-major operand: element (row, k) at P[row * ld + k].  Chunks of 8 k.
template <int ROWS>
__device__ __forceinline__ void load_kmajor(Stage& st, const bf16* __restrict__ P, int64_t ld,
                                            int row0, int rows_total, int k0, int K) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = threadIdx.x + 256 * i;
    int row = c / 8, kc = (c % 8) * 8;
    int gr = row0 + row, gk = k0 + kc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gr < rows_total && gk < K) {
      v = *reinterpret_cast<const uint4*>(P + (int64_t)gr * ld + gk);
      if (gk + 8 > K) {  // ragged k tail: zero the elements at k >= K
        Pack<bf16> pk;
        pk.u = v;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (gk + j >= K) pk.e[j] = (bf16)0.f;
        v = pk.u;
      }
    }
    st.r[i] = v;
  }
}
__device__ __forceinline__ void store_kmajor(const Stage& st, bf16* __restrict__ S) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = threadIdx.x + 256 * i;
    int row = c / 8, kc = (c % 8) * 8;
    *reinterpret_cast<uint4*>(S + row * MF_LDP + kc) = st.r[i];
  }
}

// row-major-in-k operand: element (row, k) at P[k * ld + row].  Thread
// reads k-rows kg*4 .. kg*4+3 at columns mc*8 .. mc*8+7.
__device__ __forceinline__ void load_mmajor(Stage& st, const bf16* __restrict__ P, int64_t ld,
                                            int row0, int rows_total, int k0, int K) {
  int mc = threadIdx.x % 16, kg = threadIdx.x / 16;
  int gr = row0 + mc * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int gk = k0 + kg * 4 + j;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gk < K && gr < rows_total) v = *reinterpret_cast<const uint4*>(P + (int64_t)gk * ld + gr);
    st.r[j] = v;
  }
}
__device__ __forceinline__ void store_mmajor(const Stage& st, bf16* __restrict__ S) {
  int mc = threadIdx.x % 16, kg = threadIdx.x / 16;
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.r[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.r[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&st.r[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&st.r[3]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int sh = (i & 1) * 16;
    uint32_t e0 = (w0[i / 2] >> sh) & 0xffffu;
    uint32_t e1 = (w1[i / 2] >> sh) & 0xffffu;
    uint32_t e2 = (w2[i / 2] >> sh) & 0xffffu;
    uint32_t e3 = (w3[i / 2] >> sh) & 0xffffu;
    uint2 out = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
    *reinterpret_cast<uint2*>(S + (mc * 8 + i) * MF_LDP + kg * 4) = out;
  }
}

template <bool AKM, bool BKM, int MODE>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(int M, int N, int K,
                                                        const bf16* __restrict__ A, int64_t lda,
                                                        const bf16* __restrict__ B, int64_t ldb,
                                                        Epilogue e) {
  __shared__ __attribute__((aligned(16))) bf16 As[MF_BM * MF_LDP];
  __shared__ __attribute__((aligned(16))) bf16 Bs[MF_BN * MF_LDP];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / 2, wn = wave % 2;
  const int m0 = blockIdx.y * MF_BM, n0 = blockIdx.x * MF_BN;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Stage sa, sb;
  auto gload = [&](int k0) {
    if constexpr (AKM) load_kmajor<MF_BM>(sa, A, lda, m0, M, k0, K);
    else load_mmajor(sa, A, lda, m0, M, k0, K);
    if constexpr (BKM) load_kmajor<MF_BN>(sb, B, ldb, n0, N, k0, K);
    else load_mmajor(sb, B, ldb, n0, N, k0, K);
  };
  gload(0);
  for (int k0 = 0; k0 < K; k0 += MF_BK) {
    if constexpr (AKM) store_kmajor(sa, As); else store_mmajor(sa, As);
    if constexpr (BKM) store_kmajor(sb, Bs); else store_mmajor(sb, Bs);
    __syncthreads();
    if (k0 + MF_BK < K) gload(k0 + MF_BK);
#pragma unroll
    for (int s = 0; s < MF_BK / 16; ++s) {
      bf16x8_t a[2], b[2];
      const int kof = s * 16 + (lane / 32) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 32 + lane % 32) * MF_LDP + kof);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 64 + j * 32 + lane % 32) * MF_LDP + kof);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // accumulator layout (32x32 tile): lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int n = n0 + wn * 64 + j * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (m < M && n < N) epi_apply<MODE, bf16>(e, m, n, acc[i][j][r]);
      }
    }
}

// ================================================================ dispatch
template <int MODE>
static hipError_t launch_mode(int dt, bool akm, bool bkm, int M, int N, int K, const void* A,
                              int64_t lda, const void* B, int64_t ldb, const Epilogue& e,
                              hipStream_t s) {
  if (dt == F32) {
    dim3 grid((unsigned)cdiv(N, 64), (unsigned)cdiv(M, 64));
    gemm_simt_kernel<MODE><<<grid, 256, 0, s>>>(akm, bkm, M, N, K, (const float*)A, lda,
                                                 (const float*)B, ldb, e);
    return hipGetLastError();
  }
  dim3 grid((unsigned)cdiv(N, MF_BN), (unsigned)cdiv(M, MF_BM));
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  if (akm && bkm) gemm_mfma_kernel<true, true, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
  else if (akm && !bkm) gemm_mfma_kernel<true, false, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
  else if (!akm && !bkm) gemm_mfma_kernel<false, false, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
  else gemm_mfma_kernel<false, true, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
  return hipGetLastError();
}

hipError_t gemm(int dt, bool a_kmajor, bool b_kmajor, int M, int N, int K, const void* A,
                int64_t lda, const void* B, int64_t ldb, const Epilogue& e, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dt == BF16 && (lda % 8 != 0 || ldb % 8 != 0)) return hipErrorInvalidValue;
  switch (e.mode) {
    case EPI_STORE: return launch_mode<EPI_STORE>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s);
    case EPI_BIAS: return launch_mode<EPI_BIAS>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s);
    case EPI_BIAS_RESID: return launch_mode<EPI_BIAS_RESID>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s);
    case EPI_BIAS_GELU: return launch_mode<EPI_BIAS_GELU>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s);
    case EPI_GELU_BWD: return launch_mode<EPI_GELU_BWD>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s);
    case EPI_ACC_F32: return launch_mode<EPI_ACC_F32>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gk
