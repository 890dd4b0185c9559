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
// and each kernel template covers all three with compile-time operand
// orientation.
//
// bf16 (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   gemm_big_kernel -- the production path (M >= 256, N >= 128): 256 x
//     {256, 192, 128} x 64 tiles, eight waves, operands streamed straight
//     into two LDS stages by buffer loads, m/n-major operands read with
//     transposing LDS reads, persistent or grouped (several products per
//     launch), split-K with fixed-order reductions; epilogues staged through
//     LDS (also the fc bias gradient's column sums and the head's softmax
//     row statistics).  Described in detail further down.
//   gemm_mfma_kernel -- small shapes: 128 x 128 x 64 tiles, four waves, the
//     next k-tile prefetched into registers (m/n-major operands transposed
//     in registers) while the current one is multiplied.
// fp32 (the fp32 parity mode): plain LDS-tiled FMA kernel.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- epilogue
// Returns the value stored to out[m, n] (as rounded to T; 0 for EPI_ACC_F32).
template <int MODE, class T>
__device__ __forceinline__ float epi_apply(const Epilogue& e, int m, int n, float acc) {
  T y;
  if constexpr (MODE == EPI_STORE) {
    y = from_f<T>(acc);
  } else if constexpr (MODE == EPI_BIAS) {
    y = from_f<T>(acc + e.bias[n]);
  } else if constexpr (MODE == EPI_BIAS_RESID) {
    float r = to_f(((const T*)e.resid)[(int64_t)m * e.ldr + n]);
    y = from_f<T>(acc + e.bias[n] + r);
  } else if constexpr (MODE == EPI_BIAS_GELU) {
    y = from_f<T>(acc + e.bias[n]);
    // GELU of the stored (rounded) pre-activation, so that the backward,
    // which differentiates at the stored value, is consistent with it.
    const float h = to_f(y), sg = gelu_sigmoid(h);
    ((T*)e.out2)[(int64_t)m * e.ldo2 + n] = from_f<T>(h * sg);
    if (e.dgelu) y = from_f<T>(gelu_grad_s(h, sg));  // GELU'(h) in place of h
  } else if constexpr (MODE == EPI_DLOGITS) {
    const int c = e.col0 + n;
    const int yy = min(max(e.targets[m], 0), e.vocab - 1);
    float p = c < e.vocab ? fast_exp(to_f(from_f<T>(acc)) - e.lse[m]) : 0.f;
    if (c == yy) p -= 1.f;
    y = from_f<T>(p * e.scale);
  } else if constexpr (MODE == EPI_GELU_BWD) {
    const float a = to_f(((const T*)e.aux)[(int64_t)m * e.ldx + n]);
    if (e.dgelu) {  // aux: GELU'(h) as the forward stored it
      y = from_f<T>(acc * a);
    } else {  // aux: h; GELU'(h) rounded as the forward would store it
      y = from_f<T>(acc * to_f(from_f<T>(gelu_grad_f(a))));
      // out2 (optional): GELU(h) again, as the forward's bias + GELU epilogue stored it
      if (e.out2) ((T*)e.out2)[(int64_t)m * e.ldo2 + n] = from_f<T>(gelu_f(a));
    }
  } else {  // EPI_ACC_F32
    float* of = (float*)e.out + (int64_t)m * e.ldo + n;
    *of += acc;
    return 0.f;
  }
  ((T*)e.out)[(int64_t)m * e.ldo + n] = y;
  return to_f(y);
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

// ================================================================ bf16 MFMA, large tiles
// Workgroup tile BM x BN (BM = 256, BN = 256 / 192 / 128) x 64, eight waves
// of (BM/4) x (BN/2).  Two LDS stages: while the waves multiply stage s,
// the next k-tile streams into stage s^1 by buffer loads that write LDS
// directly (BigOperand below), with one barrier per k-tile.  k-major
// operands sit in LDS as 128-byte rows with XOR-swizzled 16-byte chunks;
// m-major ones as they are in memory, read with ds_read_b64_tr_b16.
// Persistent workgroups (one per CU) walk the tiles XCD-major in groups of 8
// tile-rows, so that concurrently running tiles share operands in L2;
// grouped launches give each workgroup one tile of one of several products.
// gridDim.y > 1 (or a grouped split) divides K; with EPI_PARTIAL each split
// writes its fp32 tile to out + split * M * N and the reduce kernels add
// them in order.
// Epilogue on 8 consecutive columns n .. n+7 of row m (16-byte accesses when
// the row pitches allow it, element-wise at the ragged right edge).
// res[j]: the value stored to out[m, n + j] as rounded (bf16 outputs; 0
// past N).
// AUXV: the 16-byte path takes the GELU backward's pre-activations, or the
// residual, from auxv (loaded by the caller) instead of loading them.
template <int MODE, bool AUXV = false>
__device__ __forceinline__ void epi_apply8(const Epilogue& e, int m, int n, int N, const float* v,
                                           int split, int M, float* res,
                                           const float* bias8 = nullptr,
                                           Pack<bf16> auxv = Pack<bf16>{}) {
  if constexpr (MODE == EPI_PARTIAL) {
    float* o = (float*)e.out + (int64_t)split * M * N + (int64_t)m * N + n;
    if (n + 8 <= N && (N & 3) == 0) {
      *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      for (int j = 0; j < 8 && n + j < N; ++j) o[j] = v[j];
    }
    return;
  } else {
    const bool vec = n + 8 <= N && (e.ldo & 7) == 0 && (e.ldr & 7) == 0 && (e.ldo2 & 7) == 0 &&
                     (e.ldx & 7) == 0;
    if (!vec) {
      for (int j = 0; j < 8; ++j) res[j] = n + j < N ? epi_apply<MODE, bf16>(e, m, n + j, v[j]) : 0.f;
      return;
    }
    if constexpr (MODE == EPI_ACC_F32) {
      float* o = (float*)e.out + (int64_t)m * e.ldo + n;
      float4 a = *reinterpret_cast<float4*>(o), b = *reinterpret_cast<float4*>(o + 4);
      a.x += v[0]; a.y += v[1]; a.z += v[2]; a.w += v[3];
      b.x += v[4]; b.y += v[5]; b.z += v[6]; b.w += v[7];
      *reinterpret_cast<float4*>(o) = a;
      *reinterpret_cast<float4*>(o + 4) = b;
    } else {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = v[j];
      if constexpr (MODE == EPI_BIAS || MODE == EPI_BIAS_RESID || MODE == EPI_BIAS_GELU) {
        if (bias8) {  // bias[n .. n+7], loaded by the caller
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] += bias8[j];
        } else {
          float4 b0 = *reinterpret_cast<const float4*>(e.bias + n);
          float4 b1 = *reinterpret_cast<const float4*>(e.bias + n + 4);
          x[0] += b0.x; x[1] += b0.y; x[2] += b0.z; x[3] += b0.w;
          x[4] += b1.x; x[5] += b1.y; x[6] += b1.z; x[7] += b1.w;
        }
      }
      if constexpr (MODE == EPI_BIAS_RESID) {
        Pack<bf16> r;
        if constexpr (AUXV) r = auxv;
        else r = load_pack((const bf16*)e.resid + (int64_t)m * e.ldr + n);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] += to_f(r.e[j]);
      }
      if constexpr (MODE == EPI_DLOGITS) {
        // the cross-entropy's gradient of the logits z = bf16(acc)
        const float l = e.lse[m];
        const int yy = min(max(e.targets[m], 0), e.vocab - 1) - e.col0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float p = e.col0 + n + j < e.vocab ? fast_exp((float)(bf16)x[j] - l) : 0.f;
          if (n + j == yy) p -= 1.f;
          x[j] = p * e.scale;
        }
      }
      if constexpr (MODE == EPI_GELU_BWD) {
        Pack<bf16> h;
        if constexpr (AUXV) h = auxv;
        else h = load_pack((const bf16*)e.aux + (int64_t)m * e.ldx + n);
        if (e.dgelu) {  // h holds GELU'(pre-activation), as the forward stored it
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= to_f(h.e[j]);
        } else {  // GELU' of h, rounded as the forward would store it
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= (float)(bf16)gelu_grad_f(to_f(h.e[j]));
          if (e.out2) {  // GELU(h) again, as the forward's bias + GELU epilogue stored it
            Pack<bf16> g2;
#pragma unroll
            for (int j = 0; j < 8; ++j) g2.e[j] = (bf16)gelu_f(to_f(h.e[j]));
            store_pack((bf16*)e.out2 + (int64_t)m * e.ldo2 + n, g2);
          }
        }
      }
      Pack<bf16> o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o.e[j] = (bf16)x[j];
#pragma unroll
      for (int j = 0; j < 8; ++j) res[j] = to_f(o.e[j]);
      if constexpr (MODE == EPI_BIAS_GELU) {
        // GELU of the stored pre-activation, and with dgelu its derivative
        // (stored in its place) from the same sigmoid
        Pack<bf16> g2, so = o;
        if (e.dgelu) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float h = to_f(o.e[j]), sg = gelu_sigmoid(h);
            g2.e[j] = (bf16)(h * sg);
            so.e[j] = (bf16)gelu_grad_s(h, sg);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) g2.e[j] = (bf16)gelu_f(to_f(o.e[j]));
        }
        store_pack((bf16*)e.out + (int64_t)m * e.ldo + n, so);
        store_pack((bf16*)e.out2 + (int64_t)m * e.ldo2 + n, g2);
      } else {
        store_pack((bf16*)e.out + (int64_t)m * e.ldo + n, o);
      }
    }
  }
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int chunk) { return r * 64 + ((chunk ^ swz(r)) << 3); }

constexpr int BIG_THREADS = 512;  // 8 waves: 4 along M x 2 along N

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// Buffer-resource word 3 for raw (unswizzled, stride 0) buffers on CDNA:
// 32-bit data format, range checking against num_records.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// A per-lane buffer offset that is always out of range: the load returns
// zeros (and writes them to LDS) without touching memory.
constexpr uint32_t kOOB = 0x80000000u;

// One operand tile (R rows of the output dimension x 64 k) in LDS, filled
// by buffer loads straight into LDS: one wave instruction writes 64
// consecutive 16-byte slots, lane i at slot i, and each lane fetches the
// global vector that belongs in its slot.  No registers hold the tile in
// flight.  Each lane's byte offset inside the operand is fixed for the whole
// k loop; the k step goes into the scalar offset, and rows past the matrix
// edge carry an out-of-range offset, so the hardware range check supplies
// their zeros.
//  k-major source: [row][64 k], 128-byte rows, 16-byte chunks XOR-swizzled
//    by row (conflict-free 16-byte fragment reads).
//  m-major source: [64 k][R rows] as in memory, the chunks of each k-row
//    permuted so that the four k-rows of a transposing read land on four
//    different quarters of the 64 LDS banks; fragments via
//    ds_read_b64_tr_b16.  R >= 128.  A read takes 64 bytes (four 16-byte
//    chunks) of each of four k-rows; with R = 128 or 256 the rows are
//    pitched at a multiple of 256 bytes and rotating k-row k by 4*(k%4)
//    chunks spreads them; with R = 192 (384-byte rows, an odd multiple of
//    128 bytes) consecutive rows already differ by half the banks, and
//    swapping the 4-chunk groups of the k-rows with bit 1 set (chunk ^ 4)
//    completes the spread where a rotation modulo 24 chunks would wrap onto
//    used banks.
template <int R, bool KMAJOR, int NW>
struct BigOperand {
  static constexpr int ELEMS = R * 64;
  static constexpr int CPR = R / 8;     // 16-byte chunks per k-row (m-major)
  static constexpr int NI = R * 8 / (64 * NW);  // load instructions per wave per tile

  // physical chunk of logical chunk lc in k-row krow, and the inverse
  __device__ __forceinline__ static int mphys(int krow, int lc) {
    if constexpr (CPR == 24) return lc ^ (krow & 2 ? 4 : 0);
    else return (lc + CPR - 4 * (krow & 3)) % CPR;
  }
  __device__ __forceinline__ static int mlog(int krow, int p) {
    if constexpr (CPR == 24) return p ^ (krow & 2 ? 4 : 0);
    else return (p + 4 * (krow & 3)) % CPR;
  }

  struct Src {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff[NI];  // byte offset of each load's vector for k0 = 0, or kOOB
  };

  // k offset inside a tile of the vector that load q of this lane fetches
  __device__ __forceinline__ static int kofs(int q, int wave, int lane) {
    const int slot = (wave + NW * q) * 64 + lane;
    if constexpr (KMAJOR) return 8 * ((slot & 7) ^ swz(slot >> 3));
    else return slot / CPR;
  }

  // P: the operand, ld: its row pitch in elements, row0: first output row of
  // this tile, rows_total: rows of the output dimension, K: the k extent.
  // The host guarantees that the operand spans fewer than 2^31 bytes.
  __device__ __forceinline__ static void init(Src& st, const bf16* __restrict__ P, int64_t ld,
                                              int row0, int rows_total, int K, int wave, int lane) {
    const bf16* base = KMAJOR ? P + (int64_t)row0 * ld : P + row0;
    const int64_t span = KMAJOR ? ((int64_t)(rows_total - 1 - row0) * ld + K) * 2
                                : ((int64_t)(K - 1) * ld + (rows_total - row0)) * 2;
    st.rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)span, (int)kRsrcWord3);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int slot = (wave + NW * q) * 64 + lane;
      if constexpr (KMAJOR) {
        const int row = slot >> 3;
        const int ko = 8 * ((slot & 7) ^ swz(row));
        st.voff[q] = row0 + row < rows_total ? (uint32_t)(((int64_t)row * ld + ko) * 2) : kOOB;
      } else {
        const int krow = slot / CPR;
        const int c = 8 * mlog(krow, slot % CPR);
        st.voff[q] = row0 + c < rows_total ? (uint32_t)(((int64_t)krow * ld + c) * 2) : kOOB;
      }
    }
  }

  // Issue the loads of the tile starting at k0 into LDS tile S.  TAIL: this
  // tile extends past kend, whose columns (k-major) or rows (m-major) must
  // read as zeros.
  template <bool TAIL>
  __device__ __forceinline__ static void load(bf16* __restrict__ S, const Src& st, int64_t ld,
                                              int k0, int kend, int wave, int lane) {
    const uint32_t soff = (uint32_t)(KMAJOR ? (int64_t)k0 * 2 : (int64_t)k0 * ld * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const uint32_t v = TAIL && k0 + kofs(q, wave, lane) >= kend ? kOOB : st.voff[q];
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins exist only for the GPU target
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          st.rs, (__attribute__((address_space(3))) void*)(S + (wave + NW * q) * 512), 16, v, soff, 0, 0);
#endif
    }
  }

  // MFMA operand: lane holds row `row0 + lane%32`, k = ks*16 + 8*h2 .. +8.
  __device__ __forceinline__ static bf16x8_t frag(const bf16* S, int row0, int ks, int lane) {
    const int h2 = lane >> 5;
    if constexpr (KMAJOR) {
      return *reinterpret_cast<const bf16x8_t*>(S + lds_off(row0 + (lane & 31), ks * 2 + h2));
    } else {
      const int j = lane & 15;
      const int col = row0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const int kr = ks * 16 + 8 * h2 + (j >> 2);
      const bf16* p0 = S + kr * R + (mphys(kr, col >> 3) << 3) + (col & 7);
      const bf16* p1 = S + (kr + 4) * R + (mphys(kr + 4, col >> 3) << 3) + (col & 7);
      union {
        v4i16 s[2];
        bf16x8_t v;
      } r;
      r.s[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
      r.s[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
      return r.v;
    }
  }
  // LDS read instructions per fragment
  static constexpr int READS = KMAJOR ? 1 : 2;
};

// Scheduling hint for one k-step of NM MFMAs while the NR LDS reads of the
// next k-step are issued: the reads are spread evenly between the MFMAs.
template <int NM, int NR, int I = 0>
__device__ __forceinline__ void interleave_mfma_reads() {
  if constexpr (I < NM) {
    constexpr int r = (I + 1) * NR / NM - I * NR / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // r LDS reads
    interleave_mfma_reads<NM, NR, I + 1>();
  }
}

// Output tile of logical index pid: groups of 8 tile-rows, column-major
// inside a group, so that tiles with neighbouring indices share operand
// panels.
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  // grouped order: 8 tile-rows at a time, column-major inside a group
  const int G = 8;
  int in_group = G * tiles_n;
  int group = pid / in_group;
  int first_m = group * G;
  int gsize = min(tiles_m - first_m, G);
  int r = pid % in_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Waves per workgroup: 8 (4 x 2, wave tiles of 64 x BN/2).  (Four waves of
// 128 x 128 were measured no faster at 256 x 256.)
template <int BN> struct BigWaves { static constexpr int NW = 8; };

template <int BM, int BN, bool AKM, bool BKM>
struct BigSmem {
  static constexpr int NW = BigWaves<BN>::NW;
  using OA = BigOperand<BM, AKM, NW>;
  using OB = BigOperand<BN, BKM, NW>;
  static constexpr int STAGE = OA::ELEMS + OB::ELEMS;
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One product of a launch.  Up to kMaxGroup products with the same K and
// operand orientations share a launch (the weight gradients of one or two
// layers run as one launch this way).
struct BigProblem {
  int M, N, tiles_m, tiles_n;
  const bf16* A;
  int64_t lda;
  const bf16* B;
  int64_t ldb;
  Epilogue e;
};
constexpr int kMaxGroup = 8;
struct BigBatch {
  BigProblem p[kMaxGroup];
  // Grouped launches (grouped != 0): a 1-D grid of work items, product i owning
  // items item0[i] .. item0[i+1]-1 = its tiles x `splits` K ranges, one
  // tile per workgroup.  Items are numbered product-major, then split,
  // then tile (in tile_of order), and dealt to the XCDs in contiguous
  // ranges, so that the workgroups of an XCD cover compact blocks of tiles
  // of one product and share its operand panels in their L2.
  int grouped, n, splits;
  int item0[kMaxGroup + 1];
};

template <int BM, int BN, bool AKM, bool BKM, int MODE>
__global__ __launch_bounds__(BigWaves<BN>::NW * 64) void gemm_big_kernel(const BigBatch batch,
                                                                         int K, int kps) {
  int prob = 0, split = blockIdx.y, first = xcd_remap(blockIdx.x, gridDim.x), step = gridDim.x;
  if (batch.grouped) {
    const int item = first;
    while (prob + 1 < batch.n && item >= batch.item0[prob + 1]) ++prob;
    const int r = item - batch.item0[prob];
    const int nt = batch.p[prob].tiles_m * batch.p[prob].tiles_n;
    split = r / nt;
    first = r % nt;
    step = nt;  // this tile only
  }
  const BigProblem& P = batch.p[prob];
  const int M = P.M, N = P.N, tiles_m = P.tiles_m, tiles_n = P.tiles_n;
  const bf16* __restrict__ A = P.A;
  const bf16* __restrict__ B = P.B;
  const int64_t lda = P.lda, ldb = P.ldb;
  const Epilogue& e = P.e;
  using SM = BigSmem<BM, BN, AKM, BKM>;
  using OA = typename SM::OA;
  using OB = typename SM::OB;
  // Two stages as two separate arrays, so that the compiler can see that
  // the loads streaming into one never alias the fragment reads of the other.
  __shared__ __attribute__((aligned(16))) bf16 smem0[SM::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 smem1[SM::STAGE];
  constexpr int NW = SM::NW;
  constexpr int WM = BM / (NW / 2), WN = BN / 2, TI = WM / 32, TJ = WN / 32;
  const int lane = threadIdx.x % 64, h2 = lane / 32, l32 = lane % 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform: LDS bases in SGPRs
  const int wm = wave / 2, wn = wave % 2;
  // Persistent: workgroup w takes logical tiles w, w + G, w + 2G, ... (G
  // workgroups, at most one per CU), with w numbered XCD-major so that the
  // tiles an XCD works on at the same time are neighbours and share its L2.
  const int ntiles = tiles_m * tiles_n;
  for (int tile = first; tile < ntiles; tile += step) {
  int tm, tn;
  tile_of(tile, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * kps;
  const int kend = min(K, kbeg + kps);
  const int nk = kend > kbeg ? (int)cdiv(kend - kbeg, 64) : 0;

  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  typename OA::Src srcA;
  typename OB::Src srcB;
  OA::init(srcA, A, lda, m0, M, K, wave, lane);
  OB::init(srcB, B, ldb, n0, N, K, wave, lane);
  auto issueA = [&](bf16* st, int k0) {
    if (k0 + 64 > kend) OA::template load<true>(st, srcA, lda, k0, kend, wave, lane);
    else OA::template load<false>(st, srcA, lda, k0, kend, wave, lane);
  };
  auto issueB = [&](bf16* st, int k0) {
    if (k0 + 64 > kend) OB::template load<true>(st + OA::ELEMS, srcB, ldb, k0, kend, wave, lane);
    else OB::template load<false>(st + OA::ELEMS, srcB, ldb, k0, kend, wave, lane);
  };
  auto issue = [&](bf16* st, int k0) {
    issueA(st, k0);
    issueB(st, k0);
  };
  // Fragments are double-buffered in registers: the LDS reads of k-step s+1
  // are issued between the MFMAs of k-step s.
  constexpr int NR = TI * OA::READS + TJ * OB::READS;  // LDS reads per k-step
  auto frags = [&](const bf16* st, int s, bf16x8_t (&fa)[TI], bf16x8_t (&fb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[i] = OA::frag(st, wm * WM + i * 32, s, lane);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[j] = OB::frag(st + OA::ELEMS, wn * WN + j * 32, s, lane);
  };
  // The B fragment goes in as the MFMA's first operand, so the accumulator
  // holds the tile transposed: lane l has row l%32 of block i and, in
  // registers 4q..4q+3, the four consecutive columns 8q + 4(l/32) + 0..3 of
  // block j.
  auto mma = [&](const bf16x8_t (&fa)[TI], const bf16x8_t (&fb)[TJ]) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int i = 0; i < TI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  // iteration kt multiplies the tile in `cur` while the next tile streams
  // into `nxt`; one barrier per k-tile.  Where the next tile's loads are
  // issued: a wave whose loads back up in the address path stalls there
  // before its MFMAs, so the two waves of a SIMD should not both issue
  // theirs at one moment when the loads are slow to drain (measured on the
  // three operand orientations of the step's products):
  //   k-major x k-major: every wave at the top of the iteration;
  //   k-major x m-major: A's loads at the top, B's after k-step 0
  //     (the head's 256-wide d lnf product 4 % faster, 192-wide products
  //     unchanged);
  //   m-major x m-major: waves 0 .. NW/2-1 (one per SIMD) at the top, the
  //     others after k-step 2 (weight gradients 13-15 % faster; after
  //     k-step 1: 11-12 %; every wave at k-step 0 or A and B apart: slower).
  constexpr int kPlace = AKM ? (BKM ? 0 : 1) : 2;
  const bool early = wave < NW / 2;
  auto iter = [&](int kt, bf16* cur, bf16* nxt) {
    const bool more = kt + 1 < nk;
    const int k1 = kbeg + (kt + 1) * 64;
    if constexpr (kPlace == 0) {
      if (more) issue(nxt, k1);
    } else if constexpr (kPlace == 1) {
      if (more) issueA(nxt, k1);
    } else {
      if (more && early) issue(nxt, k1);
    }
    // keep the loads in place: the scheduler would otherwise sink them
    // below the math, next to the wait that ends the iteration
    __builtin_amdgcn_sched_barrier(0);
    // Raised issue priority from here to the last MFMA of the k-tile, so
    // that a SIMD's wave still multiplying is served before the other wave
    // reaches the wait and barrier that end its iteration (the two layers'
    // weight gradients 5 % faster, the step 0.9 %; results unchanged).
    __builtin_amdgcn_s_setprio(1);
    bf16x8_t fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];
    frags(cur, 0, fa0, fb0);
    frags(cur, 1, fa1, fb1);
    mma(fa0, fb0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NR, 0);  // all reads of k-steps 0 and 1
    __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ, 0);  // then the MFMAs of k-step 0
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPlace == 1) {
      if (more) issueB(nxt, k1);
      __builtin_amdgcn_sched_barrier(0);
    }
    frags(cur, 2, fa0, fb0);
    mma(fa1, fb1);
    interleave_mfma_reads<TI * TJ, NR>();
    __builtin_amdgcn_sched_barrier(0);
    frags(cur, 3, fa1, fb1);
    mma(fa0, fb0);
    interleave_mfma_reads<TI * TJ, NR>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPlace == 2) {
      if (more && !early) issue(nxt, k1);
      __builtin_amdgcn_sched_barrier(0);
    }
    mma(fa1, fb1);
    __builtin_amdgcn_s_setprio(0);
    wait_vmem();
    __syncthreads();
  };

  if (nk > 0) issue(smem0, kbeg);
  wait_vmem();
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    iter(kt, smem0, smem1);
    iter(kt + 1, smem1, smem0);
  }
  if (kt < nk) iter(kt, smem0, smem1);

  // Epilogue through LDS, per wave: the wave's 32 rows of block i and JB
  // column blocks at a time go to its own LDS slab (16-byte writes of four
  // consecutive columns), then come back as 8 consecutive columns per lane
  // for 16-byte global accesses.  One workgroup barrier first (the slabs
  // reuse the operand stages); after it each wave touches only its own slab,
  // and a wave's LDS accesses complete in issue order.
  constexpr int JB = (TJ % 3 == 0) ? 3 : 2;  // column blocks per round
  constexpr int SP = JB * 32 + 4;            // slab row pitch (floats)
  static_assert(TJ % JB == 0, "column blocks must divide evenly");
  // waves 0 .. NW/2-1 stage in the first operand buffer, the others in the second
  static_assert((NW / 2) * 32 * SP * 4 <= SM::STAGE * 2, "epilogue staging exceeds LDS");
  float* slab = reinterpret_cast<float*>(wave < NW / 2 ? smem0 : smem1) + (wave % (NW / 2)) * 32 * SP;
  // Column sums of the output (Epilogue::colsum): the stored values go back
  // into the slab, and lane c < 16 JB sums slab columns 2c, 2c+1 over the
  // 32 rows, then over the wave's TI row blocks -- the wave's WM = 64 rows,
  // one colsum block.
  // Softmax row statistics (EPI_ROWSTATS): lane l of a 256-column tile
  // handles rows l/8 + 8t (t < 4) of the slab and columns 8 (l%8) .. +8; it
  // keeps one running (max, sum) per row over the wave's two column rounds,
  // and the eight lanes of a row then combine theirs by shuffles, into one
  // entry per row and 128 columns.
  constexpr bool kStats = MODE == EPI_ROWSTATS;
  static_assert(!kStats || (BN == 256 && JB == 2), "row statistics need 256-column tiles");
  float rmax[kStats ? 4 : 1], rsum[kStats ? 4 : 1];
  // (m1, s1) <- the pair for the union of both sets; only the smaller
  // maximum's sum needs rescaling (the other factor is exp(0) = 1)
  auto combine = [](float& m1, float& s1, float m2, float s2) {
    const bool first = m1 >= m2;
    const float big = first ? m1 : m2, small = first ? m2 : m1;
    if (big == -INFINITY) return;  // both empty
    const float sbig = first ? s1 : s2, ssmall = first ? s2 : s1;
    s1 = sbig + ssmall * fast_exp(small - big);
    m1 = big;
  };
  // Bias of the columns this lane stores: lane c handles the 8-column
  // chunks (c + 64 t) % CPRW of each slab row, which cycle through only
  // NBD = CPRW / gcd(64, CPRW) values, so the lane loads those once per tile
  // instead of once per stored chunk (the loads would share the address path
  // with the stores).  Done for the 192-wide tiles (three chunks per lane,
  // one column round); the 256-wide ones would need one register more than
  // they have.
  constexpr int CPRW = JB * 4;        // 8-column chunks per slab row
  constexpr int CHUNKS = 32 * CPRW;   // chunks in the slab
  static_assert(CHUNKS % 64 == 0, "whole chunks per lane");
  constexpr int NBD = CPRW / gcd_c(64, CPRW);
  static_assert(JB != 3 || NBD == 3, "12 chunks per row: three per lane");
  static_assert(JB != 2 || NBD == 1, "8 chunks per row: one per lane");
  constexpr bool kBiasPre =
      (MODE == EPI_BIAS || MODE == EPI_BIAS_RESID || MODE == EPI_BIAS_GELU) && JB == 3;
  float bpre[kBiasPre ? TJ / JB : 1][kBiasPre ? NBD : 1][8];
  if constexpr (kBiasPre) {
#pragma unroll
    for (int jr = 0; jr < TJ / JB; ++jr)
#pragma unroll
      for (int d = 0; d < NBD; ++d) {
        const int n = n0 + wn * WN + jr * JB * 32 + ((lane + 64 * d) % CPRW) * 8;
        if (n + 8 <= N) {
          const float4 b0 = *reinterpret_cast<const float4*>(e.bias + n);
          const float4 b1 = *reinterpret_cast<const float4*>(e.bias + n + 4);
          bpre[jr][d][0] = b0.x; bpre[jr][d][1] = b0.y; bpre[jr][d][2] = b0.z; bpre[jr][d][3] = b0.w;
          bpre[jr][d][4] = b1.x; bpre[jr][d][5] = b1.y; bpre[jr][d][6] = b1.z; bpre[jr][d][7] = b1.w;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) bpre[jr][d][j] = 0.f;  // unused: the ragged edge reads e.bias
        }
      }
  }
  constexpr bool kColsum = MODE == EPI_GELU_BWD;
  static_assert(!kColsum || WM == 64, "colsum blocks are the waves' 64 rows");
  const bool colsum = kColsum && e.colsum != nullptr;
  float2 csum[TJ / JB];
#pragma unroll
  for (int jr = 0; jr < TJ / JB; ++jr) csum[jr] = make_float2(0.f, 0.f);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    if constexpr (kStats) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        rmax[t] = -INFINITY;
        rsum[t] = 0.f;
      }
    }
#pragma unroll
    for (int jr = 0; jr < TJ / JB; ++jr) {
#pragma unroll
      for (int jj = 0; jj < JB; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16_t& c = acc[i][jr * JB + jj];
          *reinterpret_cast<float4*>(slab + l32 * SP + jj * 32 + 8 * q + 4 * h2) =
              make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
        }
      __builtin_amdgcn_wave_barrier();
      // GELU backward and bias + residual: the round's pre-activations (or
      // residual rows) are all requested before its first store, so that
      // waiting for one of them does not also wait for the stores of the
      // chunks before it (one in-order counter covers loads and stores;
      // loaded chunk by chunk, each load waited for every store before it:
      // step 0.6 % and 0.3 % slower)
      constexpr bool kAuxBatch = MODE == EPI_GELU_BWD || MODE == EPI_BIAS_RESID;
      const bf16* const asrc = (const bf16*)(MODE == EPI_GELU_BWD ? e.aux : e.resid);
      const int64_t ald = MODE == EPI_GELU_BWD ? e.ldx : e.ldr;
      Pack<bf16> hb[kAuxBatch ? CHUNKS / 64 : 1];
      if constexpr (kAuxBatch) {
        // buffer loads without branches: a chunk that is not stored from
        // these registers carries an out-of-range offset and reads zeros
        const bool vec = (e.ldo & 7) == 0 && (e.ldr & 7) == 0 && (e.ldo2 & 7) == 0 && (e.ldx & 7) == 0;
        const int r0 = m0 + wm * WM + i * 32;  // the round's first row
        const int rows = min(M - r0, 32);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(asrc + (int64_t)r0 * ald), (short)0, rows > 0 ? (int)((int64_t)rows * ald * 2) : 0,
            (int)kRsrcWord3);
#pragma unroll
        for (int t = 0; t < CHUNKS / 64; ++t) {
          const int c = lane + 64 * t;
          const int r = c / CPRW;
          const int n = n0 + wn * WN + jr * JB * 32 + (c % CPRW) * 8;
          // exactly the chunks epi_apply8 stores on its 16-byte path
          const bool ok = vec && r < rows && n + 8 <= N;
          const uint32_t off = ok ? (uint32_t)(((int64_t)r * ald + n) * 2) : kOOB;
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins exist only for the GPU target
          const v4u32 w = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
          hb[t].u = make_uint4(w.x, w.y, w.z, w.w);
#else
          (void)rs;
          (void)off;
          hb[t].u = make_uint4(0, 0, 0, 0);
#endif
        }
      }
#pragma unroll
      for (int t = 0; t < CHUNKS / 64; ++t) {
        const int c = lane + 64 * t;
        const int row = c / CPRW, col = (c % CPRW) * 8;
        const float4 a = *reinterpret_cast<const float4*>(slab + row * SP + col);
        const float4 b = *reinterpret_cast<const float4*>(slab + row * SP + col + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const int m = m0 + wm * WM + i * 32 + row, n = n0 + wn * WN + jr * JB * 32 + col;
        if constexpr (kStats) {
          // e.ldx = V (valid columns), e.aux = targets, e.out2 = tgt
          const int V = (int)e.ldx;
          float z[8], cm = -INFINITY, cs = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            z[j] = (float)(bf16)v[j];
            if (m < M && n + j < V) cm = fmaxf(cm, z[j]);
          }
          if (cm != -INFINITY) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (m < M && n + j < V) cs += fast_exp(z[j] - cm);
          }
          if (m < M) {
            const int y = min(max(((const int32_t*)e.aux)[m], 0), V - 1);
            if (y >= n && y < n + 8) ((float*)e.out2)[m] = z[y - n];
          }
          combine(rmax[t], rsum[t], cm, cs);  // this lane's columns; lanes combine below
          continue;
        }
        float res[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (m < M && n < N) {
          if constexpr (kBiasPre && kAuxBatch) {
            epi_apply8<MODE, true>(e, m, n, N, v, split, M, res, bpre[jr][t % NBD], hb[t]);
          } else if constexpr (kBiasPre) {
            epi_apply8<MODE>(e, m, n, N, v, split, M, res, bpre[jr][t % NBD]);
          } else if constexpr (kAuxBatch) {
            epi_apply8<MODE, true>(e, m, n, N, v, split, M, res, nullptr, hb[t]);
          } else {
            epi_apply8<MODE>(e, m, n, N, v, split, M, res);
          }
        }
        if (colsum) {  // this lane alone read these slab entries
          *reinterpret_cast<float4*>(slab + row * SP + col) = make_float4(res[0], res[1], res[2], res[3]);
          *reinterpret_cast<float4*>(slab + row * SP + col + 4) = make_float4(res[4], res[5], res[6], res[7]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (colsum && lane < 16 * JB) {
        float2 t = make_float2(0.f, 0.f);
#pragma unroll 8
        for (int r = 0; r < 32; ++r) {
          const float2 x = *reinterpret_cast<const float2*>(slab + r * SP + 2 * lane);
          t.x += x.x;
          t.y += x.y;
        }
        csum[jr].x += t.x;
        csum[jr].y += t.y;
      }
      __builtin_amdgcn_wave_barrier();
    }
    if constexpr (kStats) {
      // the eight lanes of each row combine their running statistics
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int o = 1; o < 8; o <<= 1)
          combine(rmax[t], rsum[t], __shfl_xor(rmax[t], o, 64), __shfl_xor(rsum[t], o, 64));
      if (lane % 8 == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = m0 + wm * WM + i * 32 + lane / 8 + 8 * t;
          if (m < M)
            ((float2*)e.out)[(int64_t)m * e.ldo + n0 / 128 + wn] = make_float2(rmax[t], rsum[t]);
        }
      }
    }
  }
  if (colsum && lane < 16 * JB) {
    const int blk = (m0 + wm * WM) / 64;
    if (m0 + wm * WM < M) {
#pragma unroll
      for (int jr = 0; jr < TJ / JB; ++jr) {
        const int n = n0 + wn * WN + jr * JB * 32 + 2 * lane;
        float* cp = e.colsum + (int64_t)blk * e.ldcs + n;
        if (n + 1 < N) {
          *reinterpret_cast<float2*>(cp) = csum[jr];
        } else if (n < N) {
          cp[0] = csum[jr].x;
        }
      }
    }
  }
  __syncthreads();  // the next tile's loads overwrite the staging slabs
  }
}

// dst[m, n] (fp32, row pitch ldo) += sum over s of part[s][m][n], in order.
__global__ void splitk_reduce_kernel(float* __restrict__ dst, int64_t ldo,
                                     const float* __restrict__ part, int S, int M, int N) {
  int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  int64_t total = (int64_t)M * N;
  if (idx >= total) return;
  int m = (int)(idx / N), n = (int)(idx % N);
  float4 acc = *reinterpret_cast<const float4*>(part + idx);
  for (int s = 1; s < S; ++s) {
    float4 p = *reinterpret_cast<const float4*>(part + (int64_t)s * total + idx);
    acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
  }
  float4* d = reinterpret_cast<float4*>(dst + (int64_t)m * ldo + n);
  float4 o = *d;
  o.x += acc.x; o.y += acc.y; o.z += acc.z; o.w += acc.w;
  *d = o;
}

// The same for up to kMaxGroup products in one launch (the grouped weight
// gradients): product i owns the float4 indices q0[i] .. q0[i+1]-1.
struct ReduceBatch {
  int n, S;
  float* dst[kMaxGroup];
  int64_t ldo[kMaxGroup];
  const float* part[kMaxGroup];
  int M[kMaxGroup], N[kMaxGroup];
  int64_t q0[kMaxGroup + 1];
};

__global__ void splitk_reduce_group_kernel(const ReduceBatch rb) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= rb.q0[rb.n]) return;
  int i = 0;
  while (i + 1 < rb.n && q >= rb.q0[i + 1]) ++i;
  const int M = rb.M[i], N = rb.N[i];
  const int64_t total = (int64_t)M * N, idx = (q - rb.q0[i]) * 4;
  const float* part = rb.part[i];
  const int m = (int)(idx / N), n = (int)(idx % N);
  float4 acc = *reinterpret_cast<const float4*>(part + idx);
  for (int s = 1; s < rb.S; ++s) {
    float4 p = *reinterpret_cast<const float4*>(part + (int64_t)s * total + idx);
    acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
  }
  float4* d = reinterpret_cast<float4*>(rb.dst[i] + (int64_t)m * rb.ldo[i] + n);
  float4 o = *d;
  o.x += acc.x; o.y += acc.y; o.z += acc.z; o.w += acc.w;
  *d = o;
}

// ================================================================ dispatch
namespace {

constexpr int kCUs = 256;

struct Plan {
  int kind;  // 0: 128x128 kernel, 1: 256x256, 2: 256x128, 3: 256x192
  int splits;
};

// 256 x 256 tiles need all 512 registers for the accumulators and operand
// staging; the GELU epilogues would spill there, so they use 256 x 128.
constexpr bool big_square_ok(int mode) { return mode != EPI_BIAS_GELU && mode != EPI_GELU_BWD; }

Plan plan_gemm(int M, int N, int K, int mode) {
  if (M < 256 || N < 128 || K % 8 != 0) return {0, 1};
  // kind: 1 = 256 x 256, 2 = 256 x 128, 3 = 256 x 192
  const int cand[3][3] = {{1, 256, 256}, {3, 256, 192}, {2, 256, 128}};
  const double eff[4] = {0.0, 1.0, 0.8, 0.92};
  Plan best{2, 1};
  double best_t = 1e300;
  for (auto& c : cand) {
    if (c[0] == 1 && !big_square_ok(mode)) continue;
    int bm = c[1], bn = c[2];
    int64_t tiles = cdiv(M, bm) * cdiv(N, bn);
    int S = 1;
    if (mode == EPI_ACC_F32 && tiles < kCUs && K >= 2048) {
      S = (int)(kCUs / tiles);
      S = S > 16 ? 16 : S;
      int maxs = K / 1024;
      S = S > maxs ? maxs : S;
      S = S < 1 ? 1 : S;
    }
    int64_t rounds = cdiv(tiles * S, kCUs);
    double t = (double)rounds * bm * bn * (double)cdiv(K, S) / eff[c[0]];
    if (t < best_t) {
      best_t = t;
      best = {c[0], S};
    }
  }
  return best;
}

// Bytes an operand spans: rows x pitch (k-major) or K x pitch (m-major).
int64_t operand_span(bool kmajor, int rows, int K, int64_t ld) {
  return (kmajor ? (int64_t)rows : (int64_t)K) * ld * 2;
}

template <int BM, int BN, int MODE>
hipError_t launch_big(bool akm, bool bkm, int M, int N, int K, const bf16* a, int64_t lda,
                      const bf16* b, int64_t ldb, const Epilogue& e, int splits, hipStream_t s,
                      bool persistent = true) {
  int tiles_m = (int)cdiv(M, BM), tiles_n = (int)cdiv(N, BN);
  int kps = (int)round_up(cdiv(K, splits), 64);
  // one workgroup per CU (the LDS use allows no more), each looping over
  // tiles; or one workgroup per tile, so that CUs that free up while another
  // stream's kernel holds the rest keep taking tiles
  const int64_t ntiles = (int64_t)tiles_m * tiles_n;
  const int g = (int)(splits > 1 || !persistent ? ntiles : (ntiles < kCUs ? ntiles : kCUs));
  dim3 grid((unsigned)g, (unsigned)splits);
  BigBatch batch{};
  batch.p[0] = BigProblem{M, N, tiles_m, tiles_n, a, lda, b, ldb, e};
  batch.grouped = 0;
  batch.n = 1;
  batch.splits = splits;
#define GO(AK, BK_) gemm_big_kernel<BM, BN, AK, BK_, MODE><<<grid, BigWaves<BN>::NW * 64, 0, s>>>(batch, K, kps)
  if (akm && bkm) GO(true, true);
  else if (akm && !bkm) GO(true, false);
  else if (!akm && !bkm) GO(false, false);
  else GO(false, true);
#undef GO
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int dt, bool akm, bool bkm, int M, int N, int K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, const Epilogue& e, hipStream_t s, void* ws,
                       size_t ws_bytes, bool persistent) {
  if (dt == F32) {
    dim3 grid((unsigned)cdiv(N, 64), (unsigned)cdiv(M, 64));
    gemm_simt_kernel<MODE><<<grid, 256, 0, s>>>(akm, bkm, M, N, K, (const float*)A, lda,
                                                 (const float*)B, ldb, e);
    return hipGetLastError();
  }
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  Plan p = plan_gemm(M, N, K, MODE);
  // the large-tile kernels address each operand through a buffer resource
  // with 32-bit byte offsets
  const int64_t span_a = (operand_span(akm, M, K, lda)), span_b = operand_span(bkm, N, K, ldb);
  if (span_a >= (int64_t(1) << 31) || span_b >= (int64_t(1) << 31)) p = {0, 1};
  if (p.kind == 0) {
    dim3 grid((unsigned)cdiv(N, MF_BN), (unsigned)cdiv(M, MF_BM));
    if (akm && bkm) gemm_mfma_kernel<true, true, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
    else if (akm && !bkm) gemm_mfma_kernel<true, false, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
    else if (!akm && !bkm) gemm_mfma_kernel<false, false, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
    else gemm_mfma_kernel<false, true, MODE><<<grid, 256, 0, s>>>(M, N, K, a, lda, b, ldb, e);
    return hipGetLastError();
  }
  if constexpr (MODE == EPI_ACC_F32) {
    if (p.splits > 1) {
      size_t need = (size_t)p.splits * M * N * sizeof(float);
      if (!ws || ws_bytes < need || N % 4 != 0 || e.ldo % 4 != 0) {
        p.splits = 1;  // not enough scratch: run unsplit
      } else {
        Epilogue pe = e;
        pe.mode = EPI_PARTIAL;
        pe.out = ws;
        hipError_t err =
            p.kind == 1 ? launch_big<256, 256, EPI_PARTIAL>(akm, bkm, M, N, K, a, lda, b, ldb, pe, p.splits, s)
            : p.kind == 3 ? launch_big<256, 192, EPI_PARTIAL>(akm, bkm, M, N, K, a, lda, b, ldb, pe, p.splits, s)
                          : launch_big<256, 128, EPI_PARTIAL>(akm, bkm, M, N, K, a, lda, b, ldb, pe, p.splits, s);
        if (err != hipSuccess) return err;
        int64_t n4 = (int64_t)M * N / 4;
        splitk_reduce_kernel<<<(unsigned)cdiv(n4, 256), 256, 0, s>>>((float*)e.out, e.ldo,
                                                                    (const float*)ws, p.splits, M, N);
        return hipGetLastError();
      }
    }
  }
  if constexpr (big_square_ok(MODE)) {
    if (p.kind == 1) return launch_big<256, 256, MODE>(akm, bkm, M, N, K, a, lda, b, ldb, e, 1, s, persistent);
  }
  if (p.kind == 3) return launch_big<256, 192, MODE>(akm, bkm, M, N, K, a, lda, b, ldb, e, 1, s, persistent);
  return launch_big<256, 128, MODE>(akm, bkm, M, N, K, a, lda, b, ldb, e, 1, s, persistent);
}

}  // namespace

// Weight-gradient products with more 256 x 256 tiles than CUs but a last
// round less than half full (the tied-head gradient: 591 tiles on 256 CUs)
// are cut by rows: the rows that fill whole rounds run unsplit, the rest
// with split-K, so that the tail costs a fraction of a round.  Returns the
// rows of the first part, or 0 to run the product whole.
int acc_row_split(int dt, int M, int N, int K, int mode) {
  if (dt != BF16 || mode != EPI_ACC_F32) return 0;
  const Plan p = plan_gemm(M, N, K, mode);
  if (p.kind != 1 || p.splits != 1) return 0;
  const int64_t tn = cdiv(N, 256), tiles = cdiv(M, 256) * tn;
  const int64_t full = tiles / kCUs * kCUs, rest = tiles - full;
  if (full == 0 || rest == 0 || rest * 2 > kCUs) return 0;
  const int64_t rows = full / tn * 256;
  return rows > 0 && rows < M ? (int)rows : 0;
}

// ---------------------------------------------------------------- grouped weight gradients
// out_i (fp32) += A_i^T B_i for up to kMaxGroup products that share K (the
// token count): A_i[k * lda + m] (m < M_i), B_i[k * ldb + n] (n < N_i).  The
// four weight gradients of a layer have 9-36 output tiles each, far fewer
// than the CUs; run as one launch, their tiles together fill the chip with
// a split of K into S parts (S from the total tile count), so that the
// partial tiles cost S x (sum of M_i N_i) floats instead of each product's
// own, larger split; two layers' (216 tiles at GPT-2 124M) need no split at
// all.  Returns the split, or 0 where the grouped launch does not apply
// (more tiles than CUs, fp32, pitches or spans it cannot address).
int gemm_acc_group_splits(int dt, int n, const AccItem* it, int K) {
  if (dt != BF16 || n < 1 || n > kMaxGroup || K % 8 != 0 || K <= 0) return 0;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (it[i].M < 256 || it[i].N < 128 || it[i].lda % 8 || it[i].ldb % 8) return 0;
    if (operand_span(false, it[i].M, K, it[i].lda) >= (int64_t(1) << 31) ||
        operand_span(false, it[i].N, K, it[i].ldb) >= (int64_t(1) << 31))
      return 0;
    total += cdiv(it[i].M, 256) * cdiv(it[i].N, 256);
  }
  if (total > kCUs) return 0;
  int S = (int)(kCUs / total);
  S = std::min(S, 16);
  S = std::min(S, std::max(1, K / 1024));
  return std::max(S, 1);
}

size_t gemm_acc_group_workspace_bytes(int dt, int n, const AccItem* it, int K) {
  const int S = gemm_acc_group_splits(dt, n, it, K);
  if (S <= 1) return 0;
  size_t t = 0;
  for (int i = 0; i < n; ++i) t += round_up((int64_t)it[i].M * it[i].N, 64) * sizeof(float);
  return t * S;
}

hipError_t gemm_acc_group(int dt, int n, const AccItem* it, int K, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  int S = gemm_acc_group_splits(dt, n, it, K);
  bool vec4 = true;
  for (int i = 0; i < n; ++i) vec4 = vec4 && it[i].N % 4 == 0 && it[i].ldo % 4 == 0;
  if (S > 1 && (!ws || ws_bytes < gemm_acc_group_workspace_bytes(dt, n, it, K) || !vec4)) S = 0;
  if (S == 0) {  // one launch per product
    for (int i = 0; i < n; ++i) {
      Epilogue e{};
      e.mode = EPI_ACC_F32;
      e.out = it[i].out;
      e.ldo = it[i].ldo;
      hipError_t err = gemm(dt, false, false, it[i].M, it[i].N, K, it[i].A, it[i].lda, it[i].B,
                            it[i].ldb, e, s, ws, ws_bytes);
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  }
  BigBatch batch{};
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    BigProblem& p = batch.p[i];
    p.M = it[i].M;
    p.N = it[i].N;
    p.tiles_m = (int)cdiv(p.M, 256);
    p.tiles_n = (int)cdiv(p.N, 256);
    p.A = (const bf16*)it[i].A;
    p.lda = it[i].lda;
    p.B = (const bf16*)it[i].B;
    p.ldb = it[i].ldb;
    p.e = Epilogue{};
    if (S > 1) {
      p.e.mode = EPI_PARTIAL;
      p.e.out = (char*)ws + off;
      off += round_up((int64_t)p.M * p.N, 64) * sizeof(float) * S;
    } else {
      p.e.mode = EPI_ACC_F32;
      p.e.out = it[i].out;
      p.e.ldo = it[i].ldo;
    }
    batch.item0[i + 1] = batch.item0[i] + p.tiles_m * p.tiles_n * S;
  }
  batch.grouped = 1;
  batch.n = n;
  batch.splits = S;
  const int kps = (int)round_up(cdiv(K, S), 64);
  dim3 grid((unsigned)batch.item0[n]);
  if (S > 1)
    gemm_big_kernel<256, 256, false, false, EPI_PARTIAL><<<grid, 512, 0, s>>>(batch, K, kps);
  else
    gemm_big_kernel<256, 256, false, false, EPI_ACC_F32><<<grid, 512, 0, s>>>(batch, K, kps);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || S == 1) return err;
  ReduceBatch rb{};
  rb.n = n;
  rb.S = S;
  for (int i = 0; i < n; ++i) {
    rb.dst[i] = it[i].out;
    rb.ldo[i] = it[i].ldo;
    rb.part[i] = (const float*)batch.p[i].e.out;
    rb.M[i] = it[i].M;
    rb.N[i] = it[i].N;
    rb.q0[i + 1] = rb.q0[i] + (int64_t)it[i].M * it[i].N / 4;  // N % 4 == 0 here
  }
  splitk_reduce_group_kernel<<<(unsigned)cdiv(rb.q0[n], 256), 256, 0, s>>>(rb);
  return hipGetLastError();
}

size_t gemm_workspace_bytes(int dt, int M, int N, int K, int mode) {
  if (dt != BF16 || mode != EPI_ACC_F32) return 0;
  const int r = acc_row_split(dt, M, N, K, mode);
  if (r > 0) return std::max(gemm_workspace_bytes(dt, r, N, K, mode),
                             gemm_workspace_bytes(dt, M - r, N, K, mode));
  Plan p = plan_gemm(M, N, K, mode);
  if (p.kind == 0 || p.splits <= 1) return 0;
  return (size_t)p.splits * M * N * sizeof(float);
}

// The column sums come from the large-tile kernels' epilogue only: bf16,
// GELU backward, and a plan and operand spans that select those kernels.
bool gemm_colsum_ok(int dt, bool a_kmajor, bool b_kmajor, int M, int N, int K, int64_t lda,
                    int64_t ldb, int mode) {
  if (dt != BF16 || mode != EPI_GELU_BWD || M <= 0 || N <= 0 || lda % 8 || ldb % 8) return false;
  const Plan p = plan_gemm(M, N, K, mode);
  return p.kind != 0 && operand_span(a_kmajor, M, K, lda) < (int64_t(1) << 31) &&
         operand_span(b_kmajor, N, K, ldb) < (int64_t(1) << 31);
}

bool gemm_rowstats_ok(int dt, int M, int N, int K, int64_t lda, int64_t ldb) {
  return dt == BF16 && M >= 256 && N >= 256 && K > 0 && K % 8 == 0 && lda % 8 == 0 &&
         ldb % 8 == 0 && lda >= K && ldb >= K && operand_span(true, M, K, lda) < (int64_t(1) << 31) &&
         operand_span(true, N, K, ldb) < (int64_t(1) << 31);
}

hipError_t gemm_rowstats(int M, int N, int K, const void* A, int64_t lda, const void* B,
                         int64_t ldb, int V, const int32_t* target, float2* stats, int64_t ld,
                         float* tgt, hipStream_t s) {
  if (!gemm_rowstats_ok(BF16, M, N, K, lda, ldb)) return hipErrorNotSupported;
  if (V < 1 || V > N || ld < gemm_rowstats_cols(N) || !target || !stats || !tgt)
    return hipErrorInvalidValue;
  Epilogue e{};
  e.mode = EPI_ROWSTATS;
  e.out = stats;
  e.ldo = ld;
  e.aux = target;
  e.ldx = V;
  e.out2 = tgt;
  const int tiles_m = (int)cdiv(M, 256), tiles_n = (int)cdiv(N, 256);
  const int64_t ntiles = (int64_t)tiles_m * tiles_n;
  BigBatch batch{};
  batch.p[0] = BigProblem{M, N, tiles_m, tiles_n, (const bf16*)A, lda, (const bf16*)B, ldb, e};
  batch.grouped = 0;
  batch.n = 1;
  batch.splits = 1;
  dim3 grid((unsigned)(ntiles < kCUs ? ntiles : kCUs), 1);
  gemm_big_kernel<256, 256, true, true, EPI_ROWSTATS><<<grid, BIG_THREADS, 0, s>>>(
      batch, K, (int)round_up(K, 64));
  return hipGetLastError();
}

bool gemm_dlogits_ok(int dt, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldo) {
  return gemm_rowstats_ok(dt, M, N, K, lda, ldb) && ldo % 8 == 0 && ldo >= N;
}

hipError_t gemm_dlogits(int M, int N, int K, const void* A, int64_t lda, const void* B,
                        int64_t ldb, const float* lse, const int32_t* targets, int col0, int V,
                        float scale, void* out, int64_t ldo, hipStream_t s) {
  if (!gemm_dlogits_ok(BF16, M, N, K, lda, ldb, ldo)) return hipErrorNotSupported;
  if (V < 1 || col0 < 0 || !lse || !targets || !out) return hipErrorInvalidValue;
  Epilogue e{};
  e.mode = EPI_DLOGITS;
  e.out = out;
  e.ldo = ldo;
  e.lse = lse;
  e.targets = targets;
  e.col0 = col0;
  e.vocab = V;
  e.scale = scale;
  return launch_big<256, 192, EPI_DLOGITS>(true, true, M, N, K, (const bf16*)A, lda,
                                           (const bf16*)B, ldb, e, 1, s);
}

hipError_t gemm(int dt, bool a_kmajor, bool b_kmajor, int M, int N, int K, const void* A,
                int64_t lda, const void* B, int64_t ldb, const Epilogue& e, hipStream_t s,
                void* ws, size_t ws_bytes, bool persistent) {
  if (e.colsum) {
    if (!gemm_colsum_ok(dt, a_kmajor, b_kmajor, M, N, K, lda, ldb, e.mode)) return hipErrorNotSupported;
    if (e.ldcs < N || e.ldcs % 2 != 0 || reinterpret_cast<uintptr_t>(e.colsum) % 8 != 0)
      return hipErrorInvalidValue;
  }
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dt == BF16 && (lda % 8 != 0 || ldb % 8 != 0)) return hipErrorInvalidValue;
  if (const int r = acc_row_split(dt, M, N, K, e.mode)) {
    hipError_t err = launch_mode<EPI_ACC_F32>(dt, a_kmajor, b_kmajor, r, N, K, A, lda, B, ldb, e, s,
                                              ws, ws_bytes, true);
    if (err != hipSuccess) return err;
    const bf16* A2 = (const bf16*)A + (a_kmajor ? (int64_t)r * lda : (int64_t)r);
    Epilogue e2 = e;
    e2.out = (float*)e.out + (int64_t)r * e.ldo;
    return launch_mode<EPI_ACC_F32>(dt, a_kmajor, b_kmajor, M - r, N, K, A2, lda, B, ldb, e2, s,
                                    ws, ws_bytes, true);
  }
#define CASE(MD) \
  case MD: return launch_mode<MD>(dt, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, e, s, ws, ws_bytes, persistent);
  switch (e.mode) {
    CASE(EPI_STORE)
    CASE(EPI_BIAS)
    CASE(EPI_BIAS_RESID)
    CASE(EPI_BIAS_GELU)
    CASE(EPI_GELU_BWD)
    CASE(EPI_ACC_F32)
  }
#undef CASE
  return hipErrorInvalidValue;
}

}  // namespace gk
