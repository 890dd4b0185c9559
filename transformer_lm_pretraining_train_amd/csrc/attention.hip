// Causal multi-head self-attention for the GPT-2 step on gfx950, flash
// style: the T x T score matrix is never stored.  Scores S = q k^T / sqrt(hd)
// with j <= i, softmax over j, O = P v; the forward keeps the row
// log-sum-exp L so that the backward can rebuild P = exp(S - L) tile by tile.
//
// This file holds the generic kernels (any head size up to 128, fp32 or
// bf16 storage, fp32 arithmetic): one thread per query (forward, dQ) or per
// key (dK/dV), with 64-row K/V (or Q/dO) tiles staged through LDS.  They
// serve the fp32 mode and head sizes without a matrix-core kernel; the
// bf16 head-size-64 path uses the MFMA kernels in attention_mfma.hip.
//
// Backward is split in two passes so that no gradient needs atomics:
//   pass 1 (per query i): D_i = sum_d dO_i O_i, dQ_i = scale sum_j dS_ij k_j
//   pass 2 (per key j):   dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij q_i
// with dS_ij = P_ij (dO_i . v_j - D_i).
#include <mutex>

#include "common.h"
#include "kernels.h"

// Fixed device-resident scratch for the attention backward's entry point
// that allocates nothing (attention_backward_noalloc): the per-row values
// D = rowsum(dO * O) the dQ pass writes and the dK/dV pass reads.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never passes this name to a kernel: it is a host-side stand-in, not a
// device address; the address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) float scratch[gk::kNoAllocAttnScratchFloats];

namespace gk {

bool attention_mfma_supported(int dt, int hd);
hipError_t attention_forward_mfma(void* out, float* lse, const void* qkv, int B, int T, int H,
                                  hipStream_t s);
hipError_t attention_backward_mfma(void* dqkv, const void* dout, const void* qkv, const void* out,
                                   const float* lse, float* Dbuf, int B, int T, int H,
                                   hipStream_t s, float* colsum);

constexpr int AT_TILE = 64;

template <class T, int HD>
__device__ __forceinline__ void load_row(const T* p, float* v) {
#pragma unroll
  for (int d = 0; d < HD; d += 8) {
    Pack<T> a;
    if constexpr (sizeof(T) == 2) {
      a = load_pack(p + d);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[d + i] = to_f(a.e[i]);
    } else {
      float4 x = *reinterpret_cast<const float4*>(p + d);
      float4 y = *reinterpret_cast<const float4*>(p + d + 4);
      v[d + 0] = x.x; v[d + 1] = x.y; v[d + 2] = x.z; v[d + 3] = x.w;
      v[d + 4] = y.x; v[d + 5] = y.y; v[d + 6] = y.z; v[d + 7] = y.w;
    }
  }
}

// Cooperative load of a tile of up to 64 rows (head slice of width HD) into
// LDS as fp32, zero rows past T.  64 threads.
template <class T, int HD>
__device__ __forceinline__ void load_tile(float (*S)[HD + 1], const T* base, int64_t ld, int row0,
                                          int Tn) {
  for (int c = threadIdx.x; c < AT_TILE * (HD / 8); c += blockDim.x) {
    int r = c / (HD / 8), d = (c % (HD / 8)) * 8;
    float v[8];
    if (row0 + r < Tn) {
      load_row<T, 8>(base + (int64_t)(row0 + r) * ld + d, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) S[r][d + i] = v[i];
  }
}

template <class T, int HD>
__global__ __launch_bounds__(64) void attn_fwd_generic(T* __restrict__ out, float* __restrict__ lse,
                                                       const T* __restrict__ qkv, int Tn, int H) {
  __shared__ float Ks[AT_TILE][HD + 1];
  __shared__ float Vs[AT_TILE][HD + 1];
  const int C = H * HD;
  const int64_t ld = 3 * (int64_t)C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = blockIdx.x * AT_TILE;
  const int i = q0 + threadIdx.x;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const float scale = 1.0f / sqrtf((float)HD);
  float q[HD], o[HD];
  if (i < Tn) load_row<T, HD>(base + (int64_t)i * ld + h * HD, q);
  else
#pragma unroll
    for (int d = 0; d < HD; ++d) q[d] = 0.f;
#pragma unroll
  for (int d = 0; d < HD; ++d) o[d] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const int kend = min(q0 + AT_TILE, Tn);
  for (int k0 = 0; k0 < kend; k0 += AT_TILE) {
    __syncthreads();
    load_tile<T, HD>(Ks, base + C + h * HD, ld, k0, Tn);
    load_tile<T, HD>(Vs, base + 2 * C + h * HD, ld, k0, Tn);
    __syncthreads();
    float s[AT_TILE];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < AT_TILE; ++j) {
      int key = k0 + j;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc = fmaf(q[d], Ks[j][d], acc);
      s[j] = (key <= i && key < Tn) ? acc * scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    if (tmax > -INFINITY) {
      float mnew = fmaxf(mrun, tmax);
      float alpha = fast_exp(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int d = 0; d < HD; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < AT_TILE; ++j) {
        float p = fast_exp(s[j] - mnew);
        lrun += p;
#pragma unroll
        for (int d = 0; d < HD; ++d) o[d] = fmaf(p, Vs[j][d], o[d]);
      }
      mrun = mnew;
    }
  }
  if (i < Tn) {
    float inv = 1.0f / lrun;
    T* dst = out + ((int64_t)b * Tn + i) * C + h * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) dst[d] = from_f<T>(o[d] * inv);
    lse[(int64_t)bh * Tn + i] = mrun + logf(lrun);
  }
}

// pass 1: one thread per query.
template <class T, int HD>
__global__ __launch_bounds__(64) void attn_bwd_dq_generic(T* __restrict__ dqkv, float* __restrict__ Dbuf,
                                                          const T* __restrict__ dout,
                                                          const T* __restrict__ qkv,
                                                          const T* __restrict__ out,
                                                          const float* __restrict__ lse, int Tn,
                                                          int H) {
  __shared__ float Ks[AT_TILE][HD + 1];
  __shared__ float Vs[AT_TILE][HD + 1];
  const int C = H * HD;
  const int64_t ld = 3 * (int64_t)C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = blockIdx.x * AT_TILE;
  const int i = q0 + threadIdx.x;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const float scale = 1.0f / sqrtf((float)HD);
  float q[HD], dO[HD], dq[HD];
  float Di = 0.f, Li = 0.f;
  if (i < Tn) {
    float o[HD];
    load_row<T, HD>(base + (int64_t)i * ld + h * HD, q);
    load_row<T, HD>(dout + ((int64_t)b * Tn + i) * C + h * HD, dO);
    load_row<T, HD>(out + ((int64_t)b * Tn + i) * C + h * HD, o);
#pragma unroll
    for (int d = 0; d < HD; ++d) Di = fmaf(dO[d], o[d], Di);
    Li = lse[(int64_t)bh * Tn + i];
    Dbuf[(int64_t)bh * Tn + i] = Di;
  } else {
#pragma unroll
    for (int d = 0; d < HD; ++d) q[d] = dO[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < HD; ++d) dq[d] = 0.f;
  const int kend = min(q0 + AT_TILE, Tn);
  for (int k0 = 0; k0 < kend; k0 += AT_TILE) {
    __syncthreads();
    load_tile<T, HD>(Ks, base + C + h * HD, ld, k0, Tn);
    load_tile<T, HD>(Vs, base + 2 * C + h * HD, ld, k0, Tn);
    __syncthreads();
    if (i < Tn) {
      for (int j = 0; j < AT_TILE; ++j) {
        int key = k0 + j;
        if (key > i || key >= Tn) break;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
          s = fmaf(q[d], Ks[j][d], s);
          dp = fmaf(dO[d], Vs[j][d], dp);
        }
        float p = fast_exp(s * scale - Li);
        float ds = p * (dp - Di);
#pragma unroll
        for (int d = 0; d < HD; ++d) dq[d] = fmaf(ds, Ks[j][d], dq[d]);
      }
    }
  }
  if (i < Tn) {
    T* dst = dqkv + ((int64_t)b * Tn + i) * ld + h * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) dst[d] = from_f<T>(dq[d] * scale);
  }
}

// pass 2: one thread per key.
template <class T, int HD>
__global__ __launch_bounds__(64) void attn_bwd_dkv_generic(T* __restrict__ dqkv,
                                                           const float* __restrict__ Dbuf,
                                                           const T* __restrict__ dout,
                                                           const T* __restrict__ qkv,
                                                           const float* __restrict__ lse, int Tn,
                                                           int H) {
  __shared__ float Qs[AT_TILE][HD + 1];
  __shared__ float Os[AT_TILE][HD + 1];  // dO tile
  __shared__ float Ls[AT_TILE], Ds[AT_TILE];
  const int C = H * HD;
  const int64_t ld = 3 * (int64_t)C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int j0 = blockIdx.x * AT_TILE;
  const int j = j0 + threadIdx.x;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const float scale = 1.0f / sqrtf((float)HD);
  float k[HD], v[HD], dk[HD], dv[HD];
  if (j < Tn) {
    load_row<T, HD>(base + (int64_t)j * ld + C + h * HD, k);
    load_row<T, HD>(base + (int64_t)j * ld + 2 * C + h * HD, v);
  } else {
#pragma unroll
    for (int d = 0; d < HD; ++d) k[d] = v[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < HD; ++d) dk[d] = dv[d] = 0.f;
  for (int i0 = j0; i0 < Tn; i0 += AT_TILE) {
    __syncthreads();
    load_tile<T, HD>(Qs, base + h * HD, ld, i0, Tn);
    load_tile<T, HD>(Os, dout + (int64_t)b * Tn * C + h * HD, C, i0, Tn);
    for (int r = threadIdx.x; r < AT_TILE; r += blockDim.x) {
      int i = i0 + r;
      Ls[r] = i < Tn ? lse[(int64_t)bh * Tn + i] : 0.f;
      Ds[r] = i < Tn ? Dbuf[(int64_t)bh * Tn + i] : 0.f;
    }
    __syncthreads();
    if (j < Tn) {
      for (int r = 0; r < AT_TILE; ++r) {
        int i = i0 + r;
        if (i >= Tn) break;
        if (i < j) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
          s = fmaf(Qs[r][d], k[d], s);
          dp = fmaf(Os[r][d], v[d], dp);
        }
        float p = fast_exp(s * scale - Ls[r]);
        float ds = p * (dp - Ds[r]);
#pragma unroll
        for (int d = 0; d < HD; ++d) {
          dv[d] = fmaf(p, Os[r][d], dv[d]);
          dk[d] = fmaf(ds, Qs[r][d], dk[d]);
        }
      }
    }
  }
  if (j < Tn) {
    T* dst = dqkv + ((int64_t)b * Tn + j) * ld + h * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      dst[C + d] = from_f<T>(dk[d] * scale);
      dst[2 * C + d] = from_f<T>(dv[d]);
    }
  }
}

template <class T, int HD>
static void launch_fwd(void* out, float* lse, const void* qkv, int B, int Tn, int H, hipStream_t s) {
  dim3 grid((unsigned)cdiv(Tn, AT_TILE), (unsigned)(B * H));
  attn_fwd_generic<T, HD><<<grid, 64, 0, s>>>((T*)out, lse, (const T*)qkv, Tn, H);
}

template <class T, int HD>
static void launch_bwd(void* dqkv, float* Dbuf, const void* dout, const void* qkv, const void* out,
                       const float* lse, int B, int Tn, int H, hipStream_t s) {
  dim3 grid((unsigned)cdiv(Tn, AT_TILE), (unsigned)(B * H));
  attn_bwd_dq_generic<T, HD><<<grid, 64, 0, s>>>((T*)dqkv, Dbuf, (const T*)dout, (const T*)qkv,
                                                 (const T*)out, lse, Tn, H);
  attn_bwd_dkv_generic<T, HD><<<grid, 64, 0, s>>>((T*)dqkv, Dbuf, (const T*)dout, (const T*)qkv,
                                                  lse, Tn, H);
}

#define AT_DISPATCH_HD(hd, FN, ...)             \
  switch (hd) {                                 \
    case 16: FN<T, 16>(__VA_ARGS__); break;     \
    case 32: FN<T, 32>(__VA_ARGS__); break;     \
    case 64: FN<T, 64>(__VA_ARGS__); break;     \
    case 128: FN<T, 128>(__VA_ARGS__); break;   \
    default: return hipErrorInvalidValue;       \
  }

hipError_t attention_forward(int dt, void* out, float* lse, const void* qkv, int B, int Tn, int H,
                             int hd, hipStream_t s) {
  if (attention_mfma_supported(dt, hd)) return attention_forward_mfma(out, lse, qkv, B, Tn, H, s);
  if (dt == BF16) {
    using T = bf16;
    AT_DISPATCH_HD(hd, launch_fwd, out, lse, qkv, B, Tn, H, s);
  } else {
    using T = float;
    AT_DISPATCH_HD(hd, launch_fwd, out, lse, qkv, B, Tn, H, s);
  }
  return hipGetLastError();
}

size_t attention_backward_scratch_bytes(int B, int T, int H) {
  return (size_t)B * H * T * sizeof(float);
}

bool attention_colsum_ok(int dt, int hd) { return attention_mfma_supported(dt, hd); }

hipError_t attention_backward(int dt, void* dqkv, const void* dout, const void* qkv,
                              const void* out, const float* lse, int B, int Tn, int H, int hd,
                              void* scratch, hipStream_t s, float* colsum) {
  float* Dbuf = (float*)scratch;
  if (attention_mfma_supported(dt, hd))
    return attention_backward_mfma(dqkv, dout, qkv, out, lse, Dbuf, B, Tn, H, s, colsum);
  if (colsum) return hipErrorNotSupported;
  if (dt == BF16) {
    using T = bf16;
    AT_DISPATCH_HD(hd, launch_bwd, dqkv, Dbuf, dout, qkv, out, lse, B, Tn, H, s);
  } else {
    using T = float;
    AT_DISPATCH_HD(hd, launch_bwd, dqkv, Dbuf, dout, qkv, out, lse, B, Tn, H, s);
  }
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
static hipError_t noalloc_scratch(float** out) {
  static std::mutex mu;
  static float* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = (float*)p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t attention_backward_noalloc(int dt, void* dqkv, const void* dout, const void* qkv,
                                      const void* out, const float* lse, int B, int Tn, int H,
                                      int hd, hipStream_t s, float* colsum) {
  if ((int64_t)B * H * Tn > (int64_t)kNoAllocAttnScratchFloats) return hipErrorInvalidValue;
  float* D = nullptr;
  const hipError_t e = noalloc_scratch(&D);
  if (e != hipSuccess) return e;
  return attention_backward(dt, dqkv, dout, qkv, out, lse, B, Tn, H, hd, D, s, colsum);
}

}  // namespace gk
