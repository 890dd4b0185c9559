// Memory-bound kernels of the GPT-2 step for gfx950: embedding gather and
// scatter, LayerNorm forward/backward, bias gradients, the masked softmax
// cross-entropy over the padded vocabulary, and the optimizer (global norm,
// clip, AdamW), plus fills and casts.
//
// All of them stream rows with 16-byte accesses and reduce within a wave64
// (shuffles) or a workgroup (LDS); column reductions (LayerNorm gain/shift
// and bias gradients) are two-stage with partials in a scratch buffer and a
// fixed summation order, so they are bitwise repeatable.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {

// 8 consecutive elements <-> floats
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  Pack<bf16> a = load_pack(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = to_f(a.e[i]);
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
  Pack<bf16> a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.e[i] = from_f<bf16>(v[i]);
  store_pack(p, a);
}

#define DISPATCH_DT(dt, ...)                 \
  do {                                       \
    if ((dt) == BF16) {                      \
      typedef bf16 T;                        \
      __VA_ARGS__;                           \
    } else {                                 \
      typedef float T;                       \
      __VA_ARGS__;                           \
    }                                        \
  } while (0)

static inline int grid_for(int64_t n, int block) { return (int)cdiv(n, block); }

// =========================================================== embedding
// x0[m, c] = wte[tok[m], c] + wpe[m % T, c]; one thread per 8 channels.
template <class T>
__global__ void encoder_fwd_kernel(T* __restrict__ out, const int32_t* __restrict__ tok,
                                   const float* __restrict__ wte, const float* __restrict__ wpe,
                                   int M, int Tn, int C, int V, int* __restrict__ flag) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int cpr = C / 8;
  if (idx >= (int64_t)M * cpr) return;
  int m = (int)(idx / cpr);
  int c = (int)(idx % cpr) * 8;
  int t = m % Tn;
  int id = tok[m];
  if (id < 0 || id >= V) {
    if (c == 0) atomicOr(flag, 1);
    id = id < 0 ? 0 : V - 1;
  }
  float a[8], b[8];
  load8(wte + (int64_t)id * C + c, a);
  load8(wpe + (int64_t)t * C + c, b);
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] += b[i];
  store8(out + (int64_t)m * C + c, a);
}

hipError_t encoder_forward(int dt, void* out, const int32_t* tok, const float* wte,
                           const float* wpe, int M, int Tn, int C, int V, int* err_flag,
                           hipStream_t s) {
  int64_t n = (int64_t)M * (C / 8);
  DISPATCH_DT(dt, encoder_fwd_kernel<T><<<grid_for(n, 256), 256, 0, s>>>(
                      (T*)out, tok, wte, wpe, M, Tn, C, V, err_flag));
  return hipGetLastError();
}

// dwpe[t, c] += sum_b dx[b*T + t, c]; one thread per 8 channels of one t.
template <class T>
__global__ void encoder_bwd_wpe_kernel(float* __restrict__ dwpe, const T* __restrict__ dx, int B,
                                       int Tn, int C) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int cpr = C / 8;
  if (idx >= (int64_t)Tn * cpr) return;
  int t = (int)(idx / cpr);
  int c = (int)(idx % cpr) * 8;
  float acc[8], v[8];
  load8(dwpe + (int64_t)t * C + c, acc);
  for (int b = 0; b < B; ++b) {
    load8(dx + ((int64_t)b * Tn + t) * C + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  store8(dwpe + (int64_t)t * C + c, acc);
}

hipError_t encoder_backward_wpe(int dt, float* dwpe, const void* dx, int B, int Tn, int C,
                                hipStream_t s) {
  int64_t n = (int64_t)Tn * (C / 8);
  DISPATCH_DT(dt, encoder_bwd_wpe_kernel<T><<<grid_for(n, 256), 256, 0, s>>>(
                      dwpe, (const T*)dx, B, Tn, C));
  return hipGetLastError();
}

// =========================================================== LayerNorm
// One wave per row; lane j owns 8-element chunks j, j+64, ... (C % 8 == 0).
// 8 elements of T as loaded (16 or 32 bytes), unpacked to floats on use.
template <class T> struct Raw8 {  // 8 elements of T as loaded: 16 or 32 bytes
  uint4 u[sizeof(T) / 2];
};
template <class T> __device__ __forceinline__ void load_raw(const T* p, Raw8<T>& r) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.u[i] = reinterpret_cast<const uint4*>(p)[i];
}
__device__ __forceinline__ void unpack8(const Raw8<bf16>& r, float v[8]) {
  const uint32_t wd[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // element 2k in the low half of word k
    v[2 * k] = __uint_as_float(wd[k] << 16);
    v[2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float v[8]) {
  v[0] = __uint_as_float(r.u[0].x); v[1] = __uint_as_float(r.u[0].y);
  v[2] = __uint_as_float(r.u[0].z); v[3] = __uint_as_float(r.u[0].w);
  v[4] = __uint_as_float(r.u[1].x); v[5] = __uint_as_float(r.u[1].y);
  v[6] = __uint_as_float(r.u[1].z); v[7] = __uint_as_float(r.u[1].w);
}
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

constexpr int LN_MAXCH = 4;  // C <= 8 * 64 * 4 = 2048

template <class T>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(
    T* __restrict__ out, float* __restrict__ mean_out, float* __restrict__ rstd_out,
    const T* __restrict__ inp, const float* __restrict__ w, const float* __restrict__ b, int M,
    int C, float eps) {
  int row = blockIdx.x * 4 + threadIdx.x / 64;
  int lane = threadIdx.x % 64;
  if (row >= M) return;
  int nch = C / 8;
  const T* x = inp + (int64_t)row * C;
  float v[LN_MAXCH][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < LN_MAXCH; ++j) {
    int ch = lane + 64 * j;
    if (ch < nch) {
      load8(x + ch * 8, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[j][i];
    }
  }
  float mean = wave_sum(s) / C;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < LN_MAXCH; ++j) {
    int ch = lane + 64 * j;
    if (ch < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float d = v[j][i] - mean;
        ss += d * d;
      }
    }
  }
  float var = wave_sum(ss) / C;
  float rstd = 1.0f / sqrtf(var + eps);
  T* y = out + (int64_t)row * C;
#pragma unroll
  for (int j = 0; j < LN_MAXCH; ++j) {
    int ch = lane + 64 * j;
    if (ch < nch) {
      float wv[8], bv[8], o[8];
      load8(w + ch * 8, wv);
      load8(b + ch * 8, bv);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = (v[j][i] - mean) * rstd * wv[i] + bv[i];
      store8(y + ch * 8, o);
    }
  }
  if (lane == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// The same for C = 256 NC: a half-wave (32 lanes) per row, NC 8-column
// chunks per lane, so that every lane is busy and a wave has two rows in
// flight.
template <class T, int NC>
__global__ __launch_bounds__(256) void layernorm_fwd_hw_kernel(
    T* __restrict__ out, float* __restrict__ mean_out, float* __restrict__ rstd_out,
    const T* __restrict__ inp, const float* __restrict__ w, const float* __restrict__ b, int M,
    int C, float eps) {
  const int row = blockIdx.x * 8 + threadIdx.x / 32;
  const int l = threadIdx.x % 32;
  // Gain and shift staged once per workgroup through LDS: its eight rows
  // share them, and loading them per row from memory took 12 of a lane's 18
  // memory instructions per row (this kernel 9 % faster without them).
  __shared__ float4 wb[2 * 256 * NC / 4];
  for (int i = threadIdx.x; i < 2 * C / 4; i += 256)
    wb[i] = i < C / 4 ? reinterpret_cast<const float4*>(w)[i]
                      : reinterpret_cast<const float4*>(b)[i - C / 4];
  __syncthreads();
  if (row >= M) return;  // uniform over the half-wave
  Raw8<T> xr[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) load_raw(inp + (int64_t)row * C + (l + 32 * j) * 8, xr[j]);
  float v[NC][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    unpack8(xr[j], v[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[j][i];
  }
  const float mean = half_wave_sum(s) / C;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = v[j][i] - mean;
      ss += d * d;
    }
  const float rstd = 1.0f / sqrtf(half_wave_sum(ss) / C + eps);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = (l + 32 * j) * 8;
    float wv[8], bv[8], o[8];
    {
      const float4 w0 = wb[c / 4], w1 = wb[c / 4 + 1];
      const float4 b0 = wb[C / 4 + c / 4], b1 = wb[C / 4 + c / 4 + 1];
      wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
      wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
      bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
      bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (v[j][i] - mean) * rstd * wv[i] + bv[i];
    store8(out + (int64_t)row * C + c, o);
  }
  if (l == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

hipError_t layernorm_forward(int dt, void* out, float* mean, float* rstd, const void* inp,
                             const float* w, const float* b, int M, int C, float eps,
                             hipStream_t s) {
  if (C % 8 != 0 || C > 8 * 64 * LN_MAXCH) return hipErrorInvalidValue;
  if (C == 256 || C == 512 || C == 768) {
#define LNFH(NC)                                                                               \
  DISPATCH_DT(dt, layernorm_fwd_hw_kernel<T, NC><<<grid_for(M, 8), 256, 0, s>>>(               \
                      (T*)out, mean, rstd, (const T*)inp, w, b, M, C, eps))
    if (C == 256) LNFH(1);
    else if (C == 512) LNFH(2);
    else LNFH(3);
#undef LNFH
    return hipGetLastError();
  }
  DISPATCH_DT(dt, layernorm_fwd_kernel<T><<<grid_for(M, 4), 256, 0, s>>>(
                      (T*)out, mean, rstd, (const T*)inp, w, b, M, C, eps));
  return hipGetLastError();
}

// Backward: per row, g = dy * w, xhat = (x - mean) rstd,
// dx = rstd (g - mean(g) - xhat mean(g xhat)); dres = dx (first) or
// dres = dres_in + dx (dres_in may be dres itself).  Each workgroup handles
// LNB_ROWS rows and writes partial column sums of dy*xhat, of dy and of the
// new dres (the bias gradient of the linear layer whose output is that
// residual) to
// scratch[block][3][C]; column_partials_reduce adds them up.  NCH: 8-column
// chunks per lane (C <= 512 NCH), so that no registers are spent on
// columns that do not exist.
constexpr int LNB_ROWS = 32;

template <class T, int NCH>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(
    T* dres, const T* dres_in, float* __restrict__ partial, const T* __restrict__ dy,
    const T* __restrict__ inp, const float* __restrict__ mean, const float* __restrict__ rstd,
    const float* __restrict__ w, int M, int C, int accumulate) {
  extern __shared__ float red[];  // [3][C]
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int nch = C / 8;
  float dwacc[NCH][8], dbacc[NCH][8], doacc[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) dwacc[j][i] = dbacc[j][i] = doacc[j][i] = 0.f;

  const int row0 = blockIdx.x * LNB_ROWS;
  for (int r = wave; r < LNB_ROWS; r += 4) {
    const int row = row0 + r;
    if (row >= M) break;
    const float mu = mean[row], rs = rstd[row];
    const T* x = inp + (int64_t)row * C;
    const T* g = dy + (int64_t)row * C;
    T* d = dres + (int64_t)row * C;
    const T* din = dres_in + (int64_t)row * C;
    float xh[NCH][8], gw[NCH][8], dv[NCH][8];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = lane + 64 * j;
      if (ch < nch) {
        float xv[8], gv[8], wv[8];
        load8(x + ch * 8, xv);
        load8(g + ch * 8, gv);
        load8(w + ch * 8, wv);
        if (accumulate) load8(din + ch * 8, dv[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xh[j][i] = (xv[i] - mu) * rs;
          gw[j][i] = gv[i] * wv[i];
          s1 += gw[j][i];
          s2 += gw[j][i] * xh[j][i];
          dwacc[j][i] += gv[i] * xh[j][i];
          dbacc[j][i] += gv[i];
          if (!accumulate) dv[j][i] = 0.f;
        }
      }
    }
    s1 = wave_sum(s1) / C;
    s2 = wave_sum(s2) / C;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = lane + 64 * j;
      if (ch < nch) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dv[j][i] += rs * (gw[j][i] - s1 - xh[j][i] * s2);
          doacc[j][i] += dv[j][i];
        }
        store8(d + ch * 8, dv[j]);
      }
    }
  }
  // fixed-order reduction of the four waves' column sums
  for (int wv = 0; wv < 4; ++wv) {
    if (wave == wv) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int ch = lane + 64 * j;
        if (ch < nch) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = ch * 8 + i;
            if (wv == 0) {
              red[c] = dwacc[j][i];
              red[C + c] = dbacc[j][i];
              red[2 * C + c] = doacc[j][i];
            } else {
              red[c] += dwacc[j][i];
              red[C + c] += dbacc[j][i];
              red[2 * C + c] += doacc[j][i];
            }
          }
        }
      }
    }
    __syncthreads();
  }
  float* dst = partial + (int64_t)blockIdx.x * 3 * C;
  for (int c = threadIdx.x; c < 3 * C; c += blockDim.x) dst[c] = red[c];
}

// The same backward for C = 256 NC (the GPT-2 widths): a half-wave (32
// lanes) per row with NC 8-column chunks per lane, so that every lane is
// busy and each wave has two rows in flight, and the inputs of a wave's next
// pair of rows are loaded while the current pair is computed.  The two
// half-waves of a wave hold the same columns; their column sums are added by
// one lane exchange, then the four waves' sums in order through LDS.
template <class T, int NC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void layernorm_bwd_hw_kernel(
    T* dres, const T* dres_in, float* __restrict__ partial, const T* __restrict__ dy,
    const T* __restrict__ inp, const float* __restrict__ mean, const float* __restrict__ rstd,
    const float* __restrict__ w, int M, int C, int accumulate) {
  static_assert(LNB_ROWS % 8 == 0, "whole rows per half-wave");
  __shared__ float red[4][3 * 256 * NC];
  const int wave = threadIdx.x / 64, l = threadIdx.x % 32;
  const int hw = 2 * wave + (threadIdx.x / 32) % 2;  // half-wave: rows row0 + hw + 8 i
  float wv[NC][8];
#pragma unroll
  for (int j = 0; j < NC; ++j) load8(w + (l + 32 * j) * 8, wv[j]);
  float dwacc[NC][8], dbacc[NC][8], doacc[NC][8];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) dwacc[j][i] = dbacc[j][i] = doacc[j][i] = 0.f;

  // Branch-free loads through buffer resources: a row past M (and d res
  // when not accumulating: an empty resource) reads zeros, so the compiler
  // can count the loads in flight and wait only for the row it processes
  // (loaded inside branches, every row waited for the next row's prefetch
  // as well).
  const int nbytes = M * C * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)inp, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void*)dy, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)dres_in, (short)0, accumulate ? nbytes : 0, 0x00020000);
  auto bload = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t off, Raw8<T>& r) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) {
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0);
      r.u[i] = make_uint4(w.x, w.y, w.z, w.w);
    }
#else
    (void)rs;
    (void)off;
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.u[i] = make_uint4(0, 0, 0, 0);
#endif
  };
  auto fetch = [&](int row, Raw8<T> (&x)[NC], Raw8<T> (&g)[NC], Raw8<T> (&d)[NC]) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const uint32_t off = row < M ? (uint32_t)(((int64_t)row * C + (l + 32 * j) * 8) * sizeof(T))
                                   : 0x80000000u;
      bload(rx, off, x[j]);
      bload(rg, off, g[j]);
      bload(rd, off, d[j]);
    }
  };
  auto process = [&](int row, const Raw8<T> (&x)[NC], const Raw8<T> (&g)[NC],
                     const Raw8<T> (&d)[NC], float mu, float rs) {
    if (row >= M) return;  // uniform over the half-wave; its sums stay inside it
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float xv[8], gv[8];
      unpack8(x[j], xv);
      unpack8(g[j], gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xh = (xv[i] - mu) * rs, gw = gv[i] * wv[j][i];
        s1 += gw;
        s2 += gw * xh;
        dwacc[j][i] += gv[i] * xh;
        dbacc[j][i] += gv[i];
      }
    }
    s1 = half_wave_sum(s1) / C;
    s2 = half_wave_sum(s2) / C;
    // second pass over the same registers (x-hat and g*w recomputed, not kept)
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float xv[8], gv[8], dv[8];
      unpack8(x[j], xv);
      unpack8(g[j], gv);
      if (accumulate) unpack8(d[j], dv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xh = (xv[i] - mu) * rs, gw = gv[i] * wv[j][i];
        const float dx = rs * (gw - s1 - xh * s2);
        dv[i] = accumulate ? dv[i] + dx : dx;
        doacc[j][i] += dv[i];
      }
      store8(dres + (int64_t)row * C + (l + 32 * j) * 8, dv);
    }
  };

  const int r0 = blockIdx.x * LNB_ROWS + hw;
  constexpr int RPH = LNB_ROWS / 8;  // rows per half-wave
  // every row's mean and rstd first, so that waiting for them never waits
  // for a later row's prefetch (one in-order counter for all loads)
  float mus[RPH], rss[RPH];
#pragma unroll
  for (int i = 0; i < RPH; ++i) {
    const int rr = min(r0 + 8 * i, M - 1);
    mus[i] = mean[rr];
    rss[i] = rstd[rr];
  }
  Raw8<T> xa[NC], ga[NC], da[NC];
  fetch(r0, xa, ga, da);
#pragma unroll
  for (int i = 0; i < RPH; ++i) {
    Raw8<T> xb[NC], gb[NC], db[NC];
    if (i + 1 < RPH) fetch(r0 + 8 * (i + 1), xb, gb, db);
    process(r0 + 8 * i, xa, ga, da, mus[i], rss[i]);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      xa[j] = xb[j];
      ga[j] = gb[j];
      da[j] = db[j];
    }
  }
  // lanes l and l + 32 hold the same columns: add the two half-waves
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dwacc[j][i] += __shfl_xor(dwacc[j][i], 32, 64);
      dbacc[j][i] += __shfl_xor(dbacc[j][i], 32, 64);
      doacc[j][i] += __shfl_xor(doacc[j][i], 32, 64);
    }
  if (threadIdx.x % 64 < 32) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = (l + 32 * j) * 8 + i;
        red[wave][c] = dwacc[j][i];
        red[wave][C + c] = dbacc[j][i];
        red[wave][2 * C + c] = doacc[j][i];
      }
  }
  __syncthreads();
  float* dst = partial + (int64_t)blockIdx.x * 3 * C;
  for (int c = threadIdx.x; c < 3 * C; c += blockDim.x)
    dst[c] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// out_k[c] += sum_b partial[b * stride + k * C + c] for each non-null out_k
// (k = 0, 1, 2), summed in a fixed order.  A workgroup covers 4 Q columns of
// the concatenated outputs with Q float4 lanes x 256/Q groups of partial
// rows (group g sums rows g, g + 256/Q, ...); the group sums are added in
// order.  Q = 4 (16 columns) spreads one reduction over many workgroups;
// Q = 16 (64 columns, 256-byte row segments) reads more efficiently when
// many reductions share a launch.
template <int Q>
__device__ __forceinline__ void column_reduce_block(const ColReduce& d, int blk) {
  constexpr int G = 256 / Q;
  __shared__ float4 red[G][Q + 1];
  const int q = threadIdx.x % Q, g = threadIdx.x / Q;
  const int c = blk * 4 * Q + 4 * q;  // first of 4 columns (C % 4 == 0)
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < d.ncols) {
#pragma unroll 4
    for (int b = g; b < d.nb; b += G) {
      const float4 v = *reinterpret_cast<const float4*>(d.partial + (int64_t)b * d.stride + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  red[g][q] = acc;
  __syncthreads();
  if (g == 0 && c < d.ncols) {
    float4 t = red[0][q];
    for (int k = 1; k < G; ++k) {
      const float4 v = red[k][q];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    const int k = c / d.C, cc = c % d.C;
    float* o = k == 0 ? d.out0 : k == 1 ? d.out1 : d.out2;
    if (o) {
      float4* op = reinterpret_cast<float4*>(o + cc);
      float4 cur = *op;
      cur.x += t.x; cur.y += t.y; cur.z += t.z; cur.w += t.w;
      *op = cur;
    }
  }
}

__global__ __launch_bounds__(256) void column_partials_reduce_kernel(const ColReduce d) {
  column_reduce_block<4>(d, blockIdx.x);
}

// Several reductions in one launch: descriptor i owns workgroups blk0[i] ..
// blk0[i+1]-1.
constexpr int kColBatch = 32;
struct ColBatch {
  ColReduce d[kColBatch];
  int n;
  int blk0[kColBatch + 1];
};
__global__ __launch_bounds__(256) void column_reduce_batch_kernel(const ColBatch cb) {
  int i = 0;
  while (i + 1 < cb.n && (int)blockIdx.x >= cb.blk0[i + 1]) ++i;
  column_reduce_block<16>(cb.d[i], blockIdx.x - cb.blk0[i]);
}

static hipError_t column_reduce(const ColReduce& d, hipStream_t s) {
  column_partials_reduce_kernel<<<grid_for(d.ncols, 16), 256, 0, s>>>(d);
  return hipGetLastError();
}

hipError_t column_reduce_batched(const ColReduce* d, int n, hipStream_t s) {
  for (int i0 = 0; i0 < n; i0 += kColBatch) {
    ColBatch cb{};
    cb.n = std::min(kColBatch, n - i0);
    for (int i = 0; i < cb.n; ++i) {
      cb.d[i] = d[i0 + i];
      cb.blk0[i + 1] = cb.blk0[i] + grid_for(d[i0 + i].ncols, 64);
    }
    if (cb.blk0[cb.n] > 0) column_reduce_batch_kernel<<<cb.blk0[cb.n], 256, 0, s>>>(cb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t layernorm_backward_scratch_bytes(int M, int C) {
  return (size_t)cdiv(M, LNB_ROWS) * 3 * C * sizeof(float);
}

hipError_t layernorm_backward(int dt, void* dres, const void* dres_in, float* dw, float* db,
                              float* dsum, bool accumulate, const void* dy, const void* inp,
                              const float* mean,
                              const float* rstd, const float* w, int M, int C, void* scratch,
                              hipStream_t s, ColReduce* defer) {
  if (C % 8 != 0 || C > 8 * 64 * LN_MAXCH) return hipErrorInvalidValue;
  const int nb = (int)cdiv(M, LNB_ROWS);
  float* partial = (float*)scratch;
  const int nch = (int)cdiv(C / 8, 64);
  const size_t lds = 3 * C * sizeof(float);
#define LNB(NC)                                                                                \
  DISPATCH_DT(dt, layernorm_bwd_kernel<T, NC><<<nb, 256, lds, s>>>(                            \
                      (T*)dres, (const T*)(dres_in ? dres_in : dres), partial, (const T*)dy,    \
                      (const T*)inp, mean, rstd, w, M, C, accumulate ? 1 : 0))
#define LNBH(T, NC)                                                                            \
  layernorm_bwd_hw_kernel<T, NC><<<nb, 256, 0, s>>>(                                           \
      (T*)dres, (const T*)(dres_in ? dres_in : dres), partial, (const T*)dy, (const T*)inp, mean, \
      rstd, w, M, C, accumulate ? 1 : 0)
  // the half-wave kernel where its registers suffice (bf16 up to C = 768,
  // fp32 up to 512) and its 32-bit buffer ranges cover the rows
  const bool hw_ok = (int64_t)M * C * (dt == BF16 ? 2 : 4) < ((int64_t)1 << 31);
  if (!hw_ok) {
    if (nch == 1) LNB(1);
    else if (nch == 2) LNB(2);
    else if (nch == 3) LNB(3);
    else LNB(4);
  } else if (C == 256 && dt == BF16) LNBH(bf16, 1);
  else if (C == 256) LNBH(float, 1);
  else if (C == 512 && dt == BF16) LNBH(bf16, 2);
  else if (C == 512) LNBH(float, 2);
  else if (C == 768 && dt == BF16) LNBH(bf16, 3);
  else if (nch == 1) LNB(1);
  else if (nch == 2) LNB(2);
  else if (nch == 3) LNB(3);
  else LNB(4);
#undef LNB
#undef LNBH
  const ColReduce d{dw, db, dsum, partial, nb, C, 3 * C, dsum ? 3 * C : 2 * C};
  if (defer) {
    *defer = d;
    return hipGetLastError();
  }
  return column_reduce(d, s);
}

// =========================================================== bias gradient
// Workgroup: 32 column chunks of 8 (256 columns) x 8 row lanes, over a
// chunk of BG_ROWS rows; partial[rowchunk][N].
constexpr int BG_ROWS = 256;

template <class T>
__global__ __launch_bounds__(256) void bias_grad_kernel(float* __restrict__ partial,
                                                        const T* __restrict__ dy, int M, int N,
                                                        int64_t ldy) {
  __shared__ float red[8][256 + 4];
  int cc = threadIdx.x % 32, rl = threadIdx.x / 32;
  int col = blockIdx.x * 256 + cc * 8;
  int row0 = blockIdx.y * BG_ROWS;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col < N) {
    int rend = min(row0 + BG_ROWS, M);
    for (int r = row0 + rl; r < rend; r += 8) {
      float v[8];
      load8(dy + (int64_t)r * ldy + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][cc * 8 + i] = acc[i];
  __syncthreads();
  int c = threadIdx.x;  // 256 columns of this workgroup
  if (blockIdx.x * 256 + c < N) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) t += red[r][c];
    partial[(int64_t)blockIdx.y * N + blockIdx.x * 256 + c] = t;
  }
}

size_t bias_grad_scratch_bytes(int M, int N) {
  return (size_t)cdiv(M, BG_ROWS) * N * sizeof(float);
}

hipError_t bias_grad(int dt, float* db, const void* dy, int M, int N, int64_t ldy, void* scratch,
                     hipStream_t s, ColReduce* defer) {
  if (N % 8 != 0 || ldy % 8 != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)cdiv(N, 256), (unsigned)cdiv(M, BG_ROWS));
  float* partial = (float*)scratch;
  DISPATCH_DT(dt, bias_grad_kernel<T><<<grid, 256, 0, s>>>(partial, (const T*)dy, M, N, ldy));
  const ColReduce d{db, nullptr, nullptr, partial, (int)grid.y, N, N, N};
  if (defer) {
    *defer = d;
    return hipGetLastError();
  }
  return column_reduce(d, s);
}

// =========================================================== cross-entropy
// One workgroup per row: online max / sum-exp / argmax over columns < V.
struct SoftmaxState {
  float m;  // running max
  float s;  // sum of exp(z - m)
  int arg;  // lowest index attaining m
};

__device__ __forceinline__ SoftmaxState sm_combine(SoftmaxState a, SoftmaxState b) {
  SoftmaxState r;
  if (a.m > b.m || (a.m == b.m && a.arg < b.arg)) {
    r.m = a.m;
    r.arg = a.arg;
  } else {
    r.m = b.m;
    r.arg = b.arg;
  }
  float sa = a.s == 0.f ? 0.f : a.s * fast_exp(a.m - r.m);
  float sb = b.s == 0.f ? 0.f : b.s * fast_exp(b.m - r.m);
  r.s = sa + sb;
  return r;
}

template <class T>
__global__ __launch_bounds__(256) void ce_fwd_kernel(float* __restrict__ losses,
                                                     float* __restrict__ lse_out,
                                                     int32_t* __restrict__ argmax_out,
                                                     const T* __restrict__ logits, int64_t ldl,
                                                     const int32_t* __restrict__ targets, int V,
                                                     int* __restrict__ flag) {
  __shared__ SoftmaxState part[4];
  int row = blockIdx.x;
  const T* z = logits + (int64_t)row * ldl;
  SoftmaxState st = {-INFINITY, 0.f, 0x7fffffff};
  for (int c0 = threadIdx.x * 8; c0 < V; c0 += 256 * 8) {
    float v[8];
    load8(z + c0, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + i;
      if (c < V) {
        float x = v[i];
        if (x > st.m) {
          st.s = st.s * fast_exp(st.m - x) + 1.f;
          st.m = x;
          st.arg = c;
        } else {
          st.s += fast_exp(x - st.m);
        }
      }
    }
  }
  // wave reduction
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    SoftmaxState t;
    t.m = __shfl_xor(st.m, o, 64);
    t.s = __shfl_xor(st.s, o, 64);
    t.arg = __shfl_xor(st.arg, o, 64);
    st = sm_combine(st, t);
  }
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    SoftmaxState r = part[0];
    for (int w = 1; w < 4; ++w) r = sm_combine(r, part[w]);
    float lse = r.m + logf(r.s);
    int y = targets[row];
    if (y < 0 || y >= V) {
      atomicOr(flag, 2);
      y = y < 0 ? 0 : V - 1;
    }
    losses[row] = lse - to_f(z[y]);
    lse_out[row] = lse;
    argmax_out[row] = r.arg;
  }
}

hipError_t crossentropy_forward(int dt, float* losses, float* lse, int32_t* argmax,
                                const void* logits, int64_t ldl, const int32_t* targets, int M,
                                int V, int* err_flag, hipStream_t s) {
  if (ldl % 8 != 0 || ldl < V) return hipErrorInvalidValue;
  DISPATCH_DT(dt, ce_fwd_kernel<T><<<M, 256, 0, s>>>(losses, lse, argmax, (const T*)logits, ldl,
                                                     targets, V, err_flag));
  return hipGetLastError();
}

// mean of M per-row losses, one workgroup, fixed order.
__global__ __launch_bounds__(256) void mean_loss_kernel(float* __restrict__ out,
                                                        const float* __restrict__ losses, int M) {
  __shared__ double part[4];
  double acc = 0.0;
  const int M4 = M / 4;
#pragma unroll 4
  for (int i = threadIdx.x; i < M4; i += 256) {  // 16-byte loads, several in flight
    const float4 v = reinterpret_cast<const float4*>(losses)[i];
    acc += (double)v.x + (double)v.y + (double)v.z + (double)v.w;
  }
  for (int i = 4 * M4 + threadIdx.x; i < M; i += 256) acc += losses[i];
  acc = wave_sum_d(acc);
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = (float)((part[0] + part[1] + part[2] + part[3]) / M);
}

// One wave per row: the row's gemm_rowstats groups combined lane-strided,
// then by a shuffle tree (fixed order), into lse and the loss.
__global__ __launch_bounds__(256) void rowstats_loss_kernel(float* __restrict__ losses,
                                                            float* __restrict__ lse_out,
                                                            const float2* __restrict__ stats,
                                                            int64_t ld, int ncols,
                                                            const float* __restrict__ tgt,
                                                            const int32_t* __restrict__ targets,
                                                            int M, int V, int* __restrict__ flag) {
  const int lane = threadIdx.x % 64;
  const int row = blockIdx.x * 4 + threadIdx.x / 64;
  if (row >= M) return;  // wave-uniform
  auto combine = [](float& m1, float& s1, float m2, float s2) {
    const float m = fmaxf(m1, m2);
    if (m == -INFINITY) return;
    s1 = s1 * fast_exp(m1 - m) + s2 * fast_exp(m2 - m);
    m1 = m;
  };
  float m = -INFINITY, sum = 0.f;
  for (int h = lane; h < ncols; h += 64) {
    const float2 st = stats[(int64_t)row * ld + h];
    combine(m, sum, st.x, st.y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) combine(m, sum, __shfl_xor(m, o, 64), __shfl_xor(sum, o, 64));
  if (lane == 0) {
    const float lse = m + logf(sum);
    const int y = targets[row];
    if (y < 0 || y >= V) atomicOr(flag, 2);
    losses[row] = lse - tgt[row];
    lse_out[row] = lse;
  }
}

hipError_t rowstats_loss(float* losses, float* lse, const float2* stats, int64_t ld, int ncols,
                         const float* tgt, const int32_t* targets, int M, int V, int* err_flag,
                         hipStream_t s) {
  if (M <= 0) return hipSuccess;
  rowstats_loss_kernel<<<(unsigned)cdiv(M, 4), 256, 0, s>>>(losses, lse, stats, ld, ncols, tgt,
                                                             targets, M, V, err_flag);
  return hipGetLastError();
}

hipError_t mean_loss(float* out, const float* losses, int M, hipStream_t s) {
  mean_loss_kernel<<<1, 256, 0, s>>>(out, losses, M);
  return hipGetLastError();
}

// dz = seed * (exp(z - lse) - [c == y]) for c < V, 0 for V <= c < ldl
// (rows too wide for the fused kernel below).
template <class T>
__global__ void ce_bwd_kernel(T* __restrict__ dz, const T* __restrict__ logits, int64_t ldl,
                              const float* __restrict__ lse, const int32_t* __restrict__ targets,
                              int M, int V, float seed) {
  int64_t cpr = ldl / 8;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * cpr) return;
  int row = (int)(idx / cpr);
  int c0 = (int)(idx % cpr) * 8;
  const T* z = logits + (int64_t)row * ldl + c0;
  float l = lse[row];
  int y = min(max(targets[row], 0), V - 1);  // clamped as in the forward
  float v[8];
  load8(z, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int c = c0 + i;
    float p = c < V ? fast_exp(v[i] - l) : 0.f;
    if (c == y) p -= 1.f;
    v[i] = p * seed;
  }
  store8(dz + (int64_t)row * ldl + c0, v);
}

// The whole cross-entropy of a row in one workgroup of NT threads with the
// row held in registers (NCHK 8-column chunks per thread, 8 NT columns
// apart): first maximum and its column, sum of exp(z - max), then lse,
// loss = lse - z_y, and dz = seed * (exp(z - lse) - [c == y]) (0 on the
// padded columns), so the logits are read from memory once for the loss and
// the gradient together.
template <class T, int NT, int NCHK>
__global__ __launch_bounds__(NT) void ce_fused_kernel(
    float* __restrict__ losses, float* __restrict__ lse_out, int32_t* __restrict__ argmax_out,
    T* __restrict__ dz, const T* __restrict__ logits, int64_t ldl,
    const int32_t* __restrict__ targets, int V, float seed, int* __restrict__ flag) {
  constexpr int NWV = NT / 64, STEP = NT * 8;
  __shared__ SoftmaxState part[NWV];
  __shared__ float lse_s;
  const int row = blockIdx.x;
  const T* z = logits + (int64_t)row * ldl;
  // The target and its logit are read before the row, so that the serial
  // step after the reduction (one thread, the rest of the workgroup waiting
  // at the barrier) has no memory latency left in it (the kernel was waiting
  // for two dependent loads there per row).
  const int y_in = targets[row];
  const int y = y_in < 0 ? 0 : (y_in >= V ? V - 1 : y_in);  // clamped; flagged below
  const float zy = to_f(z[y]);
  Raw8<T> r[NCHK];
#pragma unroll
  for (int c = 0; c < NCHK; ++c) {
    const int c0 = threadIdx.x * 8 + c * STEP;
    if (c0 < ldl) load_raw(z + c0, r[c]);  // c0 + 7 < ldl: ldl is a multiple of 8
  }
  float m = -INFINITY;
  int arg = 0x7fffffff;
#pragma unroll
  for (int c = 0; c < NCHK; ++c) {
    const int c0 = threadIdx.x * 8 + c * STEP;
    if (c0 < V) {
      float v[8];
      unpack8(r[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c0 + i < V && v[i] > m) {  // first maximum in column order
          m = v[i];
          arg = c0 + i;
        }
    }
  }
  float sum = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int c = 0; c < NCHK; ++c) {
      const int c0 = threadIdx.x * 8 + c * STEP;
      if (c0 < V) {
        float v[8];
        unpack8(r[c], v);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c0 + i < V) sum += fast_exp(v[i] - m);
      }
    }
  }
  SoftmaxState st = {m, sum, arg};
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    SoftmaxState t;
    t.m = __shfl_xor(st.m, o, 64);
    t.s = __shfl_xor(st.s, o, 64);
    t.arg = __shfl_xor(st.arg, o, 64);
    st = sm_combine(st, t);
  }
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    SoftmaxState t = part[0];
    for (int w = 1; w < NWV; ++w) t = sm_combine(t, part[w]);
    const float lse = t.m + logf(t.s);
    if (y_in < 0 || y_in >= V) atomicOr(flag, 2);
    losses[row] = lse - zy;
    lse_out[row] = lse;
    argmax_out[row] = t.arg;
    lse_s = lse;
  }
  __syncthreads();
  const float lse = lse_s;
  T* d = dz + (int64_t)row * ldl;
#pragma unroll
  for (int c = 0; c < NCHK; ++c) {
    const int c0 = threadIdx.x * 8 + c * STEP;
    if (c0 < ldl) {
      float v[8], o[8];
      unpack8(r[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int cc = c0 + i;
        float p = cc < V ? fast_exp(v[i] - lse) : 0.f;
        if (cc == y) p -= 1.f;
        o[i] = p * seed;
      }
      store8(d + c0, o);
    }
  }
}

// threads per row for wide rows (GPT-2's 50304 columns: 13 chunks each,
// ~125 registers, two workgroups per CU)
constexpr int CE_NT = 512;

hipError_t crossentropy_fused(int dt, float* losses, float* lse, int32_t* argmax, void* dz,
                              const void* logits, int64_t ldl, const int32_t* targets, int M,
                              int V, float seed, int* err_flag, hipStream_t s) {
  if (ldl % 8 != 0 || ldl < V) return hipErrorInvalidValue;
#define CEF(T, NT, NC)                                                                         \
  ce_fused_kernel<T, NT, NC><<<M, NT, 0, s>>>(losses, lse, argmax, (T*)dz, (const T*)logits,   \
                                              ldl, targets, V, seed, err_flag)
  // chunks per thread for 256 and for CE_NT threads per row
  const int64_t nc256 = cdiv(ldl, 2048), nc = cdiv(ldl, 8 * CE_NT);
  if (nc256 <= 1) {
    if (dt == BF16) CEF(bf16, 256, 1);
    else CEF(float, 256, 1);
  } else if (nc256 <= 4) {
    if (dt == BF16) CEF(bf16, 256, 4);
    else CEF(float, 256, 4);
  } else if (dt == BF16 && nc <= 7) {
    CEF(bf16, CE_NT, 7);
  } else if (dt == BF16 && nc <= 13) {
    CEF(bf16, CE_NT, 13);  // GPT-2: 50304 columns
  } else if (dt == BF16 && nc <= 16) {
    CEF(bf16, CE_NT, 16);
  } else {  // wider rows: the loss pass, then the gradient from a second read
#undef CEF
    hipError_t e = crossentropy_forward(dt, losses, lse, argmax, logits, ldl, targets, M, V,
                                        err_flag, s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)M * (ldl / 8);
    DISPATCH_DT(dt, ce_bwd_kernel<T><<<grid_for(n, 256), 256, 0, s>>>(
                        (T*)dz, (const T*)logits, ldl, lse, targets, M, V, seed));
  }
  return hipGetLastError();
}

// =========================================================== optimizer
constexpr int NORM_BLOCKS = 1024;

struct NormScratch {
  double partial[NORM_BLOCKS];
  float result[2];  // norm, clip scale
};

size_t grad_norm_scratch_bytes() { return sizeof(NormScratch); }
const float* grad_norm_result(const void* scratch) {
  return reinterpret_cast<const NormScratch*>(scratch)->result;
}

__global__ __launch_bounds__(256) void sumsq_kernel(double* __restrict__ partial,
                                                    const float* __restrict__ g, int64_t n) {
  __shared__ double part[4];
  double acc = 0.0;
  int64_t n4 = n / 4;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 v = g4[i];
    acc += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  if (blockIdx.x == 0)
    for (int64_t i = n4 * 4 + threadIdx.x; i < n; i += 256) acc += (double)g[i] * g[i];
  acc = wave_sum_d(acc);
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

__global__ __launch_bounds__(256) void norm_finish_kernel(NormScratch* __restrict__ sc,
                                                          float clip, float* __restrict__ norm_out) {
  __shared__ double part[4];
  double acc = 0.0;
  for (int i = threadIdx.x; i < NORM_BLOCKS; i += 256) acc += sc->partial[i];
  acc = wave_sum_d(acc);
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double nrm = sqrt(part[0] + part[1] + part[2] + part[3]);
    float nf = (float)nrm;
    float scale = (nrm > (double)clip) ? (float)((double)clip / nrm) : 1.0f;
    sc->result[0] = nf;
    sc->result[1] = scale;
    if (norm_out) *norm_out = nf;
  }
}

hipError_t grad_norm(const float* g, int64_t n, float clip, void* scratch, float* norm_out,
                     hipStream_t s) {
  NormScratch* sc = (NormScratch*)scratch;
  sumsq_kernel<<<NORM_BLOCKS, 256, 0, s>>>(sc->partial, g, n);
  norm_finish_kernel<<<1, 256, 0, s>>>(sc, clip, norm_out);
  return hipGetLastError();
}

__device__ __forceinline__ bool decays(int64_t i, const DecayMap& d) {
  if (i < d.layer0) return true;  // wte, wpe
  if (i >= d.n_layer_end) return false;  // final LayerNorm
  int64_t r = (i - d.layer0) % d.layer_size;
  return (r >= d.qkvw0 && r < d.qkvw1) || (r >= d.projw0 && r < d.projw1) ||
         (r >= d.fcw0 && r < d.fcw1) || (r >= d.fcpw0 && r < d.fcpw1);
}

__device__ __forceinline__ void adamw_elem(float& p, float& m, float& v, float g, float b1, float b2,
                                           float eps, float dec, float lr, float bc1, float bc2) {
  m = b1 * m + (1.f - b1) * g;
  v = b2 * v + (1.f - b2) * g * g;
  const float mhat = m / bc1;
  const float vhat = v / bc2;
  p -= lr * (mhat / (sqrtf(vhat) + eps) + dec * p);
}

// One thread per 4 elements (tensor boundaries are multiples of C, C % 64 == 0,
// so a group of 4 never straddles two tensors), 16-byte accesses.  Skips
// everything when the norm is not finite.
__global__ __launch_bounds__(256) void adamw_kernel(
    float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, bf16* __restrict__ shadow, int64_t n, float lr, float b1, float b2,
    float eps, float wd, float bc1, float bc2, const float* __restrict__ norm_scale, DecayMap dm) {
  const float nrm = norm_scale[0];
  if (!isfinite(nrm)) return;
  const float scale = norm_scale[1];
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= n) return;
  const float dec = decays(i4, dm) ? wd : 0.f;
  if (i4 + 4 <= n) {
    float4 pp = *reinterpret_cast<const float4*>(p + i4);
    float4 gg = *reinterpret_cast<const float4*>(g + i4);
    float4 mm = *reinterpret_cast<const float4*>(m + i4);
    float4 vv = *reinterpret_cast<const float4*>(v + i4);
    adamw_elem(pp.x, mm.x, vv.x, gg.x * scale, b1, b2, eps, dec, lr, bc1, bc2);
    adamw_elem(pp.y, mm.y, vv.y, gg.y * scale, b1, b2, eps, dec, lr, bc1, bc2);
    adamw_elem(pp.z, mm.z, vv.z, gg.z * scale, b1, b2, eps, dec, lr, bc1, bc2);
    adamw_elem(pp.w, mm.w, vv.w, gg.w * scale, b1, b2, eps, dec, lr, bc1, bc2);
    *reinterpret_cast<float4*>(p + i4) = pp;
    *reinterpret_cast<float4*>(m + i4) = mm;
    *reinterpret_cast<float4*>(v + i4) = vv;
    if (shadow) {
      union {
        uint2 u;
        bf16 e[4];
      } w;
      w.e[0] = (bf16)pp.x; w.e[1] = (bf16)pp.y; w.e[2] = (bf16)pp.z; w.e[3] = (bf16)pp.w;
      *reinterpret_cast<uint2*>(shadow + i4) = w.u;
    }
  } else {
    for (int64_t i = i4; i < n; ++i) {
      float pi = p[i], mi = m[i], vi = v[i];
      adamw_elem(pi, mi, vi, g[i] * scale, b1, b2, eps, dec, lr, bc1, bc2);
      p[i] = pi;
      m[i] = mi;
      v[i] = vi;
      if (shadow) shadow[i] = (bf16)pi;
    }
  }
}

hipError_t adamw(float* p, const float* g, float* m, float* v, void* shadow, int64_t n, float lr,
                 float b1, float b2, float eps, float wd, float bc1, float bc2,
                 const float* norm_scale, DecayMap dm, hipStream_t s) {
  int64_t threads = cdiv(n, 4);
  adamw_kernel<<<grid_for(threads, 256), 256, 0, s>>>(p, g, m, v, (bf16*)shadow, n, lr, b1, b2,
                                                      eps, wd, bc1, bc2, norm_scale, dm);
  return hipGetLastError();
}

// =========================================================== fills / casts
__global__ void fill_f32_kernel(float* __restrict__ p, float value, int64_t n) {
  const int64_t n4 = n / 4;
  const float4 v4 = make_float4(value, value, value, value);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4*>(p)[i] = v4;
  if (blockIdx.x == 0)
    for (int64_t i = n4 * 4 + threadIdx.x; i < n; i += blockDim.x) p[i] = value;
}
__global__ void fill_i32_kernel(int32_t* __restrict__ p, int32_t value, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}
__global__ void cast_bf16_kernel(bf16* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (bf16)src[i];
}

static inline int stride_grid(int64_t n) {
  int64_t g = cdiv(n, 256);
  return (int)(g < 8192 ? g : 8192);
}

hipError_t fill_f32(float* p, float value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_f32_kernel<<<stride_grid(n), 256, 0, s>>>(p, value, n);
  return hipGetLastError();
}
hipError_t fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<stride_grid(n), 256, 0, s>>>(p, value, n);
  return hipGetLastError();
}
hipError_t cast_f32_to_bf16(void* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  cast_bf16_kernel<<<stride_grid(n), 256, 0, s>>>((bf16*)dst, src, n);
  return hipGetLastError();
}

}  // namespace gk
