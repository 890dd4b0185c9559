// Shared device helpers for the gfx950 kernels: element types, 16-byte
// packs, wave64 reductions, fast transcendentals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;

#define GPT2_WAVE 64

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }  // RNE

// ---------------------------------------------------------------- 16-byte packs
// One 16-byte vector of T: 4 floats or 8 bf16.
template <class T> struct Pack {
  static constexpr int N = 16 / sizeof(T);
  union {
    uint4 u;
    T e[N];
  };
};

template <class T> __device__ __forceinline__ Pack<T> load_pack(const T* p) {
  Pack<T> r;
  r.u = *reinterpret_cast<const uint4*>(p);
  return r;
}
template <class T> __device__ __forceinline__ void store_pack(T* p, const Pack<T>& v) {
  *reinterpret_cast<uint4*>(p) = v.u;
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------- math
// exp(x) via the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// tanh(u) = 1 - 2 / (exp(2u) + 1); saturates correctly at +-inf.  The
// hardware reciprocal (1 ulp) replaces the IEEE divide.
__device__ __forceinline__ float tanh_from_exp(float u) {
  float e = __builtin_amdgcn_exp2f(u * 2.8853900817779268f);  // exp(2u)
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// GELU, tanh form: 0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h + 0.044715 h^3).
// With s = 1 / (1 + exp(-2u)) = (1 + tanh(u)) / 2 this is h s.
// h^2 is formed once, so that the derivative below can reuse it.
__device__ __forceinline__ float gelu_sigmoid(float h) {
  const float k2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float u2 = k2 * h * __builtin_fmaf(0.044715f, h * h, 1.0f);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u2));
}
__device__ __forceinline__ float gelu_f(float h) { return h * gelu_sigmoid(h); }
// d gelu / d h = 0.5 (1 + t) + 0.5 h (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 h^2)
//             = s + h s (1 - s) k (1 + 0.134145 h^2),  k = 2 sqrt(2/pi).
// gelu_grad_s takes s = gelu_sigmoid(h) already computed: four operations
// (s (1 - s) as one fused multiply-add, h^2 shared with the sigmoid), as the
// fc product's epilogue evaluates it for every element while the matrix
// cores wait.
__device__ __forceinline__ float gelu_grad_s(float h, float s) {
  const float k = 2.0f * 0.7978845608028654f;
  const float q = __builtin_fmaf(k * 3.0f * 0.044715f, h * h, k);  // k (1 + 0.134145 h^2)
  return __builtin_fmaf(__builtin_fmaf(-s, s, s) * q, h, s);
}
__device__ __forceinline__ float gelu_grad_f(float h) { return gelu_grad_s(h, gelu_sigmoid(h)); }

// Workgroups are dealt to the 8 XCDs of the chip round-robin by id, and each
// XCD has its own L2.  xcd_remap turns the hardware id into a logical index
// such that every XCD receives one contiguous range of logical indices (the
// first nblocks % 8 XCDs one more than the others), so that neighbouring
// logical workgroups share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int NX = 8;
  const int xcd = bid % NX, local = bid / NX;
  const int per = (nblocks + NX - 1) / NX;
  const int tall = nblocks % NX;
  if (tall == 0 || xcd < tall) return xcd * per + local;
  return tall * per + (xcd - tall) * (per - 1) + local;
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
