// Matrix-core flash attention for bf16, head size 64, on gfx950
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation and softmax).
//
// Causal self-attention per (batch, head): S = q k^T / sqrt(64), j <= i,
// P = softmax_j(S), O = P v; the forward also stores the log-sum-exp L of
// each query row.  The T x T matrix is never stored: 64-key (or 64-query)
// tiles are staged through LDS and the softmax is computed online.
//
// Register layout.  A wave owns 32 queries (forward, dQ) or 32 keys (dK/dV).
// Scores are produced transposed where that keeps a lane on one query:
// S^T = K Q^T gives each lane one query column and 16 key rows of a 32 x 32
// tile (accumulator row = 8*(r/4) + 4*(lane/32) + r%4), so the row maximum
// needs one exchange with lane^32 and the probabilities are already laid
// out as the B operand of the next product O^T += V^T P^T: lane half h of
// slot j holds key 4h + j (j < 4) or 8 + 4h + j - 4 (j >= 4) of each
// 16-key step.
//
// LDS tiles are always stored as they sit in memory, [row][d] (16-byte
// copies).  Operands that need the transposed tile (V^T, K^T, Q^T, dO^T)
// are read with ds_read_b64_tr_b16: within each 16-lane group, lane j gets
// element j%4 of the 8-byte rows addressed by lanes j/4 + 4e (e = 0..3), so
// pointing lane i' at row kbase + i'/4, column c0 + 4 (i'%4) hands lane j
// rows kbase .. kbase+3 of column c0 + j -- four k-values of one MFMA
// operand row, in the permuted key order above.
//
// Backward (no atomics):
//   dQ pass, per query block: D_i = dO_i . O_i (stored for the next pass),
//     S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
//   dK/dV pass, per key block: S = Q K^T, dP = dO V^T (lane owns a key
//     column), P = exp(S - L), dS = P (dP - D), dV^T += dO^T P,
//     dK^T += Q^T dS.
// LDS is double-buffered (one barrier per tile) with the next tile's global
// loads (buffer loads whose range check zero-fills rows past T) in flight
// during the current tile's math; the causal mask is compiled only into the
// tiles that straddle the diagonal.  Workgroups of the causal passes are
// issued longest-first.  Optionally each backward workgroup also sums the
// columns of the dq / dk / dv rows it stores (the qkv bias gradient's first
// stage).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

namespace {

constexpr int HD = 64;    // head size
constexpr int WQ = 128;   // queries (or keys) per workgroup: 4 waves x 32
constexpr int TB = 64;    // keys (or queries) per LDS tile
constexpr int PR = 72;    // LDS pitch of [row][d] tiles (elements; 144 B, 16 B aligned)
constexpr int TILE = TB * PR;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Row of the accumulator held in register r by lane half h2.
__device__ __forceinline__ int acc_row(int r, int h2) { return 8 * (r / 4) + 4 * h2 + (r % 4); }

// 64 rows x 64 columns of bf16 from global (row stride ld), rows >= nrows
// read as zero: two 16-byte chunks per thread, through a buffer resource
// that starts at the tile's first row and ends with row nrows - 1, so the
// hardware range check supplies the zeros (no per-load branch).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer (stride 0), 32-bit data format
struct TileRegs {
  uint4 v[2];
};
__device__ __forceinline__ void tile_load(TileRegs& R, const bf16* __restrict__ src, int64_t ld,
                                          int row0, int nrows) {
  const int rem = nrows - row0;
  const int bytes = rem > 0 ? (int)(((int64_t)(rem - 1) * ld + HD) * 2) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(src + (int64_t)row0 * ld), (short)0, bytes, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / 8, d = (c % 8) * 8;
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins exist only for the GPU target
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)((row * ld + d) * 2), 0, 0);
    R.v[i] = make_uint4(w.x, w.y, w.z, w.w);
#else
    (void)rs;
    (void)row;
    (void)d;
    R.v[i] = make_uint4(0, 0, 0, 0);
#endif
  }
}
__device__ __forceinline__ void tile_store(const TileRegs& R, bf16* __restrict__ S) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int c = threadIdx.x + 256 * i;
    int row = c / 8, d = (c % 8) * 8;
    *reinterpret_cast<uint4*>(S + row * PR + d) = R.v[i];
  }
}

// Fragment from a row-major tile: row `row`, k = ks*16 + h2*8 .. +8.
__device__ __forceinline__ bf16x8_t frag_rows(const bf16* S, int row, int ks, int h2) {
  return *reinterpret_cast<const bf16x8_t*>(S + row * PR + ks * 16 + h2 * 8);
}

__device__ __forceinline__ v4i16 ds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

// Transposed fragment: lane l gets column c0 + l%32 of the tile at rows
// kb + 4*h2 .. +4 and kb + 8 + 4*h2 .. +4 (the accumulator key order).
__device__ __forceinline__ bf16x8_t frag_tr(const bf16* S, int c0, int kb, int lane) {
  const int j = lane % 16, h2 = lane / 32;
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const v4i16 lo = ds_read_tr(S + (kb + 4 * h2 + (j >> 2)) * PR + col);
  const v4i16 hi = ds_read_tr(S + (kb + 8 + 4 * h2 + (j >> 2)) * PR + col);
  union {
    v4i16 s[2];
    bf16x8_t v;
  } r;
  r.s[0] = lo;
  r.s[1] = hi;
  return r.v;
}

// Registers 8u .. 8u+7 of an accumulator as a bf16 B operand.
__device__ __forceinline__ bf16x8_t pack_b(const f32x16_t& a, int u) {
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)a[8 * u + j];
  return r;
}
// Global fragment of one row: 8 consecutive bf16 at d = ks*16 + h2*8.
__device__ __forceinline__ bf16x8_t frag_global(const bf16* __restrict__ row_ptr, int ks, int h2,
                                                bool valid) {
  union {
    uint4 u;
    bf16x8_t v;
  } r;
  r.u = valid ? *reinterpret_cast<const uint4*>(row_ptr + ks * 16 + h2 * 8) : make_uint4(0, 0, 0, 0);
  return r.v;
}

// Stores a wave's 32 rows x 64 columns of the two transposed accumulators
// a[0], a[1] (lane: row lane % 32, columns dt*32 + acc_row(r, lane / 32)),
// each value times mul and rounded to bf16, row by row: the rounded values
// go into the wave's own LDS region S (32 rows, pitch SPS) and come back as
// 16 bytes per lane, eight lanes per 128-byte row segment, so that a store
// instruction covers eight whole row segments, not 16 bytes of each of 32
// rows (attention forward 4 % faster, backward 2-4 %).  dst0: the wave's first row; rows [0, rows_valid) are stored.
// Call once the LDS tiles are free (after the last tile's barrier).
constexpr int SPS = HD + 8;  // 144-byte rows
__device__ __forceinline__ void store_rows_staged(bf16* __restrict__ dst0, int64_t ld,
                                                  int rows_valid, const f32x16_t (&a)[2],
                                                  float mul, bf16* S, int lane) {
  const int l32 = lane % 32, h2 = lane / 32;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      union {
        uint2 u;
        bf16 e[4];
      } w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w.e[j] = (bf16)(a[dt][4 * g + j] * mul);
      *reinterpret_cast<uint2*>(S + l32 * SPS + dt * 32 + 8 * g + 4 * h2) = w.u;
    }
  __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in issue order
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 8 * k + lane / 8, c = (lane % 8) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(S + r * SPS + c);
    if (r < rows_valid) *reinterpret_cast<uint4*>(dst0 + (int64_t)r * ld + c) = v;
  }
  __builtin_amdgcn_wave_barrier();
}

// Column sums of a workgroup's 128 stored rows x 64 columns (the first stage
// of the qkv bias gradient): each lane puts its row's 32 values of `a` (as
// stored: bf16 of a * mul, 0 for an invalid row) into LDS, then lane c of
// the first wave adds column c over the 128 rows in order.  Call after the
// workgroup's last barrier-ended tile (the staging LDS is free), by all
// threads.
__device__ __forceinline__ void colsum_rows128(float* __restrict__ dst, const f32x16_t (&a)[2],
                                               float mul, bool valid, bf16* smem, int wave,
                                               int l32, int h2) {
  constexpr int P = HD + 1;  // row pitch (floats)
  static_assert(128 * P * 4 <= 4 * TILE * 2, "column-sum staging exceeds the LDS tiles");
  static_assert(4 * 2 * 32 * SPS <= 4 * TILE, "row staging exceeds the LDS tiles");
  float* red = reinterpret_cast<float*>(smem);
  const int row = wave * 32 + l32;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      red[row * P + dt * 32 + acc_row(r, h2)] = valid ? (float)(bf16)(a[dt][r] * mul) : 0.f;
  __syncthreads();
  if (threadIdx.x < HD) {
    float t = 0.f;
    for (int i = 0; i < 128; ++i) t += red[i * P + threadIdx.x];
    dst[threadIdx.x] = t;
  }
  __syncthreads();
}

// Workgroup -> (batch x head, rank), rank 0 being the head's longest causal
// block.  Each XCD gets a contiguous range of logical workgroups
// (xcd_remap).  Where that range is whole heads (B*H a multiple of 8), the
// XCD runs its blocks longest-first across all of its heads, so that the
// short blocks fill the slots the long ones leave at the end (a workgroup
// slot then takes about the average work instead of up to one and a half
// times it); otherwise head by head, longest first.  The blocks of a head
// stay on one XCD and share its L2 either way.
__device__ __forceinline__ void causal_block(int bid, int nblocks, int nper, int& bh, int& rank) {
  const int pid = xcd_remap(bid, nblocks);
  const int nbh = nblocks / nper;
  if (nbh % 8 == 0) {
    const int hx = nbh / 8;  // heads per XCD
    const int xcd = pid / (hx * nper), p = pid % (hx * nper);
    bh = xcd * hx + p % hx;
    rank = p / hx;
  } else {
    bh = pid / nper;
    rank = pid % nper;
  }
}

// --------------------------------------------------------------- forward
// Online softmax with a lazily moved reference: each query keeps a running
// reference m (log2 units) and accumulates l = sum exp2(s c - m) and
// O = sum exp2(s c - m) v.  A tile's probabilities are first taken against
// the current m; only when a query's sum over the tile exceeds 64 * 2^8 (or
// is not finite: the first tile, m = -inf) is the tile's maximum computed,
// m raised to it if it exceeds m by more than 8, O and l rescaled and the
// probabilities recomputed.  So every probability stays below 2^14 (no fp32
// overflow), most tiles need neither the maximum nor a rescale, and since l
// and O always share the same m, O / l and the log-sum-exp m + log2 l are
// exact.
constexpr float RESCALE_LOG2 = 8.0f;

// The forward and dQ kernels fit in 168 registers: three workgroups (12
// waves) per CU.  The dK/dV kernel needs more and runs two.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_fwd_mfma(
    bf16* __restrict__ out, float* __restrict__ lse, const bf16* __restrict__ qkv, int T, int H,
    int nqb) {
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * TILE];  // [stage][K | V]
  const int lane = threadIdx.x % 64, h2 = lane / 32, l32 = lane % 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform per wave
  // longest query block first (causal_block)
  int bh, rank;
  causal_block(blockIdx.x, gridDim.x, nqb, bh, rank);
  const int qb = nqb - 1 - rank;
  const int b = bh / H, hh = bh % H;
  const int C = H * HD;
  const int64_t ld = 3LL * C;
  const bf16* base = qkv + (int64_t)b * T * ld;
  const bf16* kbase = base + C + hh * HD;
  const bf16* vbase = base + 2 * C + hh * HD;
  const int q0 = qb * WQ, qw = q0 + wave * 32, myq = qw + l32;
  const float c = 0.125f * LOG2E;  // 1/sqrt(64) in log2 units

  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = frag_global(base + (int64_t)myq * ld + hh * HD, ks, h2, myq < T);
  f32x16_t o[2] = {zero16(), zero16()};
  float m = -INFINITY, l = 0.f;
  const int nkb = (int)min(cdiv(q0 + WQ, TB), cdiv(T, TB));
  TileRegs rk, rv;
  tile_load(rk, kbase, ld, 0, T);
  tile_load(rv, vbase, ld, 0, T);
  tile_store(rk, smem);
  tile_store(rv, smem + TILE);
  if (nkb > 1) {
    tile_load(rk, kbase, ld, TB, T);
    tile_load(rv, vbase, ld, TB, T);
  }
  __syncthreads();
  // One 64-key tile for this wave's 32 queries.
  auto tile = [&](const bf16* Ks, const bf16* Vs, int k0, bool diag) {
    f32x16_t s[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[t] = mfma(frag_rows(Ks, t * 32 + l32, ks, h2), qf[ks], s[t]);
    if (diag) {  // wave-uniform: only the tiles that reach past the first query
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (k0 + t * 32 + acc_row(r, h2) > myq) s[t][r] = -INFINITY;
    }
    // Probabilities against the current reference m first; the tile's
    // maximum is needed only when some probability is too large (a score
    // more than 2^RESCALE_LOG2 above the reference: the partial sums show
    // it, and an infinite m - score or a first tile gives inf or NaN there).
    float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
    float pe[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pe[t][r] = exp2_(__builtin_fmaf(s[t][r], c, -m));
        ps[r % 4] += pe[t][r];
      }
    float tsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // !(x <= bound) is also true for NaN
    if (__builtin_amdgcn_ballot_w64(!(tsum <= 64.0f * (1 << (int)RESCALE_LOG2)))) {
      // row maximum as a tree (short dependency chains)
      float m8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        m8[i] = fmaxf(fmaxf(s[i / 4][4 * (i % 4)], s[i / 4][4 * (i % 4) + 1]),
                      fmaxf(s[i / 4][4 * (i % 4) + 2], s[i / 4][4 * (i % 4) + 3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) m8[i] = fmaxf(m8[i], m8[i + 4]);
      float mx = fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
      // move the reference only when this tile exceeds it by more than 2^8
      const bool move = mx > m + RESCALE_LOG2;
      const float mnew = move ? mx : m;
      const float alpha = exp2_(m - mnew);
      m = mnew;
      l *= alpha;
      o[0] *= alpha;
      o[1] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[i] = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pe[t][r] = exp2_(__builtin_fmaf(s[t][r], c, -m));
          ps[r % 4] += pe[t][r];
        }
      tsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = pe[t][r];
    l += tsum;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t pb = pack_b(s[t], u);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          o[dt] = mfma(frag_tr(Vs, dt * 32, t * 32 + 16 * u, lane), pb, o[dt]);
      }
  };
  // stage tile kb+1 into LDS and start loading tile kb+2
  auto advance = [&](int kb) {
    if (kb + 1 < nkb) {
      bf16* nxt = smem + ((kb + 1) & 1) * 2 * TILE;
      tile_store(rk, nxt);
      tile_store(rv, nxt + TILE);
      if (kb + 2 < nkb) {
        tile_load(rk, kbase, ld, (kb + 2) * TB, T);
        tile_load(rv, vbase, ld, (kb + 2) * TB, T);
      }
    }
  };
  // Tiles every wave of the block needs (those up to the first wave's last
  // query) run unconditionally, which keeps the accumulators in place; only
  // the block's last tile can be needed by some waves and not others.
  const int nall = min(nkb, (q0 + 31) / TB + 1);
  int kb = 0;
  for (; kb < nall; ++kb) {
    const bf16* Ks = smem + (kb & 1) * 2 * TILE;
    advance(kb);
    tile(Ks, Ks + TILE, kb * TB, kb * TB + TB - 1 > qw);
    __syncthreads();
  }
  for (; kb < nkb; ++kb) {
    const bf16* Ks = smem + (kb & 1) * 2 * TILE;
    advance(kb);
    if (kb * TB <= qw + 31) tile(Ks, Ks + TILE, kb * TB, true);
    __syncthreads();
  }
  l += __shfl_xor(l, 32, 64);
  store_rows_staged(out + ((int64_t)b * T + qw) * C + hh * HD, C, T - qw, o, 1.0f / l,
                    smem + wave * 32 * SPS, lane);
  if (myq < T && h2 == 0) lse[(int64_t)bh * T + myq] = (m + __builtin_amdgcn_logf(l)) * LN2;
}

// --------------------------------------------------------------- backward: dQ
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_bwd_dq_mfma(bf16* __restrict__ dqkv, float* __restrict__ Dbuf,
                                                        const bf16* __restrict__ dout,
                                                        const bf16* __restrict__ qkv,
                                                        const bf16* __restrict__ out,
                                                        const float* __restrict__ lse, int T, int H,
                                                        int nqb, float* __restrict__ colsum) {
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * TILE];  // [stage][K | V]
  const int lane = threadIdx.x % 64, h2 = lane / 32, l32 = lane % 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform per wave
  // longest query block first (causal_block)
  int bh, rank;
  causal_block(blockIdx.x, gridDim.x, nqb, bh, rank);
  const int qb = nqb - 1 - rank;
  const int b = bh / H, hh = bh % H;
  const int C = H * HD;
  const int64_t ld = 3LL * C;
  const bf16* base = qkv + (int64_t)b * T * ld;
  const bf16* kbase = base + C + hh * HD;
  const bf16* vbase = base + 2 * C + hh * HD;
  const int q0 = qb * WQ, qw = q0 + wave * 32, myq = qw + l32;
  const bool qvalid = myq < T;
  const float c = 0.125f * LOG2E;

  bf16x8_t qf[4], df[4];
  // Start-up loads without branches (a row past T is read from row T-1 and
  // zeroed), with the log-sum-exp and the first K and V tiles issued before
  // anything waits, so that one memory latency covers them all (inside
  // branches the compiler waited after each group).
  const int myqc = min(myq, T - 1);
  const bf16* dorow = dout + ((int64_t)b * T + myqc) * C + hh * HD;
  const bf16* orow = out + ((int64_t)b * T + myqc) * C + hh * HD;
  const bf16* qrow = base + (int64_t)myqc * ld + hh * HD;
  bf16x8_t of[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16 + h2 * 8);
    df[ks] = *reinterpret_cast<const bf16x8_t*>(dorow + ks * 16 + h2 * 8);
    of[ks] = *reinterpret_cast<const bf16x8_t*>(orow + ks * 16 + h2 * 8);
  }
  const float lsraw = lse[(int64_t)bh * T + myqc];
  const int nkb = (int)min(cdiv(q0 + WQ, TB), cdiv(T, TB));
  TileRegs rk, rv;
  tile_load(rk, kbase, ld, 0, T);
  tile_load(rv, vbase, ld, 0, T);
  float Dp = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (!qvalid) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[ks][j] = df[ks][j] = (bf16)0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) Dp += (float)df[ks][j] * (float)of[ks][j];
  }
  const float Dq = Dp + __shfl_xor(Dp, 32, 64);
  const float L2 = qvalid ? lsraw * LOG2E : 0.f;
  if (qvalid && h2 == 0) Dbuf[(int64_t)bh * T + myq] = Dq;
  f32x16_t dq[2] = {zero16(), zero16()};
  tile_store(rk, smem);
  tile_store(rv, smem + TILE);
  if (nkb > 1) {
    tile_load(rk, kbase, ld, TB, T);
    tile_load(rv, vbase, ld, TB, T);
  }
  __syncthreads();
  // One 64-key tile for this wave's 32 queries; DIAG (a compile-time
  // constant, so that the other tiles carry no masking code) on the tiles
  // that reach past the wave's first query.
  auto dq_tile = [&](auto diag_c, const bf16* Ks, const bf16* Vs, int k0) {
    constexpr bool diag = decltype(diag_c)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16_t s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = mfma(frag_rows(Ks, t * 32 + l32, ks, h2), qf[ks], s);
        dp = mfma(frag_rows(Vs, t * 32 + l32, ks, h2), df[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = exp2_(__builtin_fmaf(s[r], c, -L2));
        if constexpr (diag) {
          if (k0 + t * 32 + acc_row(r, h2) > myq) p = 0.f;
        }
        s[r] = p * (dp[r] - Dq);  // dS^T
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t sb = pack_b(s, u);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          dq[dt] = mfma(frag_tr(Ks, dt * 32, t * 32 + 16 * u, lane), sb, dq[dt]);
      }
    }
  };
  auto advance = [&](int kb) {
    if (kb + 1 < nkb) {
      bf16* nxt = smem + ((kb + 1) & 1) * 2 * TILE;
      tile_store(rk, nxt);
      tile_store(rv, nxt + TILE);
      if (kb + 2 < nkb) {
        tile_load(rk, kbase, ld, (kb + 2) * TB, T);
        tile_load(rv, vbase, ld, (kb + 2) * TB, T);
      }
    }
  };
  // Tiles wholly at or before every query of the block need no mask; then,
  // as in the forward, the tiles every wave needs run unconditionally, and
  // the block's last one only for the waves that reach it.
  const int nfree = min(nkb, (q0 + 1) / TB);
  const int nall = min(nkb, (q0 + 31) / TB + 1);
  int kb = 0;
  for (; kb < nfree; ++kb) {
    const bf16* Ks = smem + (kb & 1) * 2 * TILE;
    advance(kb);
    dq_tile(std::false_type{}, Ks, Ks + TILE, kb * TB);
    __syncthreads();
  }
  for (; kb < nall; ++kb) {
    const bf16* Ks = smem + (kb & 1) * 2 * TILE;
    advance(kb);
    dq_tile(std::true_type{}, Ks, Ks + TILE, kb * TB);
    __syncthreads();
  }
  for (; kb < nkb; ++kb) {
    const bf16* Ks = smem + (kb & 1) * 2 * TILE;
    advance(kb);
    if (kb * TB <= qw + 31) dq_tile(std::true_type{}, Ks, Ks + TILE, kb * TB);
    __syncthreads();
  }
  store_rows_staged(dqkv + ((int64_t)b * T + qw) * ld + hh * HD, ld, T - qw, dq, 0.125f,
                    smem + wave * 32 * SPS, lane);
  if (colsum) {
    __syncthreads();  // the column sums reuse every wave's region
    colsum_rows128(colsum + (int64_t)(b * nqb + qb) * ld + hh * HD, dq, 0.125f, qvalid, smem, wave,
                   l32, h2);
  }
}

// --------------------------------------------------------------- backward: dK, dV
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkv_mfma(bf16* __restrict__ dqkv,
                                                         const float* __restrict__ Dbuf,
                                                         const bf16* __restrict__ dout,
                                                         const bf16* __restrict__ qkv,
                                                         const float* __restrict__ lse, int T, int H,
                                                         float* __restrict__ colsum) {
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * TILE];  // [stage][Q | dO]
  __shared__ __attribute__((aligned(16))) float LD[2][2][TB];   // [stage][L | D]
  const int lane = threadIdx.x % 64, h2 = lane / 32, l32 = lane % 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform per wave
  // longest key block (the first) first (causal_block)
  const int nkb_total = (int)cdiv(T, WQ);
  int bh, kblk;
  causal_block(blockIdx.x, gridDim.x, nkb_total, bh, kblk);
  const int b = bh / H, hh = bh % H;
  const int C = H * HD;
  const int64_t ld = 3LL * C;
  const bf16* base = qkv + (int64_t)b * T * ld;
  const bf16* qbase = base + hh * HD;
  const bf16* dobase = dout + (int64_t)b * T * C + hh * HD;
  const int k0w = kblk * WQ, kw = k0w + wave * 32, mykey = kw + l32;
  const bool kvalid = mykey < T;
  const float c = 0.125f * LOG2E;

  bf16x8_t kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = frag_global(base + (int64_t)mykey * ld + C + hh * HD, ks, h2, kvalid);
    vf[ks] = frag_global(base + (int64_t)mykey * ld + 2 * C + hh * HD, ks, h2, kvalid);
  }
  f32x16_t dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};
  const int qb0 = k0w / TB, nqb = (int)cdiv(T, TB);
  TileRegs rq, rd;
  float lsv = 0.f, dsv = 0.f;
  int lqb = 0;  // the query tile lsv and dsv belong to
  auto gload = [&](int qb) {
    tile_load(rq, qbase, ld, qb * TB, T);
    tile_load(rd, dobase, C, qb * TB, T);
    // every thread loads (from a clamped index; the first TB store them):
    // loads inside a branch made the compiler wait for them, and with them
    // for the tile loads just issued, right away
    {
      const int qc = min(qb * TB + (int)(threadIdx.x % TB), T - 1);
      lsv = lse[(int64_t)bh * T + qc];  // raw: sstore applies q < T and the scale,
      dsv = Dbuf[(int64_t)bh * T + qc];  // so that nothing waits for them before
      lqb = qb;
    }
  };
  auto sstore = [&](int stage) {
    bf16* dst = smem + stage * 2 * TILE;
    tile_store(rq, dst);
    tile_store(rd, dst + TILE);
    if (threadIdx.x < TB) {
      const bool in = lqb * TB + (int)threadIdx.x < T;
      LD[stage][0][threadIdx.x] = in ? lsv * LOG2E : INFINITY;
      LD[stage][1][threadIdx.x] = in ? dsv : 0.f;
    }
  };
  // One 64-query tile for this wave's 32 keys; DIAG (compile-time) on the
  // tiles whose first queries precede some of the wave's keys.
  auto dkv_tile = [&](auto diag_c, const bf16* Qs, const bf16* Os, const float* Ls,
                      const float* Ds, int qs0) {
    constexpr bool diag = decltype(diag_c)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16_t s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = mfma(frag_rows(Qs, t * 32 + l32, ks, h2), kf[ks], s);
        dp = mfma(frag_rows(Os, t * 32 + l32, ks, h2), vf[ks], dp);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rowb = t * 32 + 8 * g + 4 * h2;  // query rows rowb .. rowb+3 of the tile
        const float4 L4 = *reinterpret_cast<const float4*>(Ls + rowb);
        const float4 D4 = *reinterpret_cast<const float4*>(Ds + rowb);
        const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          float p = exp2_(__builtin_fmaf(s[r], c, -Lv[j]));
          if constexpr (diag) {
            if (qs0 + rowb + j < mykey) p = 0.f;
          }
          s[r] = p;
          dp[r] = p * (dp[r] - Dv[j]);  // dS
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t pb = pack_b(s, u);
        bf16x8_t sb = pack_b(dp, u);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dv[dt] = mfma(frag_tr(Os, dt * 32, t * 32 + 16 * u, lane), pb, dv[dt]);
          dk[dt] = mfma(frag_tr(Qs, dt * 32, t * 32 + 16 * u, lane), sb, dk[dt]);
        }
      }
    }
  };
  gload(qb0);
  sstore(0);
  if (qb0 + 1 < nqb) gload(qb0 + 1);
  __syncthreads();
  // iteration qb: stage tile qb+1, load qb+2, multiply tile qb.  Only the
  // first query tile (it starts at the block's first key) can be skipped by
  // some waves; the rest run unconditionally, keeping the accumulators in
  // place.  The first two tiles may hold queries before some of the block's
  // keys and carry the mask; from the third on no query precedes a key.
  auto step = [&](auto diag_c, int qb, bool need) {
    const int stage = (qb - qb0) & 1;
    const bf16* Qs = smem + stage * 2 * TILE;
    if (qb + 1 < nqb) {
      sstore(stage ^ 1);
      if (qb + 2 < nqb) gload(qb + 2);
    }
    if (need) dkv_tile(diag_c, Qs, Qs + TILE, LD[stage][0], LD[stage][1], qb * TB);
    __syncthreads();
  };
  static_assert(WQ == 2 * TB, "two masked query tiles per key block");
  if (qb0 < nqb) step(std::true_type{}, qb0, qb0 * TB + TB - 1 >= kw);
  if (qb0 + 1 < nqb) step(std::true_type{}, qb0 + 1, true);
  for (int qb = qb0 + 2; qb < nqb; ++qb) step(std::false_type{}, qb, true);
  {
    bf16* dst0 = dqkv + ((int64_t)b * T + kw) * ld + hh * HD;
    bf16* S = smem + wave * 2 * 32 * SPS;
    store_rows_staged(dst0 + C, ld, T - kw, dk, 0.125f, S, lane);
    store_rows_staged(dst0 + 2 * C, ld, T - kw, dv, 1.0f, S + 32 * SPS, lane);
  }
  if (colsum) {
    __syncthreads();  // the column sums reuse every wave's region
    float* cs = colsum + (int64_t)(b * nkb_total + kblk) * ld + hh * HD;
    colsum_rows128(cs + C, dk, 0.125f, kvalid, smem, wave, l32, h2);
    colsum_rows128(cs + 2 * C, dv, 1.0f, kvalid, smem, wave, l32, h2);
  }
}

}  // namespace

bool attention_mfma_supported(int dt, int hd) { return dt == BF16 && hd == HD; }

hipError_t attention_forward_mfma(void* out, float* lse, const void* qkv, int B, int T, int H,
                                  hipStream_t s) {
  const int nqb = (int)cdiv(T, WQ);
  dim3 grid((unsigned)(nqb * B * H));
  attn_fwd_mfma<<<grid, 256, 0, s>>>((bf16*)out, lse, (const bf16*)qkv, T, H, nqb);
  return hipGetLastError();
}

hipError_t attention_backward_mfma(void* dqkv, const void* dout, const void* qkv, const void* out,
                                   const float* lse, float* Dbuf, int B, int T, int H,
                                   hipStream_t s, float* colsum) {
  const int nb = (int)cdiv(T, WQ);
  static_assert(WQ == 128, "column-sum blocks are the workgroups' 128 rows");
  dim3 grid((unsigned)(nb * B * H));
  attn_bwd_dq_mfma<<<grid, 256, 0, s>>>((bf16*)dqkv, Dbuf, (const bf16*)dout, (const bf16*)qkv,
                                        (const bf16*)out, lse, T, H, nb, colsum);
  attn_bwd_dkv_mfma<<<grid, 256, 0, s>>>((bf16*)dqkv, Dbuf, (const bf16*)dout, (const bf16*)qkv,
                                         lse, T, H, colsum);
  return hipGetLastError();
}

}  // namespace gk
