// Token-embedding backward without floating-point atomics: dwte[v] += sum of
// dx[m] over the positions m with tok[m] = v, each token's rows added in
// position order (bitwise repeatable).
//
// 1. hist:    per chunk of 512 positions, how often each token occurs, and
//             each position's rank among the earlier equal tokens of its
//             chunk.
// 2. offsets: per token, the exclusive prefix of its counts over the chunks
//             and its total, and per block of 256 tokens the exclusive scan
//             of the totals; one workgroup then scans the block sums.  Token
//             v's positions occupy slots start(v) .. start(v) + total(v) - 1
//             of the sorted order, in position order.
// 3. place:   every position writes itself into its slot.
// 4. window:  one wave per 32 consecutive slots walks them in order and sums
//             the rows of each run of equal tokens.  A run that lies wholly
//             inside the window is added to its dwte row directly (no other
//             wave touches that token); a run that crosses a window edge
//             leaves its partial sum in the window's two partial slots
//             (0: the run continued from the previous window, 1: the run
//             that continues into the next).
// 5. combine: for every run that starts in a window and crosses its end,
//             one wave adds the partials of the windows the token's segment
//             covers, in window order, to the token's dwte row.
#include "common.h"
#include "kernels.h"

namespace gk {

namespace {

constexpr int EB_CHUNK = 512;   // positions per histogram chunk (one workgroup)
constexpr int EB_SB = 256;      // tokens per scan block
constexpr int EB_WIN = 32;      // slots per window (one wave; small, so that many waves run)
constexpr int EB_MAXCH = 4;     // 8-column chunks per lane: C <= 64 * 8 * 4 = 2048

struct EmbScratch {
  int32_t *hist, *total, *start, *bsum, *lrank, *sorted, *stok;
  float* part;
};

EmbScratch carve(void* base, int M, int V, int C) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  char* p = (char*)base;
  EmbScratch s;
  const int nchunk = (int)cdiv(M, EB_CHUNK), nwin = (int)cdiv(M, EB_WIN);
  s.hist = (int32_t*)p;   p += up((size_t)nchunk * V * 4);
  s.total = (int32_t*)p;  p += up((size_t)V * 4);
  s.start = (int32_t*)p;  p += up((size_t)V * 4);
  s.bsum = (int32_t*)p;   p += up((size_t)cdiv(V, EB_SB) * 4);
  s.lrank = (int32_t*)p;  p += up((size_t)M * 4);
  s.sorted = (int32_t*)p; p += up((size_t)M * 4);
  s.stok = (int32_t*)p;   p += up((size_t)M * 4);
  s.part = (float*)p;     (void)nwin;
  return s;
}

__device__ __forceinline__ int clamp_id(int id, int V) { return id < 0 ? 0 : (id >= V ? V - 1 : id); }

__global__ __launch_bounds__(EB_CHUNK) void emb_hist_kernel(const int32_t* __restrict__ tok, int M,
                                                            int V, int32_t* __restrict__ hist,
                                                            int32_t* __restrict__ lrank) {
  __shared__ int ts[EB_CHUNK];
  const int tid = threadIdx.x;
  const int m = blockIdx.x * EB_CHUNK + tid;
  const int v = m < M ? clamp_id(tok[m], V) : -1;
  ts[tid] = v;
  __syncthreads();
  if (m >= M) return;
  atomicAdd(&hist[(int64_t)blockIdx.x * V + v], 1);  // integer: order-independent
  // rank among the earlier positions of this chunk with the same token; the
  // first loop's bound is the same for the whole wave (broadcast reads)
  int r = 0;
  const int wbase = tid & ~63;
  for (int j = 0; j < wbase; ++j) r += ts[j] == v;
  for (int j = wbase; j < tid; ++j) r += ts[j] == v;
  lrank[m] = r;
}

// per token: prefix of its chunk counts (in place) and total; per block of
// EB_SB tokens: exclusive scan of the totals (start) and the block sum
__global__ __launch_bounds__(EB_SB) void emb_offsets_kernel(int32_t* __restrict__ hist, int nchunk,
                                                            int V, int32_t* __restrict__ total,
                                                            int32_t* __restrict__ start,
                                                            int32_t* __restrict__ bsum) {
  __shared__ int sc[EB_SB];
  const int v = blockIdx.x * EB_SB + threadIdx.x;
  int run = 0;
  if (v < V) {
    for (int c = 0; c < nchunk; ++c) {
      const int h = hist[(int64_t)c * V + v];
      hist[(int64_t)c * V + v] = run;
      run += h;
    }
    total[v] = run;
  }
  sc[threadIdx.x] = run;
  __syncthreads();
  for (int o = 1; o < EB_SB; o <<= 1) {  // inclusive scan in LDS
    const int x = threadIdx.x >= o ? sc[threadIdx.x - o] : 0;
    __syncthreads();
    sc[threadIdx.x] += x;
    __syncthreads();
  }
  if (v < V) start[v] = sc[threadIdx.x] - run;
  if (threadIdx.x == EB_SB - 1) bsum[blockIdx.x] = sc[EB_SB - 1];
}

// exclusive scan of the nb block sums in place (one workgroup of 1024)
__global__ __launch_bounds__(1024) void emb_scan_kernel(int32_t* __restrict__ bsum, int nb) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < nb; b0 += 1024) {
    const int i = b0 + tid;
    const int x0 = i < nb ? bsum[i] : 0;
    sc[tid] = x0;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int x = tid >= o ? sc[tid - o] : 0;
      __syncthreads();
      sc[tid] += x;
      __syncthreads();
    }
    if (i < nb) bsum[i] = carry + sc[tid] - x0;
    carry += sc[1023];
    __syncthreads();
  }
}

__device__ __forceinline__ int seg_start(const int32_t* start, const int32_t* bsum, int v) {
  return bsum[v / EB_SB] + start[v];
}

__global__ __launch_bounds__(256) void emb_place_kernel(const int32_t* __restrict__ tok, int M, int V,
                                                        const int32_t* __restrict__ hist,
                                                        const int32_t* __restrict__ start,
                                                        const int32_t* __restrict__ bsum,
                                                        const int32_t* __restrict__ lrank,
                                                        int32_t* __restrict__ sorted,
                                                        int32_t* __restrict__ stok) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int v = clamp_id(tok[m], V);
  const int slot = seg_start(start, bsum, v) + hist[(int64_t)(m / EB_CHUNK) * V + v] + lrank[m];
  sorted[slot] = m;
  stok[slot] = v;
}

template <class T>
__device__ __forceinline__ void load_row_chunk(const T* p, float v[8]);
template <>
__device__ __forceinline__ void load_row_chunk<bf16>(const bf16* p, float v[8]) {
  Pack<bf16> a = load_pack(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = to_f(a.e[i]);
}
template <>
__device__ __forceinline__ void load_row_chunk<float>(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void add_row(float* __restrict__ dst, const float acc[8]) {
  float4* d = reinterpret_cast<float4*>(dst);
  float4 a = d[0], b = d[1];
  a.x += acc[0]; a.y += acc[1]; a.z += acc[2]; a.w += acc[3];
  b.x += acc[4]; b.y += acc[5]; b.z += acc[6]; b.w += acc[7];
  d[0] = a;
  d[1] = b;
}
__device__ __forceinline__ void put_row(float* __restrict__ dst, const float acc[8]) {
  float4* d = reinterpret_cast<float4*>(dst);
  d[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  d[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// A window's C columns are split over G waves (column groups of 64 chunks
// of 8, so that twice as many waves run at C = 768); lane l of group g owns
// chunk 64 g + l (NCH = 1) or chunks 64 (g NCH + k) + l.  Every group sees
// the same runs and adds in the same slot order.  Rows are fetched EB_BATCH /
// NCH slots at a time, and with each slot's dx row the dwte row of its token:
// a token's slots form one run, so a run that ends in this window and lies
// wholly inside it is the only writer of that dwte row, and reading the row
// before the batch's stores reads what the add needs.  All of a batch's
// loads are issued at once from valid addresses (a slot past the window or a
// lane past the columns reads a valid row it does not use), so one memory
// latency covers them; a read-modify-write per run end made every wave wait
// once per slot behind its previous store.
constexpr int EB_BATCH = 8;

template <class T, int NCH>
__global__ __launch_bounds__(256) void emb_window_kernel(const T* __restrict__ dx, int M, int C,
                                                         int G, const int32_t* __restrict__ sorted,
                                                         const int32_t* __restrict__ stok,
                                                         float* __restrict__ dwte,
                                                         float* __restrict__ part) {
  constexpr int NB = EB_BATCH / NCH;  // slots per batch
  const int lane = threadIdx.x % 64;
  const int wg = blockIdx.x * 4 + threadIdx.x / 64;
  const int w = wg / G, g = wg % G;
  const int s0 = w * EB_WIN;
  if (s0 >= M) return;
  const int n = min(EB_WIN, M - s0);
  const int nch = C / 8;
  const int ch0 = 64 * NCH * g + lane;  // this lane's first chunk
  const int mytok = lane < n ? stok[s0 + lane] : -1;
  const int mypos = lane < n ? sorted[s0 + lane] : 0;
  const int prev_tok = s0 > 0 ? stok[s0 - 1] : -1;
  const int next_tok = s0 + n < M ? stok[s0 + n] : -1;
  float acc[NCH][8];
  int run_first = 0;
  for (int i0 = 0; i0 < n; i0 += NB) {
    float rows[NB][NCH][8], old[NB][NCH][8];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int ic = min(i0 + b, n - 1);
      const int pos = __builtin_amdgcn_readlane(mypos, ic);
      const int t = __builtin_amdgcn_readlane(mytok, ic);
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int ch = min(ch0 + 64 * k, nch - 1);
        load_row_chunk(dx + (int64_t)pos * C + ch * 8, rows[b][k]);
        load_row_chunk(dwte + (int64_t)t * C + ch * 8, old[b][k]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = i0 + b;
      if (i >= n) break;
      const int t = __builtin_amdgcn_readlane(mytok, i);
      if (i == run_first) {
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[k][j] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[k][j] += rows[b][k][j];
      const int tn = i + 1 < n ? __builtin_amdgcn_readlane(mytok, i + 1) : -2;
      if (tn != t) {  // the run ends at slot i of this window
        const bool from_prev = run_first == 0 && prev_tok == t;
        const bool into_next = i == n - 1 && next_tok == t;
        const bool direct = !from_prev && !into_next;
        float* dst = direct ? dwte + (int64_t)t * C
                            : part + ((int64_t)w * 2 + (from_prev ? 0 : 1)) * C;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const int ch = ch0 + 64 * k;
          if (ch < nch) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = direct ? old[b][k][j] + acc[k][j] : acc[k][j];
            put_row(dst + ch * 8, v);
          }
        }
        run_first = i + 1;
      }
    }
  }
}

// One wave per window whose last run starts in it and continues into the
// next window: the token's segment (known from the scan) tells which windows
// hold its partials.
template <int NCH>
__global__ __launch_bounds__(256) void emb_combine_kernel(int M, int C, int G,
                                                          const int32_t* __restrict__ stok,
                                                          const int32_t* __restrict__ total,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ bsum,
                                                          const float* __restrict__ part,
                                                          float* __restrict__ dwte) {
  const int lane = threadIdx.x % 64;
  const int wg = blockIdx.x * 4 + threadIdx.x / 64;
  const int w = wg / G, g = wg % G;
  const int ch0 = 64 * NCH * g + lane;
  const int nwin = (int)cdiv(M, EB_WIN);
  if (w >= nwin) return;
  const int s0 = w * EB_WIN, n = min(EB_WIN, M - s0);
  const int t = stok[s0 + n - 1];
  const int seg0 = seg_start(start, bsum, t), seg1 = seg0 + total[t];  // slots of token t
  if (seg1 <= s0 + n) return;  // the last run ends in this window
  if (seg0 < s0) return;       // it started in an earlier window
  const int wend = (seg1 - 1) / EB_WIN;  // window holding the segment's last slot
  const int nch = C / 8;
  float acc[NCH][8];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int ch = ch0 + 64 * k;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[k][j] = 0.f;
    if (ch < nch) {
      const float* src = part + ((int64_t)w * 2 + 1) * C + ch * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[k][j] = src[j];
    }
  }
#pragma unroll 4
  for (int w2 = w + 1; w2 <= wend; ++w2) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = ch0 + 64 * k;
      if (ch < nch) {
        const float* src = part + ((int64_t)w2 * 2) * C + ch * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[k][j] += src[j];
      }
    }
  }
  float* dst = dwte + (int64_t)t * C;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int ch = ch0 + 64 * k;
    if (ch < nch) add_row(dst + ch * 8, acc[k]);
  }
}

}  // namespace

size_t encoder_backward_wte_scratch_bytes(int M, int V, int C) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t nchunk = cdiv(M, EB_CHUNK), nwin = cdiv(M, EB_WIN);
  return up(nchunk * V * 4) + 2 * up((size_t)V * 4) + up((size_t)cdiv(V, EB_SB) * 4) +
         3 * up((size_t)M * 4) + up(nwin * 2 * (size_t)C * 4);
}

hipError_t encoder_backward_wte(int dt, float* dwte, const void* dx, const int32_t* tok, int M,
                                int C, int V, void* scratch, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (C % 8 != 0 || C > 64 * 8 * EB_MAXCH || !scratch) return hipErrorInvalidValue;
  EmbScratch sc = carve(scratch, M, V, C);
  const int nchunk = (int)cdiv(M, EB_CHUNK), nwin = (int)cdiv(M, EB_WIN);
  const int nsb = (int)cdiv(V, EB_SB);
  hipError_t e = fill_i32(sc.hist, 0, (int64_t)nchunk * V, s);
  if (e != hipSuccess) return e;
  emb_hist_kernel<<<nchunk, EB_CHUNK, 0, s>>>(tok, M, V, sc.hist, sc.lrank);
  emb_offsets_kernel<<<nsb, EB_SB, 0, s>>>(sc.hist, nchunk, V, sc.total, sc.start, sc.bsum);
  emb_scan_kernel<<<1, 1024, 0, s>>>(sc.bsum, nsb);
  emb_place_kernel<<<(unsigned)cdiv(M, 256), 256, 0, s>>>(tok, M, V, sc.hist, sc.start, sc.bsum,
                                                          sc.lrank, sc.sorted, sc.stok);
  // column groups: one chunk per lane up to C = 1024 (two groups at 768),
  // two chunks per lane in at most two groups beyond
  const int nchunks = C / 8;
  const int nchl = nchunks <= 128 ? 1 : (int)cdiv(nchunks, 64 * 2);  // chunks per lane
  const int G = (int)cdiv(nchunks, 64 * nchl);
  const unsigned gw = (unsigned)cdiv((int64_t)nwin * G, 4);
#define EMB_GO(NC)                                                                                \
  do {                                                                                            \
    if (dt == BF16)                                                                               \
      emb_window_kernel<bf16, NC><<<gw, 256, 0, s>>>((const bf16*)dx, M, C, G, sc.sorted,         \
                                                     sc.stok, dwte, sc.part);                     \
    else                                                                                          \
      emb_window_kernel<float, NC><<<gw, 256, 0, s>>>((const float*)dx, M, C, G, sc.sorted,       \
                                                      sc.stok, dwte, sc.part);                    \
    emb_combine_kernel<NC><<<gw, 256, 0, s>>>(M, C, G, sc.stok, sc.total, sc.start, sc.bsum,     \
                                              sc.part, dwte);                                     \
  } while (0)
  if (nchl == 1) EMB_GO(1);
  else EMB_GO(2);
#undef EMB_GO
  return hipGetLastError();
}

}  // namespace gk
