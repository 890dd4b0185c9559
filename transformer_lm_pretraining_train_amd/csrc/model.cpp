// Runtime of libgpt2.so: config validation, the flat parameter layout, the
// carve-up of the caller's single workspace, and the launch sequences of
// forward, backward and the optimizer step on the caller's HIP stream (plus
// one internal stream, joined by events, for the paired weight-gradient
// launches of the backward); around the step, the loss-only forward, the
// guarded optimizer step and checkpoint files.
//
// The whole model state lives in the one workspace the caller allocates, in
// this order (each region 256-byte aligned): fp32 parameters, gradients,
// AdamW m and v; the bf16 copy of the parameters (bf16 mode); activations
// kept for the backward; backward buffers; reduction scratch; flags.  The
// library allocates nothing on the device after gpt2_create.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "../../include/gpt2.h"
#include "common.h"
#include "kernels.h"

using namespace gk;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(GPT2_EHIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                  __LINE__);                                                              \
  } while (0)

constexpr size_t kAlign = 256;

struct TensorInfo {
  std::string name;
  int64_t offset;
  int64_t rows, cols;  // cols == 1 for 1-D
  int ndim;
};

struct LayerOffsets {
  int64_t ln1_w, ln1_b, qkv_w, qkv_b, proj_w, proj_b, ln2_w, ln2_b, fc_w, fc_b, fcp_w, fcp_b;
};

struct Layout {
  int64_t wte, wpe, lnf_w, lnf_b, total, layer0, layer_size;
  std::vector<LayerOffsets> layers;
  std::vector<TensorInfo> tensors;
};

// Flat order: wte, wpe, per layer (ln1 w/b, qkv w/b, proj w/b, ln2 w/b,
// fc w/b, fcp w/b), lnf w/b.
Layout make_layout(const gpt2_config& c) {
  Layout L;
  const int64_t C = c.n_embd;
  int64_t off = 0;
  auto add = [&](const std::string& name, int64_t rows, int64_t cols, int ndim) {
    L.tensors.push_back({name, off, rows, cols, ndim});
    int64_t o = off;
    off += rows * cols;
    return o;
  };
  L.wte = add("wte", c.padded_vocab_size, C, 2);
  L.wpe = add("wpe", c.block_size, C, 2);
  L.layer0 = off;
  for (int l = 0; l < c.n_layer; ++l) {
    std::string p = "h" + std::to_string(l) + ".";
    LayerOffsets o;
    o.ln1_w = add(p + "ln1_w", C, 1, 1);
    o.ln1_b = add(p + "ln1_b", C, 1, 1);
    o.qkv_w = add(p + "qkv_w", 3 * C, C, 2);
    o.qkv_b = add(p + "qkv_b", 3 * C, 1, 1);
    o.proj_w = add(p + "proj_w", C, C, 2);
    o.proj_b = add(p + "proj_b", C, 1, 1);
    o.ln2_w = add(p + "ln2_w", C, 1, 1);
    o.ln2_b = add(p + "ln2_b", C, 1, 1);
    o.fc_w = add(p + "fc_w", 4 * C, C, 2);
    o.fc_b = add(p + "fc_b", 4 * C, 1, 1);
    o.fcp_w = add(p + "fcp_w", C, 4 * C, 2);
    o.fcp_b = add(p + "fcp_b", C, 1, 1);
    L.layers.push_back(o);
  }
  L.layer_size = 12 * C * C + 13 * C;
  L.lnf_w = add("lnf_w", C, 1, 1);
  L.lnf_b = add("lnf_b", C, 1, 1);
  L.total = off;
  return L;
}

// fused_head: the backward regenerates the logit gradient this many
// vocabulary columns at a time (24 tiles of 192 columns; 151 MB at
// B x T = 16 x 1024).  A remainder narrower than 256 columns (the least the
// large tiles take) joins the block before it, so a block holds at most
// kHeadChunk + 192 columns (the padded vocabulary is a multiple of 64).
constexpr int kHeadChunk = 4608;
int head_block_cols(int Vp, int col0) {
  const int rest = Vp - col0;
  return rest - kHeadChunk < 256 ? rest : kHeadChunk;
}

int validate(const gpt2_config* c) {
  if (!c) return fail(GPT2_EINVAL, "config is NULL");
  if (c->n_layer < 1 || c->n_head < 1) return fail(GPT2_EINVAL, "n_layer and n_head must be >= 1");
  if (c->n_embd < 64 || c->n_embd % 64 != 0 || c->n_embd > 2048)
    return fail(GPT2_EINVAL, "n_embd must be a multiple of 64 in [64, 2048], got %d", c->n_embd);
  if (c->n_embd % c->n_head != 0) return fail(GPT2_EINVAL, "n_embd must be divisible by n_head");
  int hd = c->n_embd / c->n_head;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(GPT2_EINVAL, "head size %d not supported (16, 32, 64, 128)", hd);
  if (c->seq_len < 1 || c->seq_len > c->block_size)
    return fail(GPT2_EINVAL, "need 1 <= seq_len <= block_size");
  if (c->vocab_size < 1 || c->padded_vocab_size < c->vocab_size)
    return fail(GPT2_EINVAL, "need 1 <= vocab_size <= padded_vocab_size");
  if (c->micro_batch < 1 || c->grad_accum_steps < 1)
    return fail(GPT2_EINVAL, "micro_batch and grad_accum_steps must be >= 1");
  if ((int64_t)c->micro_batch * c->seq_len > (1 << 24))
    return fail(GPT2_EINVAL, "micro_batch * seq_len too large");
  if (c->dtype != GPT2_FP32 && c->dtype != GPT2_BF16) return fail(GPT2_EINVAL, "dtype must be 0 or 1");
  if (!(c->ln_eps > 0.f)) return fail(GPT2_EINVAL, "ln_eps must be > 0");
  if (c->recompute < 0 || c->recompute > 2) return fail(GPT2_EINVAL, "recompute must be 0, 1 or 2");
  if (c->fused_head < 0 || c->fused_head > 1) return fail(GPT2_EINVAL, "fused_head must be 0 or 1");
  if (c->fused_head) {
    const int64_t M = (int64_t)c->micro_batch * c->seq_len;
    if (c->dtype != GPT2_BF16) return fail(GPT2_EINVAL, "fused_head needs dtype bf16");
    if (c->padded_vocab_size % 64 != 0)
      return fail(GPT2_EINVAL, "fused_head needs padded_vocab_size a multiple of 64");
    if (!gemm_rowstats_ok(BF16, (int)M, c->padded_vocab_size, c->n_embd, c->n_embd, c->n_embd) ||
        !gemm_dlogits_ok(BF16, (int)M, head_block_cols(c->padded_vocab_size, 0), c->n_embd,
                         c->n_embd, c->n_embd, kHeadChunk + 192))
      return fail(GPT2_EINVAL, "fused_head needs micro_batch * seq_len >= 256 and padded_vocab_size >= 256");
  }
  return GPT2_OK;
}

}  // namespace

int gpt2_internal_fail(int code, const char* msg) { return fail(code, "%s", msg); }

struct LayerAct {
  void *ln1, *qkv, *atty, *res2, *ln2, *fch, *fchg, *res3;
  float *ln1_mean, *ln1_rstd, *ln2_mean, *ln2_rstd, *lse;
};

struct gpt2_model {
  gpt2_config cfg;
  Layout lay;
  hipStream_t stream;
  int dt;
  int L, H, C, hd, V, Vp, B, Tn, k;
  int64_t M, N, ldl;
  // state
  float *params, *grads, *m, *v;
  void* shadow;  // bf16 parameters (bf16 mode) or nullptr
  // activations
  void* encoded;
  std::vector<LayerAct> act;
  void* lnf;
  float *lnf_mean, *lnf_rstd;
  void* logits;
  void* dlogits;  // d loss / d logits of the last forward with targets (same pitch)
  // fused_head: no logits or dlogits (both null); the backward regenerates
  // d logits per block of kHeadChunk vocabulary columns into head_chunk
  // (pitch head_ld), which the forward's row statistics also use, and sums
  // d lnf over the blocks in fp32 (dlnf32)
  bool fused_head = false;
  void* head_chunk = nullptr;
  int64_t head_ld = 0;
  float* dlnf32 = nullptr;
  int32_t* targets_keep = nullptr;  // the forward's targets, for the backward
  float *losses, *ce_lse, *loss_internal;
  int32_t* argmax;
  // backward
  // Backward buffers.  Per layer: d res3 (the layer's input gradient from
  // above), d res2, d fch and d qkv, in three sets used in turn (layer l:
  // set l % 3), so that two layers' are still intact while their weight
  // gradients run, on the side stream, beside the next layer; dres: d x of
  // the first layer (the embedding gradient); dbuf_c: scratch activation
  // gradient.
  void *bw_in[3], *bw_mid[3], *bw_d4[3], *bw_dq[3];
  // recompute >= 1: the forward's GELU output goes to fchg_tmp (read at once
  // by the next product) and the backward regenerates each layer's into
  // bw_fchg[set]; recompute 2: the same for the LayerNorm outputs (ln_tmp,
  // bw_ln1 / bw_ln2).  Null otherwise.
  void* fchg_tmp = nullptr;
  void* ln_tmp = nullptr;
  void *bw_fchg[3] = {nullptr, nullptr, nullptr};
  void *bw_ln1[3] = {nullptr, nullptr, nullptr}, *bw_ln2[3] = {nullptr, nullptr, nullptr};
  // A second stream for the weight-gradient launches of two layers, which
  // fill 216 of the 256 CUs: the next layer's work runs beside them.
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> ev_ready, ev_done;  // one pair per two layers
  void *dres, *dbuf_c;
  void* scratch;
  // Column partial sums of every LayerNorm backward and bias gradient of a
  // backward pass, each in its own slot; one batched reduction at the end.
  void* colpart;
  size_t ln_slot, bg_slot;  // bytes per LayerNorm / bias-gradient slot
  std::vector<ColReduce> cols;
  void* gemm_ws;  // split-K partial tiles of the weight-gradient GEMMs
  size_t gemm_ws_bytes;
  void* norm_scratch;
  int* err_flag;
  // bookkeeping
  const int32_t* tokens;
  const int32_t* targets;
  bool have_targets;
  int64_t step;
  // the norm of the current gradients (gpt2_grad_norm), valid until they change
  bool norm_ready = false;
  float norm_value = 0.f;
  int64_t skips_nonfinite = 0, skips_outlier = 0;
  // optional HIP event pairs around one kind of launch (gpt2_set_kernel_timer)
  int timer_which = GPT2_TIMER_NONE;
  int timer_cap = 0, timer_used = 0;
  std::vector<hipEvent_t> timer_ev;

  // weights in the GEMM input type
  const void* wt(int64_t off) const {
    return dt == BF16 ? (const void*)((const uint16_t*)shadow + off) : (const void*)(params + off);
  }
};

namespace {

// Walks the workspace plan; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  void* take(size_t bytes) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

size_t plan(const gpt2_config& c, char* base, gpt2_model* mdl) {
  Layout lay = make_layout(c);
  Carver cv{base};
  const int64_t C = c.n_embd, M = (int64_t)c.micro_batch * c.seq_len, N = lay.total;
  const int dt = c.dtype;
  const size_t es = dsize(dt);
  const int64_t ldl = round_up(c.padded_vocab_size, 64);
  const int H = c.n_head;
  gpt2_model tmp;
  gpt2_model& md = mdl ? *mdl : tmp;
  md.params = (float*)cv.take(N * 4);
  md.grads = (float*)cv.take(N * 4);
  md.m = (float*)cv.take(N * 4);
  md.v = (float*)cv.take(N * 4);
  md.shadow = dt == BF16 ? cv.take(N * 2) : nullptr;
  md.encoded = cv.take(M * C * es);
  md.act.resize(c.n_layer);
  for (int l = 0; l < c.n_layer; ++l) {
    LayerAct& a = md.act[l];
    a.ln1 = c.recompute >= 2 ? nullptr : cv.take(M * C * es);
    a.ln1_mean = (float*)cv.take(M * 4);
    a.ln1_rstd = (float*)cv.take(M * 4);
    a.qkv = cv.take(M * 3 * C * es);
    a.atty = cv.take(M * C * es);
    a.lse = (float*)cv.take((int64_t)c.micro_batch * H * c.seq_len * 4);
    a.res2 = cv.take(M * C * es);
    a.ln2 = c.recompute >= 2 ? nullptr : cv.take(M * C * es);
    a.ln2_mean = (float*)cv.take(M * 4);
    a.ln2_rstd = (float*)cv.take(M * 4);
    a.fch = cv.take(M * 4 * C * es);
    a.fchg = c.recompute >= 1 ? nullptr : cv.take(M * 4 * C * es);
    a.res3 = cv.take(M * C * es);
  }
  if (c.recompute >= 1) {
    md.fchg_tmp = cv.take(M * 4 * C * es);
    for (int i = 0; i < 3; ++i) md.bw_fchg[i] = cv.take(M * 4 * C * es);
  }
  if (c.recompute >= 2) {
    md.ln_tmp = cv.take(M * C * es);
    for (int i = 0; i < 3; ++i) {
      md.bw_ln1[i] = cv.take(M * C * es);
      md.bw_ln2[i] = cv.take(M * C * es);
    }
  }
  md.lnf = cv.take(M * C * es);
  md.lnf_mean = (float*)cv.take(M * 4);
  md.lnf_rstd = (float*)cv.take(M * 4);
  md.fused_head = c.fused_head != 0;
  if (md.fused_head) {
    md.logits = md.dlogits = nullptr;
    md.head_ld = 0;  // the widest block
    for (int col0 = 0, nc = 0; col0 < c.padded_vocab_size; col0 += nc) {
      nc = head_block_cols(c.padded_vocab_size, col0);
      md.head_ld = std::max<int64_t>(md.head_ld, nc);
    }
    const int64_t ncols = gemm_rowstats_cols(c.padded_vocab_size);
    md.head_chunk = cv.take(std::max<int64_t>(M * md.head_ld * es, round_up(M * ncols * 8, 256) + M * 4));
    md.dlnf32 = (float*)cv.take(M * C * 4);
    md.targets_keep = (int32_t*)cv.take(M * 4);
  } else {
    md.logits = cv.take(M * ldl * es);
    md.dlogits = cv.take(M * ldl * es);
  }
  md.losses = (float*)cv.take(M * 4);
  md.ce_lse = (float*)cv.take(M * 4);
  md.argmax = (int32_t*)cv.take(M * 4);
  md.loss_internal = (float*)cv.take(4);
  for (int i = 0; i < 3; ++i) {
    md.bw_in[i] = cv.take(M * C * es);
    md.bw_mid[i] = cv.take(M * C * es);
    md.bw_d4[i] = cv.take(M * 4 * C * es);
    md.bw_dq[i] = cv.take(M * 3 * C * es);
  }
  md.dres = cv.take(M * C * es);
  md.dbuf_c = cv.take(M * C * es);
  size_t sc = layernorm_backward_scratch_bytes((int)M, (int)C);
  sc = std::max(sc, bias_grad_scratch_bytes((int)M, (int)(4 * C)));
  sc = std::max(sc, attention_backward_scratch_bytes(c.micro_batch, c.seq_len, H));
  sc = std::max(sc, encoder_backward_wte_scratch_bytes((int)M, c.vocab_size, (int)C));
  md.scratch = cv.take(sc);
  md.ln_slot = (layernorm_backward_scratch_bytes((int)M, (int)C) + kAlign - 1) / kAlign * kAlign;
  md.bg_slot = std::max({bias_grad_scratch_bytes((int)M, (int)(4 * C)),
                         (size_t)gemm_colsum_blocks((int)M) * 4 * C * sizeof(float),
                         (size_t)attention_colsum_blocks(c.micro_batch, c.seq_len) * 3 * C *
                             sizeof(float)});
  md.bg_slot = (md.bg_slot + kAlign - 1) / kAlign * kAlign;
  md.colpart = cv.take((size_t)(2 * c.n_layer + 1) * md.ln_slot + (size_t)(2 * c.n_layer) * md.bg_slot);
  md.cols.reserve(4 * c.n_layer + 1);
  size_t gw = 0;
  {
    const int Mi = (int)M, Ci = (int)C;
    const int dWshapes[5][2] = {{c.padded_vocab_size, Ci}, {Ci, 4 * Ci}, {4 * Ci, Ci}, {Ci, Ci},
                                {3 * Ci, Ci}};
    for (auto& sh : dWshapes) gw = std::max(gw, gemm_workspace_bytes(dt, sh[0], sh[1], Mi, EPI_ACC_F32));
    if (c.fused_head) {  // the head's gradient per block of vocabulary rows
      const int Vp = c.padded_vocab_size;
      for (int col0 = 0; col0 < Vp; col0 += head_block_cols(Vp, col0))
        gw = std::max(gw, gemm_workspace_bytes(dt, head_block_cols(Vp, col0), Ci, Mi, EPI_ACC_F32));
    }
    // the four weight gradients of a layer as one launch (shapes and pitches only)
    const AccItem grp[4] = {{Ci, 4 * Ci, nullptr, Ci, nullptr, 4 * Ci, nullptr, 4 * Ci},
                            {4 * Ci, Ci, nullptr, 4 * Ci, nullptr, Ci, nullptr, Ci},
                            {Ci, Ci, nullptr, Ci, nullptr, Ci, nullptr, Ci},
                            {3 * Ci, Ci, nullptr, 3 * Ci, nullptr, Ci, nullptr, Ci}};
    gw = std::max(gw, gemm_acc_group_workspace_bytes(dt, 4, grp, Mi));
  }
  md.gemm_ws = gw ? cv.take(gw) : nullptr;
  md.gemm_ws_bytes = gw;
  md.norm_scratch = cv.take(grad_norm_scratch_bytes());
  md.err_flag = (int*)cv.take(4);
  return (cv.off + kAlign - 1) / kAlign * kAlign;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GPT2_EHIP, "%s: %s", what, hipGetErrorString(e));
  return GPT2_OK;
}

#define LAUNCH(expr)                                 \
  do {                                               \
    int rc_ = check_launch((expr), #expr);           \
    if (rc_ != GPT2_OK) return rc_;                  \
  } while (0)

// Brackets one launch with a HIP event pair on the model's stream when the
// timer is set to `which` and has events left.
#define TIMED(which, expr)                                                          \
  do {                                                                              \
    const bool on_ = md->timer_which == (which) && md->timer_used < md->timer_cap;  \
    if (on_) HIP_TRY(hipEventRecord(md->timer_ev[2 * md->timer_used], md->stream)); \
    LAUNCH(expr);                                                                   \
    if (on_) {                                                                      \
      HIP_TRY(hipEventRecord(md->timer_ev[2 * md->timer_used + 1], md->stream));    \
      ++md->timer_used;                                                             \
    }                                                                               \
  } while (0)

// The same on a given stream (the side stream's weight-gradient pairs).
#define TIMED_ON(which, strm, expr)                                                 \
  do {                                                                              \
    const bool on_ = md->timer_which == (which) && md->timer_used < md->timer_cap;  \
    if (on_) HIP_TRY(hipEventRecord(md->timer_ev[2 * md->timer_used], (strm)));     \
    LAUNCH(expr);                                                                   \
    if (on_) {                                                                      \
      HIP_TRY(hipEventRecord(md->timer_ev[2 * md->timer_used + 1], (strm)));        \
      ++md->timer_used;                                                             \
    }                                                                               \
  } while (0)

void release_side(gpt2_model* md) {
  if (md->side) (void)hipStreamSynchronize(md->side);
  for (hipEvent_t e : md->ev_ready)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : md->ev_done)
    if (e) (void)hipEventDestroy(e);
  md->ev_ready.clear();
  md->ev_done.clear();
  if (md->side) (void)hipStreamDestroy(md->side);
  md->side = nullptr;
}

void release_timer(gpt2_model* md) {
  for (hipEvent_t e : md->timer_ev) (void)hipEventDestroy(e);
  md->timer_ev.clear();
  md->timer_which = GPT2_TIMER_NONE;
  md->timer_cap = md->timer_used = 0;
}

Epilogue epi(int mode, void* out, int64_t ldo) {
  Epilogue e{};
  e.mode = mode;
  e.out = out;
  e.ldo = ldo;
  return e;
}

DecayMap decay_map(const gpt2_model* md) {
  const Layout& L = md->lay;
  DecayMap d{};
  d.layer0 = L.layer0;
  d.layer_size = L.layer_size;
  d.n_layer_end = L.layer0 + L.layer_size * md->L;
  if (md->L > 0) {
    const LayerOffsets& o = L.layers[0];
    d.qkvw0 = o.qkv_w - L.layer0;
    d.qkvw1 = d.qkvw0 + 3LL * md->C * md->C;
    d.projw0 = o.proj_w - L.layer0;
    d.projw1 = d.projw0 + (int64_t)md->C * md->C;
    d.fcw0 = o.fc_w - L.layer0;
    d.fcw1 = d.fcw0 + 4LL * md->C * md->C;
    d.fcpw0 = o.fcp_w - L.layer0;
    d.fcpw1 = d.fcpw0 + 4LL * md->C * md->C;
  }
  return d;
}

char* act_ptr(void* p, int64_t elems_offset, int dt) {
  return (char*)p + elems_offset * dsize(dt);
}

}  // namespace

extern "C" {

const char* gpt2_last_error(void) { return g_err.c_str(); }

int64_t gpt2_num_params(const gpt2_config* cfg) {
  if (!cfg) return -1;
  if (validate(cfg) != GPT2_OK) return -1;
  return make_layout(*cfg).total;
}

size_t gpt2_workspace_bytes(const gpt2_config* cfg) {
  if (validate(cfg) != GPT2_OK) return 0;
  return plan(*cfg, nullptr, nullptr);
}

int gpt2_param_layout(const gpt2_config* cfg, gpt2_tensor_info* out, int cap) {
  if (!cfg) return fail(GPT2_EINVAL, "config is NULL");
  int rc = validate(cfg);
  if (rc != GPT2_OK) return rc;
  Layout L = make_layout(*cfg);
  int n = (int)L.tensors.size();
  if (out) {
    for (int i = 0; i < n && i < cap; ++i) {
      const TensorInfo& t = L.tensors[i];
      memset(&out[i], 0, sizeof(out[i]));
      snprintf(out[i].name, sizeof(out[i].name), "%s", t.name.c_str());
      out[i].offset = t.offset;
      out[i].ndim = t.ndim;
      out[i].decay = t.ndim == 2 ? 1 : 0;
      out[i].shape[0] = t.rows;
      out[i].shape[1] = t.cols;
    }
  }
  return n;
}

int gpt2_create(const gpt2_config* cfg, void* dev_workspace, size_t bytes, void* hip_stream,
                gpt2_model** out) {
  int rc = validate(cfg);
  if (rc != GPT2_OK) return rc;
  if (!out) return fail(GPT2_EINVAL, "out is NULL");
  *out = nullptr;
  size_t need = plan(*cfg, nullptr, nullptr);
  if (!dev_workspace || bytes < need)
    return fail(GPT2_EWORKSPACE, "workspace of %zu bytes, need %zu", bytes, need);
  if ((uintptr_t)dev_workspace % kAlign != 0)
    return fail(GPT2_EWORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  gpt2_model* md = new gpt2_model();
  md->cfg = *cfg;
  md->lay = make_layout(*cfg);
  md->stream = (hipStream_t)hip_stream;
  md->dt = cfg->dtype;
  md->L = cfg->n_layer;
  md->H = cfg->n_head;
  md->C = cfg->n_embd;
  md->hd = cfg->n_embd / cfg->n_head;
  md->V = cfg->vocab_size;
  md->Vp = cfg->padded_vocab_size;
  md->B = cfg->micro_batch;
  md->Tn = cfg->seq_len;
  md->k = cfg->grad_accum_steps;
  md->M = (int64_t)md->B * md->Tn;
  md->N = md->lay.total;
  md->ldl = round_up(md->Vp, 64);
  plan(*cfg, (char*)dev_workspace, md);
  md->tokens = md->targets = nullptr;
  md->have_targets = false;
  md->step = 0;
  hipStream_t s = md->stream;
  // zero all state (parameters, grads, m, v, shadow, logits padding, flags)
  hipError_t e = fill_f32((float*)dev_workspace, 0.f, (int64_t)(need / 4), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete md;
    return fail(GPT2_EHIP, "initialising the workspace: %s", hipGetErrorString(e));
  }
  // side stream (default priority) and its events: host-side objects only
  if (md->dt == BF16 && md->L >= 4) {
    const int np = md->L + 1;  // at most one side-stream group per layer
    e = hipStreamCreateWithFlags(&md->side, hipStreamNonBlocking);
    md->ev_ready.assign(np, nullptr);
    md->ev_done.assign(np, nullptr);
    for (int i = 0; i < np && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&md->ev_ready[i], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&md->ev_done[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
      release_side(md);
      delete md;
      return fail(GPT2_EHIP, "creating the side stream: %s", hipGetErrorString(e));
    }
  }
  *out = md;
  g_err.clear();
  return GPT2_OK;
}

int gpt2_destroy(gpt2_model* md) {
  if (md) {
    release_timer(md);
    release_side(md);
  }
  delete md;
  return GPT2_OK;
}

int gpt2_set_params(gpt2_model* md, const float* src) {
  if (!md || !src) return fail(GPT2_EINVAL, "NULL argument");
  HIP_TRY(hipMemcpyAsync(md->params, src, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  if (md->dt == BF16) LAUNCH(cast_f32_to_bf16(md->shadow, md->params, md->N, md->stream));
  return GPT2_OK;
}

int gpt2_get_params(gpt2_model* md, float* dst) {
  if (!md || !dst) return fail(GPT2_EINVAL, "NULL argument");
  HIP_TRY(hipMemcpyAsync(dst, md->params, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  return GPT2_OK;
}

int gpt2_get_grads(gpt2_model* md, float* dst) {
  if (!md || !dst) return fail(GPT2_EINVAL, "NULL argument");
  HIP_TRY(hipMemcpyAsync(dst, md->grads, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  return GPT2_OK;
}

int gpt2_set_grads(gpt2_model* md, const float* src) {
  if (!md || !src) return fail(GPT2_EINVAL, "NULL argument");
  md->norm_ready = false;
  HIP_TRY(hipMemcpyAsync(md->grads, src, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  return GPT2_OK;
}

int gpt2_get_opt_state(gpt2_model* md, float* dm, float* dv, int64_t* step) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (dm) HIP_TRY(hipMemcpyAsync(dm, md->m, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  if (dv) HIP_TRY(hipMemcpyAsync(dv, md->v, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  if (step) *step = md->step;
  return GPT2_OK;
}

int gpt2_set_opt_state(gpt2_model* md, const float* dm, const float* dv, int64_t step) {
  if (!md || !dm || !dv || step < 0) return fail(GPT2_EINVAL, "bad argument");
  HIP_TRY(hipMemcpyAsync(md->m, dm, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  HIP_TRY(hipMemcpyAsync(md->v, dv, md->N * 4, hipMemcpyDeviceToDevice, md->stream));
  md->step = step;
  return GPT2_OK;
}

int gpt2_zero_grad(gpt2_model* md) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  md->norm_ready = false;
  LAUNCH(fill_f32(md->grads, 0.f, md->N, md->stream));
  return GPT2_OK;
}

// Embeddings, the blocks and the final LayerNorm (into md->lnf).
static int forward_trunk(gpt2_model* md, const int32_t* tokens, const int32_t* targets) {
  if (!md || !tokens) return fail(GPT2_EINVAL, "NULL argument");
  const int dt = md->dt;
  const int C = md->C, H = md->H, M = (int)md->M;
  const Layout& Ly = md->lay;
  hipStream_t s = md->stream;
  const float eps = md->cfg.ln_eps;
  float* P = md->params;
  md->tokens = tokens;
  md->targets = targets;
  md->have_targets = false;

  LAUNCH(encoder_forward(dt, md->encoded, tokens, P + Ly.wte, P + Ly.wpe, M, md->Tn, C, md->V,
                         md->err_flag, s));
  const void* x = md->encoded;
  for (int l = 0; l < md->L; ++l) {
    const LayerOffsets& o = Ly.layers[l];
    LayerAct& a = md->act[l];
    void* ln1 = a.ln1 ? a.ln1 : md->ln_tmp;  // recompute 2: not kept
    void* ln2 = a.ln2 ? a.ln2 : md->ln_tmp;
    void* fchg = a.fchg ? a.fchg : md->fchg_tmp;  // recompute >= 1: not kept
    TIMED(GPT2_TIMER_LN_FWD, layernorm_forward(dt, ln1, a.ln1_mean, a.ln1_rstd, x, P + o.ln1_w,
                                               P + o.ln1_b, M, C, eps, s));
    Epilogue e = epi(EPI_BIAS, a.qkv, 3 * C);
    e.bias = P + o.qkv_b;
    LAUNCH(gemm(dt, true, true, M, 3 * C, C, ln1, C, md->wt(o.qkv_w), C, e, s));
    TIMED(GPT2_TIMER_ATTN_FWD,
          attention_forward(dt, a.atty, a.lse, a.qkv, md->B, md->Tn, H, md->hd, s));
    e = epi(EPI_BIAS_RESID, a.res2, C);
    e.bias = P + o.proj_b;
    e.resid = x;
    e.ldr = C;
    LAUNCH(gemm(dt, true, true, M, C, C, a.atty, C, md->wt(o.proj_w), C, e, s));
    TIMED(GPT2_TIMER_LN_FWD, layernorm_forward(dt, ln2, a.ln2_mean, a.ln2_rstd, a.res2,
                                               P + o.ln2_w, P + o.ln2_b, M, C, eps, s));
    e = epi(EPI_BIAS_GELU, a.fch, 4 * C);
    e.bias = P + o.fc_b;
    e.out2 = fchg;
    e.ldo2 = 4 * C;
    // with the GELU output kept for the backward, the pre-activation itself
    // is not needed there, only GELU' at it: stored in its place, so that
    // the backward's product multiplies instead of evaluating GELU' (the
    // step 0.3 % faster)
    e.dgelu = a.fchg != nullptr;
    LAUNCH(gemm(dt, true, true, M, 4 * C, C, ln2, C, md->wt(o.fc_w), C, e, s));
    e = epi(EPI_BIAS_RESID, a.res3, C);
    e.bias = P + o.fcp_b;
    e.resid = a.res2;
    e.ldr = C;
    LAUNCH(gemm(dt, true, true, M, C, 4 * C, fchg, 4 * C, md->wt(o.fcp_w), 4 * C, e, s));
    x = a.res3;
  }
  TIMED(GPT2_TIMER_LN_FWD, layernorm_forward(dt, md->lnf, md->lnf_mean, md->lnf_rstd, x,
                                             P + Ly.lnf_w, P + Ly.lnf_b, M, C, eps, s));
  return GPT2_OK;
}

// The loss of the tied head from per-row softmax statistics of its product,
// never the logits (bf16, shapes gemm_rowstats_ok() accepts): per-row (max,
// sum) of every 128 logits and the target's logit into `work`, then
// log-sum-exp and loss per row, then the mean.
static int head_loss_rowstats(gpt2_model* md, const int32_t* targets, void* work,
                              float* dev_loss) {
  const int C = md->C, M = (int)md->M;
  hipStream_t s = md->stream;
  const int ncols = gemm_rowstats_cols(md->Vp);
  float2* stats = (float2*)work;
  float* tgt = (float*)((char*)work + round_up((int64_t)M * ncols * 8, 256));
  LAUNCH(gemm_rowstats(M, md->Vp, C, md->lnf, C, md->wt(md->lay.wte), C, md->V, targets, stats,
                       ncols, tgt, s));
  LAUNCH(rowstats_loss(md->losses, md->ce_lse, stats, ncols, ncols, tgt, targets, M, md->V,
                       md->err_flag, s));
  LAUNCH(mean_loss(dev_loss ? dev_loss : md->loss_internal, md->losses, M, s));
  return GPT2_OK;
}

int gpt2_forward(gpt2_model* md, const int32_t* tokens, const int32_t* targets, float* dev_loss) {
  if (md && md->fused_head && !targets)
    return fail(GPT2_EINVAL, "fused_head keeps no logits: gpt2_forward needs targets");
  const int rc = forward_trunk(md, tokens, targets);
  if (rc != GPT2_OK) return rc;
  const int dt = md->dt;
  const int C = md->C, M = (int)md->M;
  const Layout& Ly = md->lay;
  hipStream_t s = md->stream;
  if (md->fused_head) {
    // the loss from row statistics; the backward regenerates d logits from
    // the log-sum-exp and these targets
    LAUNCH(hipMemcpyAsync(md->targets_keep, targets, (size_t)M * 4, hipMemcpyDeviceToDevice, s));
    const int r = head_loss_rowstats(md, targets, md->head_chunk, dev_loss);
    if (r != GPT2_OK) return r;
    md->have_targets = true;
    return GPT2_OK;
  }
  // logits over the padded vocabulary (tied head: wte)
  TIMED(GPT2_TIMER_LM_HEAD_FWD, gemm(dt, true, true, M, md->Vp, C, md->lnf, C, md->wt(Ly.wte), C,
                                     epi(EPI_STORE, md->logits, md->ldl), s));
  if (targets) {
    // loss and, from the same read of the logits, their gradient for the backward
    const float seed = (float)(1.0 / ((double)md->M * md->k));
    TIMED(GPT2_TIMER_CE_FWD, crossentropy_fused(dt, md->losses, md->ce_lse, md->argmax,
                                                md->dlogits, md->logits, md->ldl, targets, M,
                                                md->V, seed, md->err_flag, s));
    LAUNCH(mean_loss(dev_loss ? dev_loss : md->loss_internal, md->losses, M, s));
    md->have_targets = true;
  }
  return GPT2_OK;
}

int gpt2_forward_loss(gpt2_model* md, const int32_t* tokens, const int32_t* targets,
                      float* dev_loss) {
  if (!md || !tokens || !targets) return fail(GPT2_EINVAL, "NULL argument");
  const int rc = forward_trunk(md, tokens, targets);
  if (rc != GPT2_OK) return rc;
  const int dt = md->dt, C = md->C, M = (int)md->M;
  const Layout& Ly = md->lay;
  hipStream_t s = md->stream;
  md->have_targets = false;  // nothing for a backward
  if (gemm_rowstats_ok(dt, M, md->Vp, C, C, C)) {
    // the gradient buffer (unused without a backward), or the fused head's
    // chunk buffer, holds the row statistics
    return head_loss_rowstats(md, targets, md->fused_head ? md->head_chunk : md->dlogits,
                              dev_loss);
  }
  // fp32 or small shapes: the logits, then the loss alone
  LAUNCH(gemm(dt, true, true, M, md->Vp, C, md->lnf, C, md->wt(Ly.wte), C,
              epi(EPI_STORE, md->logits, md->ldl), s));
  LAUNCH(crossentropy_forward(dt, md->losses, md->ce_lse, md->argmax, md->logits, md->ldl,
                              targets, M, md->V, md->err_flag, s));
  LAUNCH(mean_loss(dev_loss ? dev_loss : md->loss_internal, md->losses, M, s));
  return GPT2_OK;
}

int gpt2_backward(gpt2_model* md) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (!md->have_targets)
    return fail(GPT2_ESTATE, "backward needs a preceding forward with targets");
  md->have_targets = false;
  md->norm_ready = false;
  const int dt = md->dt;
  const int C = md->C, H = md->H, M = (int)md->M;
  const Layout& Ly = md->lay;
  hipStream_t s = md->stream;
  float* P = md->params;
  float* G = md->grads;

  // Column sums (LayerNorm gain/shift, biases) are written as partials into
  // their own slots and reduced together after the layer loop.
  md->cols.clear();
  char* colslot = (char*)md->colpart;
  auto ln_part = [&]() {
    void* p = colslot;
    colslot += md->ln_slot;
    md->cols.emplace_back();
    return p;
  };
  auto bg_part = [&]() {
    void* p = colslot;
    colslot += md->bg_slot;
    md->cols.emplace_back();
    return p;
  };
  if (md->fused_head) {
    // tied head without stored logits: per block of vocabulary columns,
    // d logits regenerated from lnf, wte and the forward's log-sum-exp, then
    // d lnf += dz wte (fp32 over the blocks) and dwte += dz^T lnf
    const float seed = (float)(1.0 / ((double)md->M * md->k));
    LAUNCH(fill_f32(md->dlnf32, 0.f, (int64_t)M * C, s));
    for (int col0 = 0, nc = 0; col0 < md->Vp; col0 += nc) {
      nc = head_block_cols(md->Vp, col0);
      const void* wc = (const char*)md->wt(Ly.wte) + (int64_t)col0 * C * dsize(dt);
      LAUNCH(gemm_dlogits(M, nc, C, md->lnf, C, wc, C, md->ce_lse, md->targets_keep, col0, md->V,
                          seed, md->head_chunk, md->head_ld, s));
      LAUNCH(gemm(dt, true, false, M, C, nc, md->head_chunk, md->head_ld, wc, C,
                  epi(EPI_ACC_F32, md->dlnf32, C), s));
      LAUNCH(gemm(dt, false, false, nc, C, M, md->head_chunk, md->head_ld, md->lnf, C,
                  epi(EPI_ACC_F32, G + Ly.wte + (int64_t)col0 * C, C), s, md->gemm_ws,
                  md->gemm_ws_bytes));
    }
    LAUNCH(cast_f32_to_bf16(md->dbuf_c, md->dlnf32, (int64_t)M * C, s));
  } else {
    // tied head (d logits from the forward's cross-entropy): dwte += dz^T lnf ; dlnf = dz wte
    LAUNCH(gemm(dt, false, false, md->Vp, C, M, md->dlogits, md->ldl, md->lnf, C,
                epi(EPI_ACC_F32, G + Ly.wte, C), s, md->gemm_ws, md->gemm_ws_bytes));
    LAUNCH(gemm(dt, true, false, M, C, md->Vp, md->dlogits, md->ldl, md->wt(Ly.wte), C,
                epi(EPI_STORE, md->dbuf_c, C), s));
  }
  const void* xfinal = md->L > 0 ? md->act[md->L - 1].res3 : md->encoded;
  // The column sums of each residual gradient a LayerNorm backward produces
  // are the bias gradient of the linear layer that wrote that residual:
  // fc-proj of the layer below (res3) or proj of the same layer (res2).
  float* fcp_b_below = md->L > 0 ? G + Ly.layers[md->L - 1].fcp_b : nullptr;
  // Layer l works in buffer set l % 3: in (d res3, from the layer above),
  // mid (d res2), d4 (d fch), dq (d qkv).  Its four weight gradients are
  // queued and launched together with the next layer's: one launch of eight
  // products when their tiles fit the chip in one round (else four at a
  // time).  Such a pair runs on the side stream, beside the next layer's
  // work (the pair of the first two layers beside the embedding and the
  // remaining bias and LayerNorm gradients); the main stream waits for it
  // before it writes either of the pair's buffer sets again.  Where two
  // layers do not fit one round (wider models), each layer's four run on the
  // side stream the same way, beside the next layer: one launch when they fit
  // a round (GPT-2 350M: 192 tiles), else one per product with its own K
  // split.  All of them run on the side stream, in order, so that it alone
  // uses the split-K workspace.
  const int Lh = md->L;
  void* top = Lh > 0 ? md->bw_in[(Lh - 1) % 3] : md->dres;
  // groups running on the side stream whose buffer sets are not yet
  // reusable, oldest first: event index and the sets they read
  struct SideGroup {
    int ev, sets[2];
  };
  constexpr int kSidePend = 8;  // the three-set rotation keeps at most ~3 pending
  SideGroup side_pend[kSidePend];
  int nside = 0;
  int npairs = 0;  // side-stream groups launched so far (event index)
  auto guard = [&](int set) -> hipError_t {  // main stream: set `set` is about to be written
    // wait for the newest group that reads `set`; the side stream runs in
    // order, so the groups before it are done then too
    for (int i = nside - 1; i >= 0; --i) {
      if (side_pend[i].sets[0] == set || side_pend[i].sets[1] == set) {
        const int ev = side_pend[i].ev;
        for (int j = i + 1; j < nside; ++j) side_pend[j - i - 1] = side_pend[j];
        nside -= i + 1;
        return hipStreamWaitEvent(s, md->ev_done[ev], 0);
      }
    }
    return hipSuccess;
  };
  // launch n_ queued products reading buffer sets s0_ and s1_ (-1: none) on
  // the side stream, once the main stream has produced their inputs
#define SIDE_LAUNCH(n_, s0_, s1_)                                                               \
  do {                                                                                          \
    if (nside == kSidePend) LAUNCH(guard(side_pend[0].sets[0]));                                \
    LAUNCH(hipEventRecord(md->ev_ready[npairs], s));                                            \
    LAUNCH(hipStreamWaitEvent(md->side, md->ev_ready[npairs], 0));                              \
    TIMED_ON(GPT2_TIMER_WGRAD, md->side,                                                        \
             gemm_acc_group(dt, (n_), pend, M, md->gemm_ws, md->gemm_ws_bytes, md->side));      \
    LAUNCH(hipEventRecord(md->ev_done[npairs], md->side));                                      \
    side_pend[nside++] = SideGroup{npairs, {(s0_), (s1_)}};                                     \
    ++npairs;                                                                                   \
  } while (0)
  {
    void* slot = ln_part();
    TIMED(GPT2_TIMER_LN_BWD,
          layernorm_backward(dt, top, nullptr, G + Ly.lnf_w, G + Ly.lnf_b, fcp_b_below, false,
                             md->dbuf_c, xfinal, md->lnf_mean, md->lnf_rstd, P + Ly.lnf_w, M, C,
                             slot, s, &md->cols.back()));
  }
  AccItem pend[8];
  int npend = 0;
  // with a side stream every weight-gradient launch goes there, in order,
  // so that it alone uses the split-K workspace
  auto on_side = [&]() { return md->side != nullptr && npairs < (int)md->ev_done.size(); };
  for (int l = Lh - 1; l >= 0; --l) {
    const LayerOffsets& o = Ly.layers[l];
    LayerAct& a = md->act[l];
    const void* xin = l > 0 ? md->act[l - 1].res3 : md->encoded;
    const int set = l % 3;
    void* in = md->bw_in[set];
    void* mid = md->bw_mid[set];
    void* d4 = md->bw_d4[set];
    void* dq = md->bw_dq[set];
    LAUNCH(guard(set));
    // MLP output projection: res3 = res2 + fchg fcp_w^T + fcp_b
    // recomputed activations of this layer (bit-identical to the forward's:
    // the same kernels on the same kept inputs)
    void* fchg = a.fchg ? a.fchg : md->bw_fchg[set];
    void* ln2 = a.ln2 ? a.ln2 : md->bw_ln2[set];
    void* ln1 = a.ln1 ? a.ln1 : md->bw_ln1[set];
    if (!a.ln2)
      LAUNCH(layernorm_forward(dt, ln2, a.ln2_mean, a.ln2_rstd, a.res2, P + o.ln2_w, P + o.ln2_b,
                               M, C, md->cfg.ln_eps, s));
    if (!a.ln1)
      LAUNCH(layernorm_forward(dt, ln1, a.ln1_mean, a.ln1_rstd, xin, P + o.ln1_w, P + o.ln1_b, M,
                               C, md->cfg.ln_eps, s));
    Epilogue e = epi(EPI_GELU_BWD, d4, 4 * C);
    e.aux = a.fch;  // GELU' at the pre-activation where the GELU output was kept, else the pre-activation
    e.ldx = 4 * C;
    e.dgelu = a.fchg != nullptr;
    if (!a.fchg) {  // the GELU output again, from the pre-activation this product reads
      e.out2 = fchg;
      e.ldo2 = 4 * C;
    }
    // d fc_b = column sums of d4: per 64-row block in the product's epilogue
    // where it can, else a pass over d4 after the next product
    const bool fcb_fused = gemm_colsum_ok(dt, true, false, M, 4 * C, C, C, 4 * C, EPI_GELU_BWD);
    if (fcb_fused) {
      float* slot = (float*)bg_part();
      e.colsum = slot;
      e.ldcs = 4 * C;
      md->cols.back() = ColReduce{G + o.fc_b, nullptr, nullptr, slot, gemm_colsum_blocks(M),
                                  4 * C, 4 * C, 4 * C};
    }
    // With weight-gradient pairs on the second stream (216 CUs each, often
    // still running here), this product takes one workgroup per tile, so
    // that the CUs the pair leaves free keep working through its tiles.
    LAUNCH(gemm(dt, true, false, M, 4 * C, C, in, C, md->wt(o.fcp_w), 4 * C, e, s, nullptr, 0,
                md->side == nullptr));
    // fc: fch = ln2 fc_w^T + fc_b  (d4 holds d fch)
    LAUNCH(gemm(dt, true, false, M, C, 4 * C, d4, 4 * C, md->wt(o.fc_w), C,
                epi(EPI_STORE, md->dbuf_c, C), s));
    if (!fcb_fused) {
      void* slot = bg_part();
      LAUNCH(bias_grad(dt, G + o.fc_b, d4, M, 4 * C, 4 * C, slot, s, &md->cols.back()));
    }
    // mid = d res2 = d res3 + the LayerNorm-2 backward
    {
      void* slot = ln_part();
      TIMED(GPT2_TIMER_LN_BWD,
            layernorm_backward(dt, mid, in, G + o.ln2_w, G + o.ln2_b, G + o.proj_b, true,
                               md->dbuf_c, a.res2, a.ln2_mean, a.ln2_rstd, P + o.ln2_w, M, C,
                               slot, s, &md->cols.back()));
    }
    // attention output projection: res2 = x + atty proj_w^T + proj_b
    LAUNCH(gemm(dt, true, false, M, C, C, mid, C, md->wt(o.proj_w), C,
                epi(EPI_STORE, md->dbuf_c, C), s));
    // d qkv_b = column sums of dq: per 128-row block in the attention
    // backward where it can, else a pass over dq after the next product
    float* qkvb_part = nullptr;
    if (attention_colsum_ok(dt, md->hd)) {
      qkvb_part = (float*)bg_part();
      md->cols.back() = ColReduce{G + o.qkv_b, nullptr, nullptr, qkvb_part,
                                  attention_colsum_blocks(md->B, md->Tn), 3 * C, 3 * C, 3 * C};
    }
    TIMED(GPT2_TIMER_ATTN_BWD, attention_backward(dt, dq, md->dbuf_c, a.qkv, a.atty, a.lse,
                                                  md->B, md->Tn, H, md->hd, md->scratch, s,
                                                  qkvb_part));
    // qkv = ln1 qkv_w^T + qkv_b
    LAUNCH(gemm(dt, true, false, M, C, 3 * C, dq, 3 * C, md->wt(o.qkv_w), C,
                epi(EPI_STORE, md->dbuf_c, C), s));
    if (!qkvb_part) {
      void* slot = bg_part();
      LAUNCH(bias_grad(dt, G + o.qkv_b, dq, M, 3 * C, 3 * C, slot, s, &md->cols.back()));
    }
    // the layer's weight gradients dW += dy^T x
    const AccItem dw[4] = {
        {C, 4 * C, in, C, fchg, 4 * C, G + o.fcp_w, 4 * C},
        {4 * C, C, d4, 4 * C, ln2, C, G + o.fc_w, C},
        {C, C, mid, C, a.atty, C, G + o.proj_w, C},
        {3 * C, C, dq, 3 * C, ln1, C, G + o.qkv_w, C}};
    std::copy(dw, dw + 4, pend + npend);
    npend += 4;
    if (npend == 8) {
      if (gemm_acc_group_splits(dt, 8, pend, M) > 0) {  // both layers in one round of tiles
        if (on_side()) {  // beside the next layer's work
          SIDE_LAUNCH(8, (l + 1) % 3, l % 3);
        } else {
          TIMED(GPT2_TIMER_WGRAD, gemm_acc_group(dt, 8, pend, M, md->gemm_ws, md->gemm_ws_bytes, s));
        }
        npend = 0;
      } else {  // the layer above alone; this one waits for the next
        if (on_side()) {
          SIDE_LAUNCH(4, (l + 1) % 3, -1);
        } else {
          TIMED(GPT2_TIMER_WGRAD, gemm_acc_group(dt, 4, pend, M, md->gemm_ws, md->gemm_ws_bytes, s));
        }
        std::copy(pend + 4, pend + 8, pend);
        npend = 4;
      }
    }
    if (l == 0 && npend > 0) {
      if (npend == 4 && on_side()) {
        SIDE_LAUNCH(4, 0, -1);
      } else {
        TIMED(GPT2_TIMER_WGRAD, gemm_acc_group(dt, npend, pend, M, md->gemm_ws, md->gemm_ws_bytes, s));
      }
      npend = 0;
    }
    // d x = d res2 + the LayerNorm-1 backward, into the next layer's input
    // buffer (the next set), or for the first layer the embedding gradient
    if (l > 0) LAUNCH(guard((l - 1) % 3));
    void* dx = l > 0 ? md->bw_in[(l - 1) % 3] : md->dres;
    {
      void* slot = ln_part();
      TIMED(GPT2_TIMER_LN_BWD,
            layernorm_backward(dt, dx, mid, G + o.ln1_w, G + o.ln1_b,
                               l > 0 ? G + Ly.layers[l - 1].fcp_b : nullptr, true, md->dbuf_c,
                               xin, a.ln1_mean, a.ln1_rstd, P + o.ln1_w, M, C, slot, s,
                               &md->cols.back()));
    }
  }
#undef SIDE_LAUNCH
  LAUNCH(column_reduce_batched(md->cols.data(), (int)md->cols.size(), s));
  // embeddings
  LAUNCH(encoder_backward_wte(dt, G + Ly.wte, md->dres, md->tokens, M, C, md->V, md->scratch, s));
  LAUNCH(encoder_backward_wpe(dt, G + Ly.wpe, md->dres, md->B, md->Tn, C, s));
  // every weight gradient is in place before the backward returns (the side
  // stream's pairs write only the layers' matrices, none of the above)
  if (npairs > 0) LAUNCH(hipStreamWaitEvent(s, md->ev_done[npairs - 1], 0));
  return GPT2_OK;
}

int gpt2_sync(gpt2_model* md) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  HIP_TRY(hipStreamSynchronize(md->stream));
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(&flag, md->err_flag, sizeof(int), hipMemcpyDeviceToHost, md->stream));
  HIP_TRY(hipStreamSynchronize(md->stream));
  if (flag) {
    LAUNCH(fill_i32(md->err_flag, 0, 1, md->stream));
    HIP_TRY(hipStreamSynchronize(md->stream));
    return fail(GPT2_ETOKEN, "a token (bit 1) or target (bit 2) id was out of range: flags %d",
                flag);
  }
  return GPT2_OK;
}

int gpt2_clip_and_adamw(gpt2_model* md, float lr, float beta1, float beta2, float eps,
                        float weight_decay, float grad_clip, float* dev_norm_out) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (!(grad_clip > 0.f)) return fail(GPT2_EINVAL, "grad_clip must be > 0");
  hipStream_t s = md->stream;
  LAUNCH(grad_norm(md->grads, md->N, grad_clip, md->norm_scratch, dev_norm_out, s));
  const int64_t t = md->step + 1;
  const float bc1 = (float)(1.0 - std::pow((double)beta1, (double)t));
  const float bc2 = (float)(1.0 - std::pow((double)beta2, (double)t));
  TIMED(GPT2_TIMER_ADAMW,
        adamw(md->params, md->grads, md->m, md->v, md->dt == BF16 ? md->shadow : nullptr, md->N,
              lr, beta1, beta2, eps, weight_decay, bc1, bc2, grad_norm_result(md->norm_scratch),
              decay_map(md), s));
  float res[2] = {0.f, 0.f};
  HIP_TRY(hipMemcpyAsync(res, grad_norm_result(md->norm_scratch), sizeof(res),
                         hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  md->norm_ready = false;
  if (!std::isfinite(res[0])) {
    ++md->skips_nonfinite;
    return fail(GPT2_ENONFINITE, "gradient norm is %f: update skipped", (double)res[0]);
  }
  md->step = t;
  return gpt2_sync(md);
}

int gpt2_grad_norm(gpt2_model* md, float grad_clip, float* norm_out) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (!(grad_clip > 0.f)) return fail(GPT2_EINVAL, "grad_clip must be > 0");
  hipStream_t s = md->stream;
  LAUNCH(grad_norm(md->grads, md->N, grad_clip, md->norm_scratch, nullptr, s));
  float res[2] = {0.f, 0.f};
  HIP_TRY(hipMemcpyAsync(res, grad_norm_result(md->norm_scratch), sizeof(res),
                         hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  md->norm_ready = true;
  md->norm_value = res[0];
  if (norm_out) *norm_out = res[0];
  return GPT2_OK;
}

int gpt2_adamw_update(gpt2_model* md, float lr, float beta1, float beta2, float eps,
                      float weight_decay) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (!md->norm_ready)
    return fail(GPT2_ESTATE, "adamw_update needs gpt2_grad_norm after the last gradient change");
  md->norm_ready = false;
  if (!std::isfinite(md->norm_value)) {
    ++md->skips_nonfinite;
    return fail(GPT2_ENONFINITE, "gradient norm is %f: update skipped", (double)md->norm_value);
  }
  // the same launch as gpt2_clip_and_adamw, reading the norm and clip scale
  // gpt2_grad_norm left in the norm scratch
  const int64_t t = md->step + 1;
  const float bc1 = (float)(1.0 - std::pow((double)beta1, (double)t));
  const float bc2 = (float)(1.0 - std::pow((double)beta2, (double)t));
  TIMED(GPT2_TIMER_ADAMW,
        adamw(md->params, md->grads, md->m, md->v, md->dt == BF16 ? md->shadow : nullptr, md->N,
              lr, beta1, beta2, eps, weight_decay, bc1, bc2, grad_norm_result(md->norm_scratch),
              decay_map(md), md->stream));
  md->step = t;
  return GPT2_OK;
}

int gpt2_guarded_step(gpt2_model* md, gpt2_zscore* loss_z, gpt2_zscore* norm_z, float loss,
                      float z_max_loss, float z_max_norm, float lr, float beta1, float beta2,
                      float eps, float weight_decay, float grad_clip, float* norm_out,
                      double* zloss_out, double* znorm_out, int* skipped) {
  if (skipped) *skipped = 0;
  float norm = 0.f;
  int rc = gpt2_grad_norm(md, grad_clip, &norm);
  if (rc != GPT2_OK) return rc;
  if (norm_out) *norm_out = norm;
  double zl = std::nan(""), zn = std::nan("");
  if (loss_z && (rc = gpt2_zscore_update(loss_z, (double)loss, &zl)) != GPT2_OK) return rc;
  if (norm_z && (rc = gpt2_zscore_update(norm_z, (double)norm, &zn)) != GPT2_OK) return rc;
  if (zloss_out) *zloss_out = zl;
  if (znorm_out) *znorm_out = zn;
  if (!std::isfinite(norm)) {
    md->norm_ready = false;
    ++md->skips_nonfinite;
    if (skipped) *skipped = 1;
    return fail(GPT2_ENONFINITE, "gradient norm is %f: update skipped", (double)norm);
  }
  // a spike upwards is the instability; NaN z-scores (no history yet) never trigger
  const bool outlier = (loss_z && z_max_loss > 0.f && zl > z_max_loss) ||
                       (norm_z && z_max_norm > 0.f && zn > z_max_norm);
  if (outlier) {
    md->norm_ready = false;
    ++md->skips_outlier;
    if (skipped) *skipped = 1;
    return GPT2_OK;
  }
  rc = gpt2_adamw_update(md, lr, beta1, beta2, eps, weight_decay);
  if (rc != GPT2_OK) return rc;
  return gpt2_sync(md);
}

int gpt2_skip_counts(gpt2_model* md, int64_t* nonfinite, int64_t* outlier) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (nonfinite) *nonfinite = md->skips_nonfinite;
  if (outlier) *outlier = md->skips_outlier;
  return GPT2_OK;
}

namespace {

// Checkpoint file: this header, then params, m, v (num_params floats each).
struct CkptHeader {
  char magic[8];
  uint32_t version, header_bytes;
  int32_t n_layer, n_head, n_embd, block_size, vocab_size, padded_vocab_size;
  int32_t dtype, reserved0;
  int64_t num_params, step, skips_nonfinite, skips_outlier;
  int64_t reserved1[2];
};
static_assert(sizeof(CkptHeader) == 96, "checkpoint header layout");
constexpr char kCkptMagic[8] = {'G', 'P', 'T', '2', 'C', 'K', 'P', 'T'};
constexpr uint32_t kCkptVersion = 1;
constexpr size_t kCkptChunk = size_t(64) << 20;  // bytes staged through host memory at a time

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) std::fclose(f);
  }
};

}  // namespace

int gpt2_save_state(gpt2_model* md, const char* path) {
  if (!md || !path) return fail(GPT2_EINVAL, "NULL argument");
  hipStream_t s = md->stream;
  HIP_TRY(hipStreamSynchronize(s));
  CkptHeader h{};
  std::memcpy(h.magic, kCkptMagic, 8);
  h.version = kCkptVersion;
  h.header_bytes = sizeof(CkptHeader);
  h.n_layer = md->cfg.n_layer;
  h.n_head = md->cfg.n_head;
  h.n_embd = md->cfg.n_embd;
  h.block_size = md->cfg.block_size;
  h.vocab_size = md->cfg.vocab_size;
  h.padded_vocab_size = md->cfg.padded_vocab_size;
  h.dtype = md->cfg.dtype;
  h.num_params = md->N;
  h.step = md->step;
  h.skips_nonfinite = md->skips_nonfinite;
  h.skips_outlier = md->skips_outlier;
  File fh;
  fh.f = std::fopen(path, "wb");
  if (!fh.f) return fail(GPT2_EINVAL, "cannot open %s for writing", path);
  if (std::fwrite(&h, sizeof(h), 1, fh.f) != 1) return fail(GPT2_EINVAL, "write to %s failed", path);
  std::vector<char> buf(kCkptChunk);
  for (const float* src : {md->params, md->m, md->v}) {
    const size_t total = (size_t)md->N * sizeof(float);
    for (size_t off = 0; off < total; off += kCkptChunk) {
      const size_t n = std::min(kCkptChunk, total - off);
      HIP_TRY(hipMemcpyAsync(buf.data(), (const char*)src + off, n, hipMemcpyDeviceToHost, s));
      HIP_TRY(hipStreamSynchronize(s));
      if (std::fwrite(buf.data(), 1, n, fh.f) != n) return fail(GPT2_EINVAL, "write to %s failed", path);
    }
  }
  FILE* f = fh.f;
  fh.f = nullptr;
  if (std::fclose(f) != 0) return fail(GPT2_EINVAL, "closing %s failed", path);
  return GPT2_OK;
}

int gpt2_load_state(gpt2_model* md, const char* path) {
  if (!md || !path) return fail(GPT2_EINVAL, "NULL argument");
  File fh;
  fh.f = std::fopen(path, "rb");
  if (!fh.f) return fail(GPT2_EINVAL, "cannot open %s", path);
  CkptHeader h{};
  if (std::fread(&h, sizeof(h), 1, fh.f) != 1) return fail(GPT2_EINVAL, "%s: short header", path);
  if (std::memcmp(h.magic, kCkptMagic, 8) != 0 || h.version != kCkptVersion ||
      h.header_bytes != sizeof(CkptHeader))
    return fail(GPT2_EINVAL, "%s is not a version-%u checkpoint", path, kCkptVersion);
  const gpt2_config& c = md->cfg;
  if (h.n_layer != c.n_layer || h.n_head != c.n_head || h.n_embd != c.n_embd ||
      h.block_size != c.block_size || h.vocab_size != c.vocab_size ||
      h.padded_vocab_size != c.padded_vocab_size || h.num_params != md->N)
    return fail(GPT2_EINVAL, "%s holds a model of another shape", path);
  if (h.step < 0) return fail(GPT2_EINVAL, "%s: negative step count", path);
  hipStream_t s = md->stream;
  HIP_TRY(hipStreamSynchronize(s));
  std::vector<char> buf(kCkptChunk);
  for (float* dst : {md->params, md->m, md->v}) {
    const size_t total = (size_t)md->N * sizeof(float);
    for (size_t off = 0; off < total; off += kCkptChunk) {
      const size_t n = std::min(kCkptChunk, total - off);
      if (std::fread(buf.data(), 1, n, fh.f) != n) return fail(GPT2_EINVAL, "%s is short", path);
      HIP_TRY(hipMemcpyAsync((char*)dst + off, buf.data(), n, hipMemcpyHostToDevice, s));
      HIP_TRY(hipStreamSynchronize(s));
    }
  }
  if (md->dt == BF16) LAUNCH(cast_f32_to_bf16(md->shadow, md->params, md->N, s));
  LAUNCH(fill_f32(md->grads, 0.f, md->N, s));
  HIP_TRY(hipStreamSynchronize(s));
  md->step = h.step;
  md->skips_nonfinite = h.skips_nonfinite;
  md->skips_outlier = h.skips_outlier;
  md->norm_ready = false;
  md->have_targets = false;
  return GPT2_OK;
}

int gpt2_set_kernel_timer(gpt2_model* md, int which, int max_launches) {
  if (!md) return fail(GPT2_EINVAL, "NULL model");
  if (which < GPT2_TIMER_NONE || which > GPT2_TIMER_LN_BWD)
    return fail(GPT2_EINVAL, "unknown timer %d", which);
  if (which != GPT2_TIMER_NONE && (max_launches < 1 || max_launches > (1 << 20)))
    return fail(GPT2_EINVAL, "max_launches must be in [1, 2^20]");
  HIP_TRY(hipStreamSynchronize(md->stream));
  if (md->side) HIP_TRY(hipStreamSynchronize(md->side));
  release_timer(md);
  if (which == GPT2_TIMER_NONE) return GPT2_OK;
  md->timer_ev.resize(2 * (size_t)max_launches);
  for (size_t i = 0; i < md->timer_ev.size(); ++i) {
    hipError_t e = hipEventCreate(&md->timer_ev[i]);
    if (e != hipSuccess) {
      md->timer_ev.resize(i);
      release_timer(md);
      return fail(GPT2_EHIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  md->timer_which = which;
  md->timer_cap = max_launches;
  return GPT2_OK;
}

int gpt2_read_kernel_timer(gpt2_model* md, int* launches, double* total_ms) {
  if (!md || !launches || !total_ms) return fail(GPT2_EINVAL, "NULL argument");
  HIP_TRY(hipStreamSynchronize(md->stream));
  if (md->side) HIP_TRY(hipStreamSynchronize(md->side));
  double sum = 0.0;
  for (int i = 0; i < md->timer_used; ++i) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, md->timer_ev[2 * i], md->timer_ev[2 * i + 1]));
    sum += ms;
  }
  *launches = md->timer_used;
  *total_ms = sum;
  md->timer_used = 0;
  return GPT2_OK;
}

int gpt2_debug_read(gpt2_model* md, int which, int layer, void* dst, size_t bytes) {
  if (!md || !dst) return fail(GPT2_EINVAL, "NULL argument");
  const size_t es = dsize(md->dt);
  const int64_t M = md->M, C = md->C;
  const void* src = nullptr;
  size_t n = 0;
  auto need_layer = [&]() { return layer >= 0 && layer < md->L; };
  switch (which) {
    case GPT2_DBG_LOGITS:
      if (!md->logits) return fail(GPT2_EINVAL, "fused_head keeps no logits");
      src = md->logits;
      n = M * md->ldl * es;
      break;
    case GPT2_DBG_LOSSES: src = md->losses; n = M * 4; break;
    case GPT2_DBG_ARGMAX:
      if (md->fused_head) return fail(GPT2_EINVAL, "fused_head computes no argmax");
      src = md->argmax;
      n = M * 4;
      break;
    case GPT2_DBG_ACT_LNF: src = md->lnf; n = M * C * es; break;
    case GPT2_DBG_ENCODED: src = md->encoded; n = M * C * es; break;
    case GPT2_DBG_ACT_LN1:
    case GPT2_DBG_ACT_QKV:
    case GPT2_DBG_ACT_ATTY:
    case GPT2_DBG_ACT_RES2:
    case GPT2_DBG_ACT_FCH:
    case GPT2_DBG_ACT_RES3:
    case GPT2_DBG_ATT_LSE: {
      if (!need_layer()) return fail(GPT2_EINVAL, "layer %d out of range", layer);
      const LayerAct& a = md->act[layer];
      if (which == GPT2_DBG_ACT_LN1) {
        if (!a.ln1) return fail(GPT2_EINVAL, "ln1 outputs are not kept with recompute = 2");
        src = a.ln1;
        n = M * C * es;
      }
      if (which == GPT2_DBG_ACT_QKV) { src = a.qkv; n = M * 3 * C * es; }
      if (which == GPT2_DBG_ACT_ATTY) { src = a.atty; n = M * C * es; }
      if (which == GPT2_DBG_ACT_RES2) { src = a.res2; n = M * C * es; }
      if (which == GPT2_DBG_ACT_FCH) { src = a.fch; n = M * 4 * C * es; }
      if (which == GPT2_DBG_ACT_RES3) { src = a.res3; n = M * C * es; }
      if (which == GPT2_DBG_ATT_LSE) { src = a.lse; n = (size_t)md->B * md->H * md->Tn * 4; }
      break;
    }
    default: return fail(GPT2_EINVAL, "unknown debug buffer %d", which);
  }
  if (bytes < n) return fail(GPT2_EINVAL, "destination holds %zu bytes, need %zu", bytes, n);
  HIP_TRY(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, md->stream));
  return GPT2_OK;
}

}  // extern "C"
