/*
 * gpt2.h -- C ABI of libgpt2.so: one GPT-2 pretraining step on one AMD
 * Instinct MI355X (gfx950), every step in hand-written HIP kernels.
 *
 * What is computed (the web pages this method comes from are cited by title
 * and section):
 *   - Model: decoder-only GPT-2 -- learned token (wte) and position (wpe)
 *     embeddings, pre-LayerNorm blocks of causal multi-head self-attention and
 *     a 4C GELU MLP with residual connections, a final LayerNorm, and an
 *     output head tied to wte (news post on Karpathy's 4-hour GPT-2 124M
 *     lecture, rgzn1.com, lecture outline; qntz.me "From 0 to 1 build GPT",
 *     section on building the Transformer; "Let's reproduce GPT-2 (124M)"
 *     notes, training-recipe section: weight tying).
 *   - Loss: mean cross-entropy over B*T positions, vocabulary padded (e.g.
 *     50257 -> 50304, "Let's reproduce GPT-2 (124M)", GPU optimisation
 *     ladder, "nice numbers") with the padded logits excluded.
 *   - Gradient accumulation over k micro-steps with the loss divided by k,
 *     global gradient-norm clipping, and AdamW with weight decay on 2-D
 *     tensors only ("Let's reproduce GPT-2 (124M)", training recipe;
 *     dszhyy.com llm.c 1.5B post, flags section).
 *   - LayerNorm eps 1e-5 (GPT2Config block on the dszhyy.com page).
 *
 * Conventions for every call:
 *   - Pointers named dev_* are device pointers; everything else is host.
 *   - Memory is owned by the caller.  The caller allocates one device
 *     workspace of gpt2_workspace_bytes() bytes and passes it, together
 *     with a HIP stream, to gpt2_create; the library never allocates or
 *     frees device memory and never frees caller memory.  gpt2_destroy
 *     frees only the host handle.
 *   - Every call enqueues work on the model's stream and returns without
 *     waiting, except gpt2_clip_and_adamw and gpt2_sync, which wait for the
 *     stream.  A handle must be used from one host thread at a time.
 *   - Return value: GPT2_OK (0) or a negative GPT2_E* code; the text of the
 *     last error on the calling thread is returned by gpt2_last_error().
 *
 * Data layout:
 *   - Parameters form one flat fp32 vector in the order of
 *     gpt2_param_layout(): wte (Vp, C), wpe (block_size, C), then for each
 *     layer ln1_w, ln1_b (C), qkv_w (3C, C), qkv_b (3C), proj_w (C, C),
 *     proj_b (C), ln2_w, ln2_b (C), fc_w (4C, C), fc_b (4C), fcp_w (C, 4C),
 *     fcp_b (C); last lnf_w, lnf_b (C).  Linear weights are (out, in),
 *     row-major, applied as y = x W^T + b.  qkv columns are [q | k | v],
 *     head h at columns h*hd .. (h+1)*hd - 1 within each third.
 *   - Gradients, AdamW m and v use the same flat layout, fp32.
 *   - Tokens and targets are int32, row-major (B, T).
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GPT2_OK = 0,
  GPT2_EINVAL = -1,      /* bad config, null pointer, or shape mismatch */
  GPT2_EWORKSPACE = -2,  /* workspace too small or misaligned (256 B) */
  GPT2_ESTATE = -3,      /* call out of order, e.g. backward before a forward with targets */
  GPT2_ETOKEN = -4,      /* a token or target id was outside [0, vocab_size) */
  GPT2_ENONFINITE = -5,  /* gradient norm NaN/Inf: update skipped, state unchanged */
  GPT2_EHIP = -6         /* a HIP runtime call failed; see gpt2_last_error() */
};

enum { GPT2_FP32 = 0, GPT2_BF16 = 1 };

typedef struct {
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;            /* C; multiple of 64 */
  int32_t block_size;        /* rows of wpe; seq_len <= block_size */
  int32_t vocab_size;        /* V: ids in [0, V) */
  int32_t padded_vocab_size; /* Vp >= V: rows of wte, columns of the logits */
  int32_t micro_batch;       /* B */
  int32_t seq_len;           /* T */
  int32_t grad_accum_steps;  /* k: backward scales the loss by 1/k */
  int32_t dtype;             /* GPT2_FP32 or GPT2_BF16 (activations + GEMM inputs) */
  int32_t deterministic;     /* accepted either way: no kernel uses floating-point atomics and
                                every reduction runs in a fixed order, so a step is bitwise
                                repeatable for a given config and device */
  float ln_eps;              /* LayerNorm eps, 1e-5 */
  int32_t recompute;         /* activations the backward regenerates instead of keeping one per
                                layer (dszhyy.com llm.c 1.5B post, flags -r 1 / -r 2):
                                0 none; 1 the GELU output (rewritten by the GELU-backward
                                product from the kept pre-activation); 2 also the two
                                LayerNorm outputs of each block (rerun from the kept block
                                inputs).  Results are bit-identical across the three. */
  int32_t fused_head;        /* 0: the forward stores the B*T x Vp logits and, with the loss,
                                their gradient (2 x 1.65 GB at GPT-2 124M, B x T = 16 x 1024).
                                1: neither is ever stored (the fused classifier carried to the
                                head's products; dszhyy.com llm.c 1.5B post, PyTorch-comparison
                                section): the forward takes the loss from per-row softmax
                                statistics of the head's product, and the backward
                                recomputes the product 4608 vocabulary columns at a time,
                                turning each block straight into its logit gradient for the
                                two gradient products (one more head-sized product per
                                micro-step).  Needs bf16, padded_vocab_size a multiple of 64
                                and >= 256, micro_batch * seq_len >= 256; then gpt2_forward
                                requires targets and GPT2_DBG_LOGITS / GPT2_DBG_ARGMAX
                                return GPT2_EINVAL.  The gradients match mode 0's to bf16
                                rounding (not bit for bit: the log-sum-exp is combined in
                                another order). */
} gpt2_config;

typedef struct {
  char name[32];     /* e.g. "wte", "h3.qkv_w", "lnf_b" */
  int64_t offset;    /* element offset in the flat vector */
  int32_t ndim;      /* 1 or 2 */
  int32_t decay;     /* 1 if AdamW weight decay applies (2-D tensors) */
  int64_t shape[2];  /* shape[1] == 1 when ndim == 1 */
} gpt2_tensor_info;

typedef struct gpt2_model gpt2_model;

/* Bytes of device workspace a model with this config needs (0 if the config
 * is invalid; the reason is in gpt2_last_error()). */
size_t gpt2_workspace_bytes(const gpt2_config* cfg);

/* Number of parameters, Vp*C + block_size*C + L*(12C^2 + 13C) + 2C
 * (wte counted once, lm_head tied).  -1 on an invalid config. */
int64_t gpt2_num_params(const gpt2_config* cfg);

/* Fills up to cap entries of out with the flat parameter layout and returns
 * the number of tensors (2 + 12 L + 2), or a negative error code.  out may be
 * NULL to query the count.  Host only; needs no GPU. */
int gpt2_param_layout(const gpt2_config* cfg, gpt2_tensor_info* out, int cap);

/* Creates a model over dev_workspace (>= gpt2_workspace_bytes, 256-byte
 * aligned, owned by the caller, must outlive the model) on the HIP stream
 * hip_stream (a hipStream_t; NULL = default stream).  Parameters, gradients,
 * m, v and the step count start at zero.  Synchronous. */
int gpt2_create(const gpt2_config* cfg, void* dev_workspace, size_t bytes, void* hip_stream,
                gpt2_model** out);
int gpt2_destroy(gpt2_model* model);

/* Copy the fp32 flat parameter vector in (also refreshes the bf16 copy used
 * by the bf16 GEMMs) or out.  dev_* hold gpt2_num_params() floats. */
int gpt2_set_params(gpt2_model* model, const float* dev_src);
int gpt2_get_params(gpt2_model* model, float* dev_dst);
/* Copy the accumulated fp32 gradient vector out or in. */
int gpt2_get_grads(gpt2_model* model, float* dev_dst);
int gpt2_set_grads(gpt2_model* model, const float* dev_src);
/* AdamW state: first and second moments (flat fp32) and the number of
 * updates applied so far. */
int gpt2_get_opt_state(gpt2_model* model, float* dev_m, float* dev_v, int64_t* step);
int gpt2_set_opt_state(gpt2_model* model, const float* dev_m, const float* dev_v, int64_t step);

/* Forward pass on dev_tokens (B, T): embeddings, the pre-LayerNorm blocks,
 * the final LayerNorm and the tied head over the padded vocabulary (qntz.me
 * "From 0 to 1 build GPT", building the Transformer; "Let's reproduce GPT-2
 * (124M)" notes, training recipe: weight tying; GPU optimisation ladder:
 * vocabulary 50257 -> 50304).  With dev_targets (B, T) non-NULL it also
 * evaluates the cross-entropy and writes the mean over the B*T positions
 * (not divided by k) to dev_loss (one float; may be NULL).
 * Out-of-range ids are clamped for memory safety and reported as
 * GPT2_ETOKEN by the next gpt2_sync / gpt2_clip_and_adamw. */
int gpt2_forward(gpt2_model* model, const int32_t* dev_tokens, const int32_t* dev_targets,
                 float* dev_loss);

/* Evaluation forward: the loss of gpt2_forward with targets (dev_targets
 * required; mean written to dev_loss, may be NULL; per-position losses
 * readable as GPT2_DBG_LOSSES) without materialising the B*T x Vp logits:
 * in bf16 the tied head's product leaves only each row's (max, sum of
 * exponentials) per 128 vocabulary columns and the target's logit, which
 * one more pass combines into log-sum-exp and loss (the extension of the
 * fused classifier that never stores the logits; dszhyy.com llm.c 1.5B
 * post, PyTorch-comparison section).  In fp32, or for shapes the large
 * tiles do not cover, the logits are computed and the loss taken from them.
 * Neither the logits nor their gradient are left for reading, and a
 * following gpt2_backward returns GPT2_ESTATE.  Ids as in gpt2_forward. */
int gpt2_forward_loss(gpt2_model* model, const int32_t* dev_tokens, const int32_t* dev_targets,
                      float* dev_loss);

/* Backward pass of the last forward (which must have had targets):
 * gradients += d(mean loss / k) / d params, the micro-step's share under
 * gradient accumulation ("Let's reproduce GPT-2 (124M)" notes, training
 * recipe: the loss is divided by the number of accumulation steps; the tied
 * wte gets both its head and its embedding gradient).  The logit gradient comes from
 * the forward's cross-entropy (computed with the loss, from the same read of
 * the logits); the logits themselves are left as the forward wrote them.
 * With fused_head = 1 it is regenerated here instead (see gpt2_config).
 * The forward's dev_tokens are read again here (the embedding gradient);
 * its targets are kept by the model. */
int gpt2_backward(gpt2_model* model);

/* Gradients = 0: the start of an optimizer step's k accumulated micro-steps
 * ("Let's reproduce GPT-2 (124M)" notes, training recipe: gradient
 * accumulation). */
int gpt2_zero_grad(gpt2_model* model);

/* One optimizer step ("Let's reproduce GPT-2 (124M)", training recipe):
 * n = ||g||_2 over all gradients; s = min(1, grad_clip / n); g' = s g;
 * t += 1; m = b1 m + (1-b1) g'; v = b2 v + (1-b2) g'^2;
 * p -= lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd p [2-D tensors]).
 * Writes n to dev_norm_out (may be NULL).  Waits for the stream; returns
 * GPT2_ENONFINITE (nothing updated, t unchanged) if n is NaN or Inf, and
 * GPT2_ETOKEN if an id since the last check was out of range. */
int gpt2_clip_and_adamw(gpt2_model* model, float lr, float beta1, float beta2, float eps,
                        float weight_decay, float grad_clip, float* dev_norm_out);

/* Waits for the model's stream and reports pending device-side errors. */
int gpt2_sync(gpt2_model* model);

/* ---- Training-loop robustness.  The llm.c GPT-2 1.5B post (dszhyy.com)
 * shows a training log with the z-score of the loss and of the gradient
 * norm at every step (setup section), flags that save a checkpoint every n
 * steps and resume a crashed run with bit-identical results (flags
 * section), and a restart that skips an update whose loss or norm z-score
 * exceeds 5 (400B-token run section).  These calls provide those pieces. */

/* Rolling z-score detector over the last `window` finite values of a
 * series, 2 <= window <= 65536 (host only, no GPU calls).
 * gpt2_zscore_update sets *z_out to (x - mean) / std of the values held
 * before x (population std, double precision), or NaN while fewer than
 * `window` values are held, when x is not finite, or when std is 0; then it
 * adds x if x is finite (the oldest value leaves).  z_out may be NULL. */
typedef struct gpt2_zscore gpt2_zscore;
int gpt2_zscore_create(int window, gpt2_zscore** out);
int gpt2_zscore_update(gpt2_zscore* detector, double x, double* z_out);
int gpt2_zscore_destroy(gpt2_zscore* detector);

/* A detector's state, for checkpoints of a guarded run: the values it
 * holds, oldest first.  gpt2_zscore_get_state writes the window size and
 * the number of values held (either pointer may be NULL) and, if `values`
 * is non-NULL, the values (cap must be >= that number).
 * gpt2_zscore_set_state replaces the held values with `count` values,
 * oldest first (0 <= count <= window, all finite); updates then continue
 * exactly as in the detector the values came from.  EINVAL otherwise. */
int gpt2_zscore_get_state(const gpt2_zscore* detector, double* values, int cap, int* window,
                          int* count);
int gpt2_zscore_set_state(gpt2_zscore* detector, const double* values, int count);

/* The optimizer step of gpt2_clip_and_adamw in two calls.  gpt2_grad_norm
 * computes the global L2 norm of the gradients and the clip scale
 * min(1, grad_clip / norm), waits, and returns the norm in *norm_out (host,
 * may be NULL).  gpt2_adamw_update then applies clipping and AdamW with
 * that norm exactly as gpt2_clip_and_adamw does (same result bit for bit).
 * gpt2_adamw_update returns GPT2_ESTATE unless gpt2_grad_norm ran after the
 * last change of the gradients (backward, zero_grad, set_grads,
 * load_state), and GPT2_ENONFINITE (nothing updated, counted) when that
 * norm was not finite.  gpt2_adamw_update does not wait. */
int gpt2_grad_norm(gpt2_model* model, float grad_clip, float* norm_out);
int gpt2_adamw_update(gpt2_model* model, float lr, float beta1, float beta2, float eps,
                      float weight_decay);

/* One guarded optimizer step: gpt2_grad_norm, the z-scores of `loss` in
 * loss_z and of the norm in norm_z (gpt2_zscore_update: both values join
 * their windows), then gpt2_adamw_update unless the norm is not finite
 * (GPT2_ENONFINITE) or a z-score exceeds its threshold -- z_max_loss,
 * z_max_norm; a detector that is NULL or a threshold <= 0 is not checked,
 * a NaN z-score never triggers.  An outlier skip returns GPT2_OK with
 * *skipped = 1; both kinds of skip leave parameters, m, v and the step
 * count unchanged and are counted (gpt2_skip_counts).  norm_out, zloss_out,
 * znorm_out and skipped may be NULL.  Waits for the stream. */
int gpt2_guarded_step(gpt2_model* model, gpt2_zscore* loss_z, gpt2_zscore* norm_z, float loss,
                      float z_max_loss, float z_max_norm, float lr, float beta1, float beta2,
                      float eps, float weight_decay, float grad_clip, float* norm_out,
                      double* zloss_out, double* znorm_out, int* skipped);

/* Updates skipped since the model was created or loaded: for a non-finite
 * gradient norm (here, in gpt2_clip_and_adamw and gpt2_adamw_update) and
 * for a z-score outlier (gpt2_guarded_step).  Either pointer may be NULL. */
int gpt2_skip_counts(gpt2_model* model, int64_t* nonfinite, int64_t* outlier);

/* Checkpoints.  gpt2_save_state writes the fp32 parameters, AdamW m and v,
 * the step count, the skip counts and the shape of the model to the file
 * `path` (binary, native byte order: a 96-byte header, then params, m, v as
 * num_params floats each).  gpt2_load_state reads such a file into a model
 * of the same shape (n_layer, n_head, n_embd, block_size, vocab_size,
 * padded_vocab_size; the dtype and batch shape may differ), refreshes the
 * bf16 parameter copy and zeroes the gradients.  A run resumed from a
 * checkpoint taken between optimizer steps, fed the same micro-batches,
 * reproduces the uninterrupted run bit for bit: the file holds all the
 * model's state that carries from one step to the next.  The z-score
 * detectors of gpt2_guarded_step are the caller's host objects and are not
 * in the file: a guarded run resumes bit for bit when their windows are
 * saved and restored beside it (gpt2_zscore_get_state / set_state).  EINVAL: the file cannot be opened, read or
 * written, is short, has another magic or version, or another shape.  Both
 * wait for the stream. */
int gpt2_save_state(gpt2_model* model, const char* path);
int gpt2_load_state(gpt2_model* model, const char* path);

/* Debug / test reads of internal buffers (copied on the stream into dev_dst,
 * which must hold `bytes`).  which = GPT2_DBG_*; layer used by per-layer
 * buffers.  Element types: LOGITS, ACT_* in the activation dtype (fp32 or
 * bf16, row pitch listed below); LSE, LOSSES fp32; ARGMAX int32. */
enum {
  GPT2_DBG_LOGITS = 0,   /* (B*T, Vp) logits of the last forward, row pitch Vp */
  GPT2_DBG_LOSSES = 1,   /* (B*T) per-position cross-entropy */
  GPT2_DBG_ARGMAX = 2,   /* (B*T) argmax over the unpadded vocab, lowest index on ties */
  GPT2_DBG_ACT_LN1 = 3,  /* (B*T, C) ln1 output of `layer` (EINVAL with recompute = 2) */
  GPT2_DBG_ACT_QKV = 4,  /* (B*T, 3C) */
  GPT2_DBG_ACT_ATTY = 5, /* (B*T, C) attention output before the projection */
  GPT2_DBG_ACT_RES2 = 6, /* (B*T, C) residual after attention */
  GPT2_DBG_ACT_FCH = 7,  /* (B*T, 4C) fc pre-activation h; with recompute 0 (GELU(h) kept)
                            GELU'(h) instead, the only form of it the backward reads */
  GPT2_DBG_ACT_RES3 = 8, /* (B*T, C) residual after the MLP (block output) */
  GPT2_DBG_ACT_LNF = 9,  /* (B*T, C) final LayerNorm output */
  GPT2_DBG_ATT_LSE = 10, /* (B, H, T) fp32 log-sum-exp of the scaled scores */
  GPT2_DBG_ENCODED = 11  /* (B*T, C) wte[tok] + wpe[t] */
};
int gpt2_debug_read(gpt2_model* model, int which, int layer, void* dev_dst, size_t bytes);

/* Measurement hook: when set, the library records a HIP event pair on its
 * stream around every launch of the chosen step, for up to max_launches
 * launches (further launches run untimed).  The events are created here
 * (host-side objects; no device memory is allocated), so set the timer
 * outside a timed region.  which = GPT2_TIMER_NONE releases the events.
 * Waits for the stream first.  EINVAL on an unknown `which` or
 * max_launches outside [1, 2^20]; EHIP if event creation fails.
 *   LM_HEAD_FWD  the tied-head logits GEMM of each forward
 *   ATTN_FWD     causal attention forward, one pair per layer
 *   ATTN_BWD     attention backward (both of its kernels), one pair per layer
 *   CE_FWD       the fused softmax cross-entropy of each forward with targets
 *                (loss, lse, argmax and the logit gradient)
 *   ADAMW        the AdamW update of each optimizer step (not the norm)
 *   WGRAD        each grouped launch of the layers' weight gradients (the
 *                four products of one layer, or of two layers as one
 *                launch), on the stream it runs on (the library's second
 *                stream for most two-layer launches)
 *   LN_FWD       every LayerNorm forward of the forward pass
 *   LN_BWD       every LayerNorm backward of the backward pass */
enum {
  GPT2_TIMER_NONE = 0,
  GPT2_TIMER_LM_HEAD_FWD = 1,
  GPT2_TIMER_ATTN_FWD = 2,
  GPT2_TIMER_ATTN_BWD = 3,
  GPT2_TIMER_CE_FWD = 4,
  GPT2_TIMER_ADAMW = 5,
  GPT2_TIMER_WGRAD = 6,
  GPT2_TIMER_LN_FWD = 7,
  GPT2_TIMER_LN_BWD = 8
};
int gpt2_set_kernel_timer(gpt2_model* model, int which, int max_launches);

/* Waits for the streams, then reports how many launches were timed since the
 * timer was set or last read (*launches) and the sum of their event-pair
 * durations in milliseconds (*total_ms), and restarts the count. */
int gpt2_read_kernel_timer(gpt2_model* model, int* launches, double* total_ms);

/* Message of the last failed call on this thread ("" if none). */
const char* gpt2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_H */
