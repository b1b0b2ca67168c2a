/*
 * lmstep.h - C ABI of the MI355X (gfx950) training-step library.
 *
 * One training step of a pre-LayerNorm decoder-only transformer, as the pages
 * on building GPT-style models without a framework describe it:
 *   - token embedding plus a learned positional embedding added directly
 *     (Feste page, "Model Architecture");
 *   - blocks of LayerNorm -> causal multi-head self-attention (future
 *     positions masked with -inf before the softmax) -> residual, then
 *     LayerNorm -> GELU MLP -> residual; a final LayerNorm (Feste page,
 *     "Model Architecture"; RustGPT page, file list: layer_norm, self_attention,
 *     feed_forward);
 *   - the vocabulary projection with softmax cross-entropy (RustGPT page,
 *     technical-implementation list; Smallem page, "Ce qu'est un modele de
 *     langage": V probabilities that sum to 1);
 *   - a hand-derived backward pass and AdamW with decoupled weight decay and
 *     global L2 gradient clipping (Feste page, "Manual Backpropagation";
 *     RustGPT page: clip to an L2 norm of 5.0);
 *   - optional packing of several documents per row (LucilleAI page, "what
 *     makes it special": sequence packing), with a block-diagonal causal mask.
 *
 * Readings fixed by this library where the pages are silent: GELU is the tanh
 * form 0.5u(1 + tanh(sqrt(2/pi)(u + 0.044715u^3))); LayerNorm uses the biased
 * variance; the attention scale is 1/sqrt(D); positions restart at 0 in every
 * packed document; the vocabulary projection is tied to wte and has no bias
 * unless untied_head asks for a separate one with a bias (RustGPT page, file
 * list: its output projection is a layer of its own);
 * the loss is the mean over positions whose target is >= 0; the clip factor is
 * clip/n only when the global norm n exceeds clip; weight decay applies to
 * every parameter as lr*wd*p on the pre-update p.
 *
 * Conventions
 *   - Every call returns lm_status (0 = LM_OK). On error lm_last_error()
 *     returns a thread-local message. No C++ exception crosses this ABI.
 *   - "d_" pointers are device pointers (hipMalloc'd or torch CUDA memory);
 *     "stream" is a hipStream_t passed as void*. NULL means the null stream.
 *   - The library never allocates device memory: the caller passes one arena
 *     of lm_workspace_bytes() bytes (256-byte aligned) to model_create and
 *     keeps it alive until model_destroy. The library owns only the opaque
 *     host-side lm_model.
 *   - train_step and forward_logits only enqueue work on the stream; they
 *     return before the GPU finishes. Host-checkable argument errors are
 *     returned before anything is enqueued. Inputs must stay valid until the
 *     stream's work completes. One exception: a 16-bit model whose blocks'
 *     weight gradients run as one grouped launch (wide enough models, steps
 *     of at least 2048 tokens; the vocabulary projection's weight gradient
 *     joins it where that takes fewer rounds of the compute units than two
 *     launches) uploads that launch's table of GEMMs when a
 *     step's token count B*T differs from the previous such step's, and
 *     first synchronizes the stream (so such a step cannot be captured into
 *     a HIP graph; steps at an unchanged token count can).
 *   - A model is not thread-safe; separate models are independent.
 */
#ifndef LMSTEP_H
#define LMSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LM_OK = 0,
  LM_ERR_ARG = -1,         /* null pointer or out-of-range argument        */
  LM_ERR_WORKSPACE = -2,   /* arena too small or misaligned                */
  LM_ERR_SHAPE = -3,       /* B > max_batch, T > max_seq, bad model dims    */
  LM_ERR_HIP = -4,         /* a HIP runtime call failed                    */
  LM_ERR_UNSUPPORTED = -5  /* valid but not implemented (e.g. head dim 48) */
} lm_status;

/* Model dimensions. d_model must be a multiple of 128 (at most 1024) and of
 * n_heads; the head dimension d_model / n_heads must be 32 or 64; d_mlp a
 * multiple of 64; max_batch * max_seq at most 2^24, and small enough that
 * every 16-bit GEMM operand of a step (the largest is the vocabulary-wide
 * logits, max_batch * max_seq * round_up(vocab, 128) values) spans less than
 * 2 GiB: lm_workspace_bytes returns 0 and model_create LM_ERR_UNSUPPORTED
 * otherwise.
 * precision: 0 = fp32 everywhere; 1 = bf16 GEMM/attention operands with fp32
 * accumulation, fp32 residual stream, statistics, loss, gradients, Adam
 * moments and master weights; 2 = the same with fp16 operands and dynamic
 * loss scaling (LucilleAI page: FP16 autocast with a GradScaler): the loss
 * gradient is multiplied by a scale S, the gradients are divided by S before
 * the clip and the update, and a step whose gradients overflow (non-finite
 * norm) is skipped and S multiplied by the backoff factor (lm_loss_scaler).
 * untied_head: 0 = logits z = h_f wte^T (tied, no bias); 1 = z = h_f
 * head.w^T + head.b with a separate head.w [V,C] and head.b [V]. */
typedef struct {
  int32_t vocab, d_model, n_heads, d_mlp, n_layers, max_seq, max_batch;
  int32_t precision;
  float ln_eps; /* LayerNorm epsilon, e.g. 1e-5 */
  int32_t untied_head;
} lm_config;

/* Optimiser settings for one step. step is 1-based and drives the Adam bias
 * corrections 1 - beta^step. clip_norm <= 0 disables clipping. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay, clip_norm;
  int32_t step;
} lm_optim;

typedef enum { LM_PARAMS = 0, LM_GRADS = 1, LM_ADAM_M = 2, LM_ADAM_V = 3 } lm_buf;

/* One entry of the parameter table. offset is in floats from the start of the
 * flat fp32 buffer; rows x cols is the tensor's shape (cols = 1 for vectors).
 * Order: wte[V,C], wpe[max_seq,C]; per block l: ln1.g, ln1.b [C],
 * attn.w_qkv [3C,C], attn.b_qkv [3C], attn.w_o [C,C], attn.b_o [C], ln2.g,
 * ln2.b [C], mlp.w_fc [F,C], mlp.b_fc [F], mlp.w_proj [C,F], mlp.b_proj [C];
 * then lnf.g, lnf.b [C]; with untied_head, head.w [V,C] and head.b [V] last.
 * Names are "wte", "blocks.<l>.attn.w_qkv", "lnf.g", "head.w"...
 * Offsets are 64-float (256-byte) aligned; gaps hold zeros. With bf16
 * precision wte and head.w reserve round_up(V, 128) rows, and head.b as many
 * entries; model_set keeps those padding rows zero in every buffer. Weight
 * matrices are [out, in] row-major (Y = X W^T + b). */
typedef struct {
  char name[48];
  int64_t offset, rows, cols;
} lm_tensor_info;

typedef struct lm_model lm_model;

/* Bytes of device arena the model needs (0 if the config is invalid). */
size_t lm_workspace_bytes(const lm_config* cfg);

/* Validates cfg, carves d_arena (arena_bytes >= lm_workspace_bytes(cfg),
 * 256-byte aligned) and zeroes parameters, gradients and Adam moments on
 * stream. Parameters are then set by the caller with model_set(LM_PARAMS). */
lm_status model_create(const lm_config* cfg, void* d_arena, size_t arena_bytes, void* stream,
                       lm_model** out);

/* Frees the host-side handle; the arena stays the caller's. NULL is a no-op. */
void model_destroy(lm_model* model);

/* Copies up to *count entries of the parameter table into out (if out is
 * non-NULL), sets *count to the number of tensors and *total to the length
 * of the flat buffer in floats. */
lm_status model_param_table(const lm_model* model, lm_tensor_info* out, int32_t* count,
                            int64_t* total);

/* Copy a whole flat fp32 buffer (total floats, layout of the table) in or out.
 * With *_on_device = 0 the host pointer is copied synchronously; with 1 the
 * copy is enqueued on stream. Setting LM_PARAMS also refreshes the bf16
 * operand copies of the weights. */
lm_status model_set(lm_model* model, lm_buf which, const float* src, int src_on_device, void* stream);
lm_status model_get(const lm_model* model, lm_buf which, float* dst, int dst_on_device, void* stream);

/* One training step on a batch of B rows of T tokens (B <= max_batch,
 * T <= max_seq): the forward pass of the pre-LayerNorm stack (Feste page,
 * "Model Architecture"), the mean softmax cross-entropy over the valid
 * targets (RustGPT page, technical-implementation list), the hand-derived
 * backward pass through every layer (Feste page, "Manual Backpropagation"),
 * the global L2 gradient norm with clipping (RustGPT page: clip to an L2 norm
 * of 5.0) and one AdamW update with decoupled weight decay (Feste page,
 * "Manual Backpropagation"). Arguments:
 *   d_tokens  [B,T] int32 in [0, vocab)
 *   d_targets [B,T] int32 in [-1, vocab); -1 = no loss at this position
 *   d_doc_ids [B,T] int32 non-decreasing per row, or NULL for one document per
 *             row; a maximal run of equal ids is one document, attention stays
 *             inside it and positions restart at its first token
 * Computes the mean loss over valid targets, every gradient (kept raw,
 * before clipping, in the LM_GRADS buffer; with precision 2 multiplied by the
 * loss scale of the step), the global norm n, the clip factor and the AdamW
 * update of parameters and moments.
 *   d_stats (may be NULL): 4 floats written on the device:
 *     [0] loss, [1] pre-clip gradient norm, [2] flags, [3] number of valid
 *     targets. flags bit 0: the norm was not finite, so the update was skipped
 *     and parameters and moments are unchanged (precision 2: the loss scale
 *     is multiplied by its backoff factor); bit 1: a token, target or doc id
 *     was out of range or doc ids decreased along a row (checked on the device
 *     in every step; an out-of-range token is clamped into [0, vocab) and an
 *     out-of-range target counts as ignored, so the step stays in bounds).
 * Every shape rule of the kernels is checked when the model is created, so
 * train_step either returns an error before enqueuing anything (NULL
 * pointers, B or T out of range, bad optimiser settings) or enqueues the
 * whole step. */
lm_status train_step(lm_model* model, const int32_t* d_tokens, const int32_t* d_targets,
                     const int32_t* d_doc_ids, int32_t B, int32_t T, const lm_optim* opt,
                     float* d_stats, void* stream);

/* Forward pass only (Feste page, "Model Architecture"; Smallem page, "Ce
 * qu'est un modele de langage": one score per vocabulary entry at every
 * position): d_logits [B,T,vocab] fp32 (row-major) receives z = LN_f(x_L)
 * wte^T (tied head), or z = LN_f(x_L) head.w^T + head.b with untied_head.
 * No loss, no backward, no update. Errors as for train_step. */
lm_status forward_logits(lm_model* model, const int32_t* d_tokens, const int32_t* d_doc_ids,
                         int32_t B, int32_t T, float* d_logits, void* stream);

/* Dynamic loss scale of precision 2. scale: S, the factor on the loss
 * gradient (default 65536); after `interval` steps in a row with a finite
 * gradient norm S is multiplied by growth (default 2000 and 2), after a
 * non-finite one (the step is skipped) by backoff (default 0.5); good_steps:
 * the current run of finite steps. S and good_steps live on the device and
 * change inside train_step without a host round trip. Models of precision 0
 * and 1 have no scaler (LM_ERR_UNSUPPORTED). */
typedef struct {
  float scale, growth, backoff;
  int32_t interval, good_steps;
} lm_loss_scaler;

/* Sets the scaler (synchronises stream). Requires scale > 0 finite, growth
 * >= 1, 0 < backoff <= 1, interval >= 1, 0 <= good_steps < interval. */
lm_status model_set_loss_scaler(lm_model* model, const lm_loss_scaler* scaler, void* stream);
/* Reads the scaler (synchronises stream). */
lm_status model_get_loss_scaler(const lm_model* model, lm_loss_scaler* out, void* stream);

/* Thread-local message for the last non-OK status of this thread. */
const char* lm_last_error(void);

/* The configuration the model was created with. */
lm_status model_config(const lm_model* model, lm_config* out);

/* ---- multi-step training (LucilleAI page, usage of its trainers: a cosine
 * learning-rate scheduler with warm-up steps and a minimum rate, checkpoints
 * every N steps and runs resumed from one; Smallem page, "Les regles du jeu":
 * weight files carry a JSON header) ---- */

/* Learning rate of 1-based step `step` (values below 1 count as 1): linear
 * warm-up lr_max * step / warmup_steps while step <= warmup_steps; then a half
 * cosine from lr_max down to lr_min, lr_min + (lr_max - lr_min) (1 + cos(pi p))
 * / 2 with p = (step - warmup_steps) / (total_steps - warmup_steps); lr_min
 * from total_steps on. total_steps <= warmup_steps: lr_max after the warm-up
 * (no decay). Pure host function, evaluated in double. */
float lm_lr_schedule(int32_t step, int32_t warmup_steps, int32_t total_steps, float lr_max, float lr_min);

/* Checkpoint file in the safetensors layout: 8-byte little-endian header
 * length, JSON header, raw little-endian fp32 data. Tensors "param.<name>",
 * "adam_m.<name>", "adam_v.<name>" for every entry of the parameter table
 * (shape [rows, cols], or [rows] for vectors), back to back in that order;
 * "__metadata__" holds format "lmstep-checkpoint", version, step and the model
 * dimensions as strings. model_save synchronises `stream`, writes path.tmp and
 * renames it to path. model_load checks the format, every dimension, dtype,
 * shape and offset (LM_ERR_SHAPE on a model mismatch, LM_ERR_ARG on a bad
 * file), restores parameters (and their bf16 copy) and both moments, and
 * returns the saved step in *step (nullable). Gradients are not saved: the
 * next train_step recomputes them. */
lm_status model_save(const lm_model* model, const char* path, int32_t step, void* stream);
lm_status model_load(lm_model* model, const char* path, int32_t* step, void* stream);

/* ---- generation (RustGPT page, technical list: greedy decoding; LucilleAI
 * page: a sampler with temperature and top-k) ----
 * Next token of each of `rows` rows of fp32 logits (row r starts at
 * d_logits + r * ld, `vocab` columns; ld >= vocab), into d_out [rows] int32.
 * temperature <= 0: greedy, the largest logit, ties to the smallest id
 * (d_uniforms may be NULL). Otherwise the top_k largest logits (top_k <= 0 or
 * >= vocab: all; ties at the k-th value go to the smaller ids) with weights
 * exp((z - z_max) / temperature); the caller's uniform u in [0, 1) for the row
 * (d_uniforms [rows], device) picks the smallest kept id whose running weight
 * sum, in ascending id order, reaches u times the total. Deterministic: the
 * same inputs give the same ids. Enqueued on `stream`. */
lm_status sample_tokens(const float* d_logits, int32_t rows, int32_t vocab, int64_t ld, float temperature,
                        int32_t top_k, const float* d_uniforms, int32_t* d_out, void* stream);

/* Key/value cache for `batch` rows: per layer, K [batch][max_seq][d_model]
 * then V of the same shape, in the activation type (bf16 for precision 1,
 * else fp32). The caller allocates lm_kv_cache_bytes(cfg, batch) bytes of
 * device memory and passes the same batch to every call on that cache.
 * model_prefill runs the forward pass over d_tokens [B, T] (one document per
 * row), fills cache positions 0 .. T-1 and writes the logits of each row's
 * last position to d_logits [B, vocab] fp32. model_decode takes one new token
 * per row (d_tokens [B]) at position pos (1 <= pos < max_seq; positions
 * 0 .. pos-1 already cached), appends its keys and values at pos, attends
 * over positions 0 .. pos and writes its logits to d_logits [B, vocab].
 * Both overwrite the model's forward activations (not its parameters). */
size_t lm_kv_cache_bytes(const lm_config* cfg, int32_t batch);
lm_status model_prefill(lm_model* model, const int32_t* d_tokens, int32_t B, int32_t T, void* d_cache,
                        float* d_logits, void* stream);
lm_status model_decode(lm_model* model, const int32_t* d_tokens, int32_t B, int32_t pos, void* d_cache,
                       float* d_logits, void* stream);

/* model_decode_at is model_decode with the position in device memory
 * (d_pos, one int32), read by the kernels when they run rather than when the
 * call is made: a graph captured from one call (hipStreamBeginCapture on
 * `stream`) can then be replayed at successive positions by rewriting
 * *d_pos (and the tokens at d_tokens) between replays. The call itself
 * allocates nothing and does not synchronize. A position outside
 * [1, max_seq) is clamped into it (the kernels never touch memory outside
 * the cache); keeping it in range is the caller's part. Errors: NULL
 * pointers, a batch outside [1, max_batch], max_seq < 2. */
lm_status model_decode_at(lm_model* model, const int32_t* d_tokens, int32_t B, const int32_t* d_pos,
                          void* d_cache, float* d_logits, void* stream);

/* ---- measurement hooks (used by the benchmark) ----
 * With profiling on, every kernel launch of train_step is bracketed by a pair
 * of HIP events recorded on the step's stream, and model_profile_read sums
 * their elapsed times per kernel class. Off by default; enabling it adds a
 * few microseconds per launch. */
typedef struct {
  char name[40];     /* kernel class, e.g. "gemm_head_fwd"             */
  int64_t launches;  /* launches recorded since the last reset          */
  double ms;         /* summed event time over those launches           */
  double flops;      /* algorithmic flops per step of this class        */
  double bytes;      /* algorithmic HBM bytes per step of this class    */
} lm_profile_entry;

lm_status model_profile_enable(lm_model* model, int enable);
/* Synchronises the events, fills up to cap entries, returns the number of
 * classes in *n, and resets the accumulators when reset != 0. */
lm_status model_profile_read(lm_model* model, lm_profile_entry* out, int32_t cap, int32_t* n,
                             int reset);

#ifdef __cplusplus
}
#endif

#endif /* LMSTEP_H */
