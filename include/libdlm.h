/*
 * libdlm -- masked block-diffusion denoising on one AMD Instinct MI355X (gfx950).
 *
 * The calls follow the decoding problem as the pages state it:
 *   - the prompt is prefilled causally into a KV cache (MLX-VLM Nemotron Labs
 *     Diffusion guide, sec. 3.1 and sec. 6: causal prefill, use_causal_mask);
 *   - a block of masked positions is denoised by a bidirectional pass that
 *     reads the cached prefix and every position of the block (Modern LLMs,
 *     Module 12, sec. 14; MLX guide, sec. 6);
 *   - each pass ends with a commit: positions whose confidence is above a
 *     threshold are unmasked, at least a quota per step, the rest stay masked,
 *     and the last allowed step commits everything left (MLX guide, sec. 5.2
 *     and sec. 6; NLD tutorial, sec. 3.1; DiffusionGemma docs,
 *     BlockRefinementScheduler);
 *   - the finished block goes through a separate causal pass whose keys and
 *     values are appended to the cache (MLX guide, sec. 6; Module 12, sec. 14:
 *     the last denoise pass's keys/values were computed from masks and may not
 *     enter the history).
 *
 * Conventions for every call:
 *   - [dev] pointers are device memory owned by the caller; [host] pointers are
 *     host memory owned by the caller.  The library keeps no pointer past the
 *     call except the weight pointers borrowed by a dlm_model (and, per GPU,
 *     the address of its own fixed scratch array, dlm_denoise_step_noalloc).
 *   - The library never allocates or frees device memory and never
 *     synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream) and may still be running when the call returns.
 *   - Every argument the host can check is checked before anything is
 *     enqueued; on a non-OK return nothing was enqueued and dlm_last_error()
 *     gives the reason.  Device-side conditions (non-finite logits,
 *     out-of-range token ids) are counted into the optional `flags` array and
 *     are visible after the caller synchronises.
 *   - bf16 = IEEE-754 binary32 truncated to its upper 16 bits (stored as
 *     uint16); all accumulation is fp32.
 *   - Calls that overlap on one stream are ordered; calls on different streams
 *     that share a workspace, a KV cache or a canvas race.
 */
#ifndef LIBDLM_H
#define LIBDLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DLM_OK = 0,
  DLM_ERR_INVALID_ARG = -1, /* null / misaligned pointer, non-finite or out-of-range scalar */
  DLM_ERR_SHAPE = -2,       /* sizes inconsistent with each other or with the model */
  DLM_ERR_CAPACITY = -3,    /* KV cache too small for the positions written */
  DLM_ERR_UNSUPPORTED = -4, /* a shape the library has no kernel for (e.g. head_dim not 32/128) */
  DLM_ERR_HIP = -5,         /* a kernel launch failed (text in dlm_last_error) */
  DLM_ERR_WORKSPACE = -6    /* ws_bytes smaller than the call needs */
} dlm_status;

/* Model shape.  Dense pre-norm decoder (MLX guide, sec. 7): RMSNorm ->
 * grouped-query attention with RoPE -> residual -> RMSNorm -> SwiGLU ->
 * residual, final RMSNorm, untied head over `vocab`.  Requirements:
 * head_dim in {32, 128}; n_heads / n_kv_heads in {1, 2, 4}; d_model,
 * n_heads*head_dim and d_ffn multiples of 256 (or 64..256 and multiples of 64);
 * (n_heads + 2*n_kv_heads)*head_dim, d_model and 2*d_ffn multiples of 128;
 * d_model <= 8192;
 * vocab a multiple of 256; 0 <= mask_id < vocab; rope_base > 0; rms_eps > 0. */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, mask_id;
  float rope_base; /* RoPE: pair (i, i+hd/2) turns by pos * rope_base^(-2i/hd) */
  float rms_eps;   /* RMSNorm: x / sqrt(mean(x^2) + eps) * g */
} dlm_config;

/* Weights, all bf16, row-major [out_features][in_features] (y = x W^T).
 * Per-layer fields are [host] arrays of n_layers [dev] pointers; the arrays are
 * copied by dlm_model_create, the device memory is borrowed until
 * dlm_model_destroy.  All device pointers 16-byte aligned.
 *   embed      [V][d]              final_norm [d]          lm_head [V][d]
 *   attn_norm  [d]                 ffn_norm   [d]
 *   wqkv       [(H + 2G) hd][d]    rows: H query heads, G key heads, G value heads
 *   wo         [d][H hd]
 *   wgu        [2F][d]             gate/up interleaved by 16 rows: rows 32c..32c+15
 *                                  are gate rows 16c..16c+15, rows 32c+16..32c+31
 *                                  the up rows of the same 16 outputs
 *   wdown      [d][F]                                                         */
typedef struct {
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* ffn_norm;
  const void* const* wgu;
  const void* const* wdown;
} dlm_weights;

/* KV cache of `batch` rows and `capacity` positions per row (capacity a
 * multiple of 64), keys after RoPE.  Layouts (bf16):
 *   k [n_layers][batch][n_kv_heads][capacity][head_dim]
 *   v [n_layers][batch][n_kv_heads][capacity/16][head_dim][16]
 * (values in blocks of 16 positions, position fastest).  Row b of every call
 * uses cache row b. */
typedef struct {
  void* k;
  void* v;
  int32_t batch;
  int32_t capacity;
} dlm_kv;

typedef struct dlm_model dlm_model; /* opaque, host-side */

/* Validate the shape and weight pointers and build a model handle (host memory only). */
dlm_status dlm_model_create(const dlm_config* cfg, const dlm_weights* w, dlm_model** out);
void dlm_model_destroy(dlm_model* m);

/* Low-rank adapter on every layer's attention output projection, used by the
 * draft passes of linear self-speculation (MLX guide, sec. 3.3: rank 128,
 * scale 4.0, on self_attn.o_proj only; sec. 8: enabled while drafting, disabled
 * for the causal verification).  While enabled, every pass computes
 *   o_proj(y) = y Wo^T + scale * (y A^T) B^T
 *   a, b   [host] arrays of n_layers [dev] pointers (16-byte aligned), borrowed
 *          like the weights: A bf16 [rank][n_heads*head_dim], B bf16 [d_model][rank]
 *   rank   a multiple of 128, at most DLM_MAX_LORA_RANK
 * a == b == NULL removes the adapter.  Setting an adapter leaves it disabled.
 * The switch is host state of the handle: calls that overlap with it (on any
 * thread) see either setting.  Errors: INVALID_ARG for NULL or misaligned
 * matrices, a non-finite scale, or enabling with no adapter set; UNSUPPORTED
 * for another rank. */
#define DLM_MAX_LORA_RANK 256
dlm_status dlm_model_set_lora(dlm_model* m, const void* const* a, const void* const* b, int32_t rank, float scale);
dlm_status dlm_model_enable_lora(dlm_model* m, int32_t on);

/* Bytes of workspace that a pass over up to `max_rows` rows (batch x tokens per
 * pass) against at most `max_kv` keys per row needs.  Enough for
 * dlm_denoise_step and dlm_append_block with B*L <= max_rows and
 * max_prefix + L <= max_kv, and lets dlm_prefill use passes of max_rows rows. */
size_t dlm_workspace_bytes(const dlm_model* m, int32_t max_rows, int32_t max_kv);

/* Causal prefill of a prompt of T tokens per row for rows 0..B-1, all starting
 * at position 0.  Writes keys/values for positions [0, T) and prefix_len[b] = T.
 *   tokens      [dev] int32 [B][T], ids in [0, vocab)
 *   prefix_len  [dev] int32 [B], out
 *   last_argmax [dev] int32 [B] or NULL: greedy next token after the prompt
 *   last_conf   [dev] fp32 [B] or NULL: its probability
 *   flags       [dev] int32 [2] or NULL: [0] += rows with non-finite logits,
 *               [1] += out-of-range token ids (read as zeros)
 *   ws          [dev] workspace, 256-byte aligned; the prompt is processed in
 *               passes of as many positions as ws_bytes allows (at least 32 rows
 *               per row of the batch must fit).
 * Errors: SHAPE if B < 1, B > kv->batch or T < 1; CAPACITY if T > capacity. */
dlm_status dlm_prefill(const dlm_model* m, const dlm_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                       int32_t* prefix_len, int32_t* last_argmax, float* last_conf, int32_t* flags,
                       void* ws, size_t ws_bytes, void* stream);

/* One denoise pass over a canvas of L positions per row (MLX guide, sec. 6;
 * Module 12, sec. 14): position j of row b sits at prefix_len[b] + j and reads
 * every cached key of row b and every canvas position, masked or not.  The
 * canvas's own keys/values are written to cache slots [prefix_len[b],
 * prefix_len[b] + L) as scratch (prefix_len is not changed; the post-block
 * append overwrites them).  Only masked positions are scored (MLX guide,
 * sec. 5.3, chunked head scoring): for each, over the vocabulary without the
 * mask id, conf = max softmax probability = 1 / sum_v exp(l_v - max l) and
 * argmax = the lowest id reaching the max.  Full logits never reach memory
 * unless `logits` is given.
 *   prefix_len [dev] int32 [B]; 0 <= prefix_len[b] <= max_prefix (host bound)
 *   canvas     [dev] int32 [B][L] token ids (mask id at masked positions)
 *   masked     [dev] uint8 [B][L], nonzero = masked
 *   conf       [dev] fp32 [B][L], argmax [dev] int32 [B][L]: written at masked
 *              positions only, left unchanged elsewhere
 *   logits     [dev] fp32 [B][L][vocab] or NULL (parity checks only): written at
 *              masked positions, -inf at the mask id
 *   flags      as for dlm_prefill
 * Errors: SHAPE if B < 1, B > kv->batch, L < 1 or L > 64; CAPACITY if
 * max_prefix + L > capacity; WORKSPACE if ws_bytes is too small. */
dlm_status dlm_denoise_step(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len, int32_t max_prefix,
                            const int32_t* canvas, const uint8_t* masked, int32_t B, int32_t L, float* conf,
                            int32_t* argmax, float* logits, int32_t* flags, void* ws, size_t ws_bytes,
                            void* stream);

/* dlm_denoise_step that also writes, at the masked positions, the entropy in
 * nats of each position's softmax over the vocabulary without the mask id,
 * -sum_v p_v ln p_v = ln S - sum_v e_v (l_v - max) / S with e_v = exp(l_v - max)
 * and S = sum_v e_v (the ranking and stopping quantity of the DiffusionGemma
 * docs' EntropyBoundScheduler and adaptive stopping).  The head accumulates the
 * second sum beside S in the same pass; no logits are written for it.
 *   entropy [dev] fp32 [B][L] or NULL (then exactly dlm_denoise_step).
 * Errors as dlm_denoise_step; INVALID_ARG if entropy is misaligned. */
dlm_status dlm_denoise_step_ex(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len, int32_t max_prefix,
                               const int32_t* canvas, const uint8_t* masked, int32_t B, int32_t L, float* conf,
                               int32_t* argmax, float* entropy, float* logits, int32_t* flags, void* ws,
                               size_t ws_bytes, void* stream);

/* dlm_denoise_step_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  The pass's scratch is a fixed array of
 * DLM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, resident on each
 * GPU the library has run this call on until the process ends; the call
 * allocates nothing (no hipMalloc, no library allocation).  The array's device
 * address is taken on the first call on a device, with that device current;
 * call it with the device of `stream` current.  64 MiB holds a batch-1 pass of
 * the 8B-class model (32 canvas positions) up to a 65536-position prefix;
 * dlm_workspace_bytes bounds what a pass needs.  Every call on one GPU uses
 * that GPU's one array, which keeps the last call's contents: calls that
 * overlap on one GPU (other streams, other threads) race; calls on one stream
 * are ordered.  Arguments, outputs and results as dlm_denoise_step_ex.
 * Errors as dlm_denoise_step_ex; WORKSPACE (before any device call) if the
 * pass needs more than DLM_NOALLOC_SCRATCH_BYTES; HIP if the scratch's device
 * address cannot be obtained. */
#define DLM_NOALLOC_SCRATCH_BYTES (64u << 20)
dlm_status dlm_denoise_step_noalloc(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len,
                                    int32_t max_prefix, const int32_t* canvas, const uint8_t* masked, int32_t B,
                                    int32_t L, float* conf, int32_t* argmax, float* entropy, float* logits,
                                    int32_t* flags, void* stream);

/* Commit / remask (MLX guide, sec. 5.2 native sampler and sec. 6; DiffusionGemma
 * docs, BlockRefinementScheduler).  Per row b with at least one masked position:
 *   A = { masked j : conf[b][j] > threshold[b] }          (strictly above)
 *   q = #masked if steps[b] >= max_steps - 1, else min(quota[b], #masked)
 *   n = max(|A|, q); the n masked positions first in (-conf, j) order get
 *   canvas = argmax and masked = 0; the others stay masked; steps[b] += 1.
 * Rows with no masked position are left unchanged (steps too).
 *   conf [dev] fp32 [B][L] (read at masked positions; must not be NaN there),
 *   argmax [dev] int32 [B][L], canvas/masked [dev] [B][L] in/out,
 *   threshold [dev] fp32 [B], quota [dev] int32 [B], steps [dev] int32 [B] in/out,
 *   n_committed / n_left [dev] int32 [B] out.
 * Errors: SHAPE if B < 1, L < 1 or L > 64; INVALID_ARG if max_steps < 1. */
dlm_status dlm_commit(const float* conf, const int32_t* argmax, int32_t* canvas, uint8_t* masked, int32_t B,
                      int32_t L, const float* threshold, const int32_t* quota, int32_t* steps, int32_t max_steps,
                      int32_t* n_committed, int32_t* n_left, void* stream);

/* Sampler variants of the commit step. */
typedef enum {
  DLM_RULE_THRESHOLD = 0, /* native: conf > threshold (dlm_commit) */
  DLM_RULE_BOUND = 1,     /* MLX guide, sec. 5.2, confidence_threshold_bound: conf >= threshold, or
                             conf >= min_threshold and conf >= 1 - scaling / (j + 2), j = position
                             in the block (float32 arithmetic) */
  DLM_RULE_ENTROPY = 2    /* DiffusionGemma docs, EntropyBoundScheduler: masked positions in
                             (entropy, position) order while the float32 running sum of their
                             entropies stays <= entropy_bound */
} dlm_commit_rule;

typedef struct {
  int32_t rule;            /* dlm_commit_rule */
  float min_threshold;     /* DLM_RULE_BOUND floor (the page's default 0.45) */
  float scaling;           /* DLM_RULE_BOUND position scaling (the page's default 2.0) */
  float entropy_bound;     /* DLM_RULE_ENTROPY bound on the summed entropy */
  int32_t max_transfer;    /* > 0: at most this many positions per step (MLX guide, sec. 5.5,
                              --max-transfer-per-step); the last allowed step still completes */
  int32_t stability_steps; /* > 0: adaptive stopping (DiffusionGemma docs): a row whose argmax at
                              every masked position has not changed for this many consecutive steps
                              and whose mean masked entropy (float32 sum in position order) is below
                              stop_entropy commits every remaining mask */
  float stop_entropy;      /* the page's default 0.005 */
  int32_t* prev_argmax;    /* [dev] int32 [B][L]: adaptive-stopping state; set to -1 when a block
                              starts; takes each step's argmax at the masked positions */
  int32_t* stable;         /* [dev] int32 [B]: consecutive stable steps; 0 when a block starts */
} dlm_commit_opts;

/* dlm_commit with a sampler rule.  Per row with a masked position: adaptive
 * stopping first (when enabled); then A as the rule defines it; on the last
 * allowed step every remaining mask; else A when |A| >= q = min(quota[b],
 * #masked), otherwise A plus the best-ranked other masked positions up to q;
 * then the max_transfer cap keeps the best-ranked.  Rank: (-conf, position), or
 * (entropy, position) for DLM_RULE_ENTROPY.  With DLM_RULE_THRESHOLD and no
 * cap or stopping this is exactly dlm_commit.
 *   entropy [dev] fp32 [B][L] (dlm_denoise_step_ex), required by DLM_RULE_ENTROPY
 *           and by adaptive stopping, else may be NULL
 *   opts    host struct, read during the call
 * Errors as dlm_commit; INVALID_ARG for an unknown rule, a non-finite
 * parameter, max_transfer < 0, stability_steps < 0, or a missing entropy /
 * state buffer the options need. */
dlm_status dlm_commit_ex(const float* conf, const int32_t* argmax, const float* entropy, int32_t* canvas,
                         uint8_t* masked, int32_t B, int32_t L, const float* threshold, const int32_t* quota,
                         int32_t* steps, int32_t max_steps, const dlm_commit_opts* opts, int32_t* n_committed,
                         int32_t* n_left, void* stream);

/* Post-block pass (MLX guide, sec. 6; Module 12, sec. 14): a causal pass of the
 * finished block at positions prefix_len[b] + j; its keys/values overwrite cache
 * slots [prefix_len[b], prefix_len[b] + L); then prefix_len[b] += L.
 *   block       [dev] int32 [B][L]
 *   argmax_out  [dev] int32 [B][L] or NULL: greedy prediction of the next token at
 *               every position (causal head; for AR decoding and verification)
 *   conf_out    [dev] fp32 [B][L] or NULL
 * Errors as dlm_denoise_step. */
dlm_status dlm_append_block(const dlm_model* m, const dlm_kv* kv, int32_t* prefix_len, int32_t max_prefix,
                            const int32_t* block, int32_t B, int32_t L, int32_t* argmax_out, float* conf_out,
                            int32_t* flags, void* ws, size_t ws_bytes, void* stream);

/* Kernel timing hook (measurement only).  When set, the next calls on this host
 * thread record `start` (a hipEvent_t) on their stream right before the named
 * kernel is launched and `stop` right after it; NULL events switch it off.
 *   DLM_TIMER_LM_HEAD      the fused LM-head GEMM of dlm_denoise_step
 *   DLM_TIMER_ATTENTION    block attention (with its split merge) of the first layer
 *   DLM_TIMER_GATE_UP      the SwiGLU gate/up GEMM of the first layer
 *   DLM_TIMER_DOWN         the down-projection GEMM of the first layer (with its residual
 *                          add and the next RMSNorm; for the last layer, when split over
 *                          K, only the partial products: DLM_TIMER_FINAL_NORM sums them)
 *   DLM_TIMER_QKV          the fused QKV GEMM of the first layer (with its K-split
 *                          reduction, fused with RoPE and the cache write, when split)
 *   DLM_TIMER_O            the attention output projection of the first layer with its
 *                          residual add and the FFN RMSNorm
 *   DLM_TIMER_FINAL_NORM   masked-row compaction + final RMSNorm of dlm_denoise_step,
 *                          which also sums the last layer's down-projection K-split
 *                          partials when that product is split
 * Errors: INVALID_ARG for an unknown kernel id. */
enum { DLM_TIMER_LM_HEAD = 0, DLM_TIMER_ATTENTION = 1, DLM_TIMER_GATE_UP = 2, DLM_TIMER_DOWN = 3,
       DLM_TIMER_QKV = 4, DLM_TIMER_O = 5, DLM_TIMER_FINAL_NORM = 6, DLM_TIMER_COUNT = 7 };
dlm_status dlm_set_kernel_timer(int32_t kernel, void* start_event, void* stop_event);

const char* dlm_status_string(dlm_status s);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* dlm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBDLM_H */
