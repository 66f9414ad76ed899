/*
 * libdlm kernel-level entry points: each runs one step of the denoising pass on
 * caller-provided buffers, so that every step can be checked on its own.
 * Conventions as in libdlm.h ([dev]/[host] ownership, bf16 storage with fp32
 * accumulation, host validation before anything is enqueued, nothing allocated,
 * asynchronous on `stream`).
 */
#ifndef LIBDLM_OPS_H
#define LIBDLM_OPS_H

#include "libdlm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of dlm_op_gemm. */
enum { DLM_EPI_STORE_BF16 = 0, DLM_EPI_RESIDUAL_F32 = 1, DLM_EPI_SWIGLU = 2 };

/* Dense projection C = A W^T (MLX guide, sec. 7: every projection of the
 * decoder is a plain matrix product, no bias).
 *   a   [dev] bf16 [M][lda]  (first K columns used)
 *   w   [dev] bf16 [N][K]
 *   out DLM_EPI_STORE_BF16:   bf16 [M][ldc], out = A W^T
 *       DLM_EPI_RESIDUAL_F32: fp32 [M][ldc], out += A W^T (residual stream)
 *       DLM_EPI_SWIGLU:       bf16 [M][ldc] with N/2 columns: w holds gate and up
 *                             rows interleaved by 16 (as dlm_weights.wgu);
 *                             out = silu(gate) * up, silu(z) = z / (1 + e^-z)
 * Requirements: N a multiple of 128; K a multiple of 256, or of 64 up to 256.
 * ws: dlm_op_gemm_workspace_bytes(M, N, K) bytes, 256-byte aligned: fp32
 * partial products when K is split over workgroups (short products, M <= 64);
 * when that size is 0, ws may be NULL.  WORKSPACE if it is too small. */
size_t dlm_op_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);
dlm_status dlm_op_gemm(const void* a, const void* w, void* out, int32_t M, int32_t N, int32_t K, int32_t lda,
                       int32_t ldc, int32_t epilogue, void* ws, size_t ws_bytes, void* stream);

/* RMSNorm (a reading: x / sqrt(mean(x^2) + eps) * g; the pages name the norm
 * without its formula): x [dev] fp32 [M][d] -> out [dev] bf16 [M][d]; g [dev] bf16 [d]. */
dlm_status dlm_op_rmsnorm(const float* x, int32_t M, int32_t d, const void* g, float eps, void* out, void* stream);

/* RoPE and KV-cache write for one layer's fused QKV rows (row m = b*Lq + j at
 * position prefix[b] + pos_offset + j; prefix may be NULL = zeros):
 * query heads are rotated in place in qkv [dev] bf16 [B*Lq][(H+2G)hd]; rotated
 * keys and the values go to k_cache / v_cache of one layer, laid out as one
 * layer of dlm_kv.  Positions outside [0, cap) are not written.
 * ws: dlm_op_rope_workspace_bytes(B, Lq, hd) bytes (angle table). */
size_t dlm_op_rope_workspace_bytes(int32_t B, int32_t Lq, int32_t hd);
dlm_status dlm_op_rope_kv(void* qkv, int32_t B, int32_t Lq, int32_t H, int32_t G, int32_t hd, float rope_base,
                          void* k_cache, void* v_cache, const int32_t* prefix, int32_t pos_offset, int32_t cap,
                          void* ws, size_t ws_bytes, void* stream);

/* Block attention of one layer (Module 12, sec. 14; MLX guide, sec. 6).  Query
 * j of row b (position p = prefix[b] + pos_offset + j) attends, with scale
 * 1/sqrt(hd) and query head h reading KV head h / (H/G), to keys
 * [0, prefix[b] + pos_offset + Lq) of cache row b -- all of them when causal = 0
 * (the denoise pass), those at positions <= p when causal = 1.
 *   q  [dev] bf16, query head h of row m at q[m*ldq + h*hd]
 *   o  [dev] bf16 [B*Lq][H*hd]
 *   max_kv: host bound on prefix[b] + pos_offset + Lq (<= cap)
 * ws: dlm_op_attention_workspace_bytes(...) bytes (split-KV partials). */
size_t dlm_op_attention_workspace_bytes(int32_t B, int32_t Lq, int32_t H, int32_t G, int32_t hd, int32_t max_kv);
dlm_status dlm_op_attention(const void* q, int32_t ldq, const void* k_cache, const void* v_cache, void* o,
                            const int32_t* prefix, int32_t pos_offset, int32_t B, int32_t Lq, int32_t H, int32_t G,
                            int32_t hd, int32_t cap, int32_t causal, int32_t max_kv, void* ws, size_t ws_bytes,
                            void* stream);

/* LM head to confidence (MLX guide, sec. 5.3): for R already-normalised rows
 * hidden [dev] bf16 [R][d] and head [dev] bf16 [V][d], conf[r] = max softmax
 * probability over the vocabulary without mask_id and argmax[r] = lowest id
 * reaching the max logit, computed per vocabulary tile and merged, without
 * writing the logits (unless logits [dev] fp32 [R][V] is given; -inf at mask_id).
 * entropy [dev] fp32 [R] or NULL: the softmax's entropy in nats (as for
 * dlm_denoise_step_ex).
 * flags [dev] int32 [2] or NULL: flags[0] += rows' tiles with non-finite logits.
 * Requirements: V a multiple of 256; d as K of dlm_op_gemm.
 * ws: dlm_op_lm_head_workspace_bytes(R, V) bytes. */
size_t dlm_op_lm_head_workspace_bytes(int32_t R, int32_t V);
dlm_status dlm_op_lm_head(const void* hidden, int32_t R, int32_t d, const void* head, int32_t V, int32_t mask_id,
                          float* conf, int32_t* argmax, float* entropy, float* logits, int32_t* flags, void* ws,
                          size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBDLM_OPS_H */
