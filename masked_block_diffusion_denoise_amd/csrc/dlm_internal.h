// Host-side launchers of the libdlm kernels.  Every launcher enqueues work on
// `stream` and returns the launch status; none allocates, frees or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dlm {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

// ---------------------------------------------------------------- GEMM ----
// C = A[M][K] * W[N][K]^T with bf16 operands and fp32 accumulation.
enum GemmEpilogue : int {
  EPI_STORE_BF16 = 0,  // out bf16 [M][ldc]
  EPI_RESID_F32 = 1,   // out fp32 [M][ldc] += acc (residual stream)
  EPI_SWIGLU = 2,      // W rows gate/up interleaved in 16-row groups; out bf16 [M][N/2] = silu(g)*u
  EPI_HEAD = 3,        // per (row, vocab tile) partial max / sum exp / argmax; optional fp32 logits
  EPI_SPLITK = 4,      // internal: fp32 partial products of one K range, reduced by a second kernel
};

struct GemmArgs {
  const void* a;        // bf16 [M][lda]
  const void* w;        // bf16 [N][K]
  void* out;            // see epilogue
  int M, N, K;
  int lda, ldc;
  float alpha = 1.f;    // EPI_RESID_F32: out += alpha * A W^T
  const int* m_dev;     // optional device row count (rows >= *m_dev are skipped); M is the bound
  // EPI_HEAD only
  void* partials;       // MaxSumIdx-like records [n_tiles][M]
  float* logits;        // optional fp32 [rows][N]
  const int* logit_rows; // optional: logits of result row m go to row logit_rows[m]
  int mask_id;
  int* nonfinite;       // device counter, incremented on non-finite logits
  // K-split (set by gemm() when gemm_ksplit() > 1): fp32 [ksplit][M][N] partials
  float* kpart;         // workspace of gemm_workspace_bytes(M, N, K) bytes, from the caller
  int ksplit;
  // tile order: 0 = row tiles fastest, then K ranges, then weight tiles (the
  // workgroups sharing a weight tile share an XCD's L2); 1 = weight tiles
  // fastest, then row tiles, then K ranges (set for long-K split products)
  int weights_fastest = 0;
};

int gemm_head_tile_n(int M);                       // vocab columns per EPI_HEAD partial
// Number of K ranges gemm() splits an (M, N, K) product into (1: no split; the
// LM head never splits), and the workspace (g.kpart) it then needs.
int gemm_ksplit(int M, int N, int K);
size_t gemm_workspace_bytes(int M, int N, int K);
hipError_t gemm(const GemmArgs& g, GemmEpilogue epi, hipStream_t s);
// Only the K-split partial products, fp32 [S][M][N] into g.kpart, with
// S = gemm_ksplit(M, N, K) > 1 (else an error): for callers that fuse the
// reduction into the next step (resid_norm, rope_kv).
hipError_t gemm_partials(const GemmArgs& g, hipStream_t s);

// --------------------------------------------------------- attention ----
struct AttnArgs {
  const void* q;          // bf16, row m = b*Lq + j, head h at q[m*ldq + h*hd]
  int ldq;
  const void* kc;         // bf16 K cache of this layer [B][G][cap][hd]
  const void* vc;         // bf16 V cache of this layer [B][G][cap/16][hd][16]
  void* o;                // bf16 [B*Lq][H*hd]
  const int* prefix;      // device [B] or null
  int pos_offset;         // query j of row b sits at prefix[b] + pos_offset + j
  int B, Lq, H, G, hd, cap;
  int causal;             // 0: every key < prefix+pos_offset+Lq visible; 1: key <= query position
  int max_kv;             // host bound on prefix[b] + pos_offset + Lq
  float* part_o;          // fp32 [splits][B*Lq][H][hd]
  float* part_ml;         // fp32 [splits][B*Lq][H][2]
};
int attn_splits(const AttnArgs& a, int* chunk_out);
size_t attn_partial_floats(int splits, int rows, int H, int hd);
// bound of attn_partial_floats over every B, Lq with B*Lq <= R and max_kv keys
size_t attn_partial_floats_bound(int R, int H, int G, int hd, int max_kv);
hipError_t attention(const AttnArgs& a, hipStream_t s);

// ------------------------------------------------------------ small ----
enum CommitRule : int { COMMIT_THRESHOLD = 0, COMMIT_BOUND = 1, COMMIT_ENTROPY = 2 };
struct CommitOpts {
  int rule = COMMIT_THRESHOLD;
  float min_threshold = 0.45f, scaling = 2.f;  // COMMIT_BOUND
  float entropy_bound = 0.1f;                  // COMMIT_ENTROPY
  int max_transfer = 0;                        // > 0: at most this many per step (not on the last)
  int stability_steps = 0;                     // > 0: adaptive stopping
  float stop_entropy = 0.005f;
  int* prev_argmax = nullptr;                  // [B][L] adaptive-stopping state
  int* stable = nullptr;                       // [B]
};
// entropy: per-position entropies [B][L] (the entropy rule, adaptive stopping)
hipError_t commit(const float* conf, const int* argmax, int* canvas, uint8_t* masked, int B, int L,
                  const float* tau, const int* quota, int* steps, int max_steps, int* n_committed,
                  int* n_left, hipStream_t s, const float* entropy = nullptr, const CommitOpts* opts = nullptr);
// row m = b*Lq + j takes token tokens[b*tok_ld + j]; with tab, the same launch
// fills the RoPE table of the pass (rope_table's layout)
hipError_t embed_norm(const int* tokens, int M, int Lq, int tok_ld, const void* embed, int V, int d,
                      const void* gain, float eps, float* x, void* xn, int* bad_token, const int* prefix,
                      int pos_offset, int hd, float base, float2* tab, hipStream_t s);
hipError_t rmsnorm(const float* x, int M, int d, const void* gain, float eps, void* xn,
                   const int* rows, const int* m_dev, hipStream_t s);
hipError_t rope_table(const int* prefix, int pos_offset, int B, int Lq, int hd, float base, float2* tab,
                      hipStream_t s);
// part (with S splits): the row values are the sum of fp32 K-split partials
// [S][M][(H+2G)hd] instead of bf16 qkv
hipError_t rope_kv(void* qkv, int M, int Lq, int H, int G, int hd, const float2* tab, void* kc, void* vc,
                   const int* prefix, int pos_offset, int cap, hipStream_t s, const float* part = nullptr,
                   int S = 1);
// x[m] += sum_s part[s][m] over S fp32 partial planes [S][M][d], then
// xn[m] = RMSNorm(x[m]) * gain (bf16)
hipError_t resid_norm(const float* part, int S, int M, float* x, int d, const void* gain, float eps, void* xn,
                      hipStream_t s);
// rows[0..count) = indices m with masked[m] != 0, ascending, and count[0] = how
// many, fused with the final RMSNorm of those rows into xn[0..count).  With
// S > 0 the rows are x[m] + sum_s part[s][m] (S fp32 partial planes [S][M][d]
// of the last residual product, summed in split order); x is not written.
hipError_t masked_norm(const uint8_t* masked, int M, const float* x, int d, const void* gain, float eps, void* xn,
                       int* rows, int* count, hipStream_t s, const float* part = nullptr, int S = 0);
// entropy (optional): ln(sum exp) - sum exp*(l - max) / sum exp per row, in nats
hipError_t head_merge(const void* partials, int n_tiles, int M, const int* rows, const int* m_dev,
                      float* conf, int* argmax, int total_rows, hipStream_t s, float* entropy = nullptr);
hipError_t fill_i32(int* p, int n, int v, hipStream_t s);
hipError_t fill_f32(float* p, int n, float v, hipStream_t s);
// prefix[b] = (add ? prefix[b] : 0) + value
hipError_t set_prefix(int* prefix, int B, int add, int value, hipStream_t s);
// rows[b] = b*stride + start
hipError_t strided_rows(int* rows, int n, int start, int stride, hipStream_t s);

}  // namespace dlm
