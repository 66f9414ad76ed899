// libdlm C ABI: host-side validation, workspace planning and the launch
// sequence of each call.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/libdlm.h"
#include "../../include/libdlm_ops.h"
#include "dlm_internal.h"

using namespace dlm;

struct dlm_model {
  dlm_config c;
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  std::vector<const void*> attn_norm, wqkv, wo, ffn_norm, wgu, wdown;
  // optional low-rank adapter on the output projection (dlm_model_set_lora)
  std::vector<const void*> lora_a, lora_b;
  int lora_rank = 0;
  float lora_scale = 0.f;
  bool lora_on = false;
};

namespace {

thread_local char g_err[512] = "";

// Optional event pairs bracketing one kernel launch (measurement only).
thread_local hipEvent_t g_timer[DLM_TIMER_COUNT][2] = {};

struct TimerScope {
  int k;
  hipStream_t s;
  bool on;
  TimerScope(int kernel, hipStream_t st, bool enabled = true) : k(kernel), s(st), on(enabled && g_timer[kernel][0]) {
    if (on) (void)hipEventRecord(g_timer[k][0], s);
  }
  ~TimerScope() {
    if (on) (void)hipEventRecord(g_timer[k][1], s);
  }
};

dlm_status fail(dlm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dlm_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return DLM_OK;
  return fail(DLM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define DLM_TRY(expr, what)                                \
  do {                                                     \
    dlm_status _s = hip_check((expr), (what));             \
    if (_s != DLM_OK) return _s;                           \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// K dimension accepted by the GEMMs: a multiple of 256, or a multiple of 64 up to 256.
bool gemm_k_ok(long k) { return k > 0 && (k % 256 == 0 || (k <= 256 && k % 64 == 0)); }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Carves the workspace of one pass.  With base == 0 it only measures.
struct Carver {
  uintptr_t base;
  size_t off = 0;
  template <class T>
  T* take(size_t n) {
    off = align256(off);
    T* p = reinterpret_cast<T*>(base + off);
    off += n * sizeof(T);
    return p;
  }
};

struct PassBufs {
  float* x;
  bf16_t* xn;
  bf16_t* qkv;
  bf16_t* attn;
  bf16_t* u;
  float2* tab;
  float* part_o;
  float* part_ml;
  int* rows;
  int* count;
  float4* head_part;
  float* kpart;  // K-split partials of the layer projections (short passes only)
  bf16_t* lora_t;  // [R][DLM_MAX_LORA_RANK] adapter activations (o A^T)
  size_t bytes;
};

int qkv_dim(const dlm_config& c) { return (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; }

// attention partial floats: exact for (B, Lq, max_kv), or a bound over every
// split of R rows into batch x tokens when B == 0.
size_t attn_floats(const dlm_config& c, int R, int B, int Lq, int max_kv) {
  if (B > 0) {
    AttnArgs a{};
    a.B = B;
    a.Lq = Lq;
    a.H = c.n_heads;
    a.G = c.n_kv_heads;
    a.hd = c.head_dim;
    a.max_kv = max_kv;
    const int splits = attn_splits(a, nullptr);
    return attn_partial_floats(splits, B * Lq, c.n_heads, c.head_dim);
  }
  return attn_partial_floats_bound(R, c.n_heads, c.n_kv_heads, c.head_dim, max_kv);
}

size_t head_part_records(const dlm_config& c, int R, bool bound) {
  size_t r = static_cast<size_t>(c.vocab / gemm_head_tile_n(R)) * R;
  if (bound) r = std::max(r, static_cast<size_t>(c.vocab / gemm_head_tile_n(std::min(R, 64))) * std::min(R, 64));
  return r;
}

// Workspace of the largest K-split layer projection over R rows, or with
// `bound` over every row count r <= R.  The split count of a product falls as
// its rows fill more tiles, so S(r) * r is not monotone in r (the down
// projection at 483 rows takes 8 splits, at 544 rows 6): the bound takes the
// largest value over the row counts where it can peak.  S(r) only changes
// where the count of 128-row (or 256-row) tiles changes, or at 64 rows (short
// products: S does not depend on r), so within each interval (128(k-1), 128k]
// S is constant and S * r peaks at its right end.
size_t layer_gemm_ws(const dlm_config& c, int R, bool bound) {
  const int d = c.d_model, qd = c.n_heads * c.head_dim;
  size_t b = 0;
  auto at = [&](int r) {
    b = std::max(b, gemm_workspace_bytes(r, qkv_dim(c), d));
    b = std::max(b, gemm_workspace_bytes(r, d, qd));
    b = std::max(b, gemm_workspace_bytes(r, 2 * c.d_ffn, d));
    b = std::max(b, gemm_workspace_bytes(r, d, c.d_ffn));
    for (int rank = 128; rank <= DLM_MAX_LORA_RANK; rank += 128) {  // adapter: o A^T, then (.) B^T
      b = std::max(b, gemm_workspace_bytes(r, rank, qd));
      b = std::max(b, gemm_workspace_bytes(r, d, rank));
    }
  };
  at(R);
  if (bound) {
    at(std::min(R, 64));
    for (int r = 128; r < R; r += 128) at(r);
  }
  return b;
}

PassBufs carve(const dlm_config& c, uintptr_t base, int R, int B, int Lq, int max_kv, bool bound) {
  Carver cv{base};
  PassBufs p{};
  p.x = cv.take<float>(static_cast<size_t>(R) * c.d_model);
  p.xn = cv.take<bf16_t>(static_cast<size_t>(R) * c.d_model);
  p.qkv = cv.take<bf16_t>(static_cast<size_t>(R) * qkv_dim(c));
  p.attn = cv.take<bf16_t>(static_cast<size_t>(R) * c.n_heads * c.head_dim);
  p.u = cv.take<bf16_t>(static_cast<size_t>(R) * c.d_ffn);
  p.tab = cv.take<float2>(static_cast<size_t>(R) * (c.head_dim / 2));
  const size_t af = attn_floats(c, R, bound ? 0 : B, Lq, max_kv);
  const size_t per = static_cast<size_t>(c.head_dim + 2);
  p.part_o = cv.take<float>(af / per * c.head_dim);
  p.part_ml = cv.take<float>(af / per * 2);
  p.rows = cv.take<int>(R);
  p.count = cv.take<int>(1);
  p.head_part = cv.take<float4>(head_part_records(c, R, bound));
  p.kpart = cv.take<float>(layer_gemm_ws(c, R, bound) / sizeof(float));
  p.lora_t = cv.take<bf16_t>(static_cast<size_t>(R) * DLM_MAX_LORA_RANK);
  p.bytes = align256(cv.off);
  return p;
}

dlm_status check_model(const dlm_model* m) {
  if (!m) return fail(DLM_ERR_INVALID_ARG, "model is NULL");
  return DLM_OK;
}

dlm_status check_kv(const dlm_model* m, const dlm_kv* kv, int B) {
  if (!kv || !kv->k || !kv->v) return fail(DLM_ERR_INVALID_ARG, "kv cache or its k/v pointer is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(DLM_ERR_INVALID_ARG, "kv pointers must be 16-byte aligned");
  if (kv->capacity <= 0 || kv->capacity % 64 != 0)
    return fail(DLM_ERR_SHAPE, "kv capacity %d must be a positive multiple of 64", kv->capacity);
  if (B < 1 || B > kv->batch) return fail(DLM_ERR_SHAPE, "batch %d must be in [1, kv batch %d]", B, kv->batch);
  (void)m;
  return DLM_OK;
}

size_t layer_kv_elems(const dlm_config& c, const dlm_kv* kv) {
  return static_cast<size_t>(kv->batch) * c.n_kv_heads * kv->capacity * c.head_dim;
}

// The decoder stack over B*Lq rows whose query j of row b sits at
// prefix[b] + pos_offset + j; leaves the final residual stream in p.x.  With
// defer_splits, a K-split last down projection leaves its partials in p.kpart
// unsummed and *defer_splits = their count (0 when p.x is complete): the caller
// adds them to the rows it reads.
dlm_status run_layers(const dlm_model* m, const dlm_kv* kv, const int32_t* tokens, int tok_ld, int B, int Lq,
                      const int32_t* prefix, int pos_offset, int causal, int max_kv, int32_t* flags,
                      const PassBufs& p, hipStream_t s, int* defer_splits = nullptr) {
  if (defer_splits) *defer_splits = 0;
  const dlm_config& c = m->c;
  const int R = B * Lq;
  const int d = c.d_model, qd = c.n_heads * c.head_dim, nq = qkv_dim(c);
  DLM_TRY(embed_norm(tokens, R, Lq, tok_ld, m->embed, c.vocab, d, m->attn_norm[0], c.rms_eps, p.x, p.xn,
                     flags ? flags + 1 : nullptr, prefix, pos_offset, c.head_dim, c.rope_base, p.tab, s),
          "embed_norm");
  // x += A W^T; with gain, then xn = RMSNorm(x) * gain.  Short products split
  // over K fuse their reduction with the norm (one kernel instead of two).
  auto resid_gemm = [&](const GemmArgs& g, const void* gain, const char* what) -> dlm_status {
    const int S = gemm_ksplit(g.M, g.N, g.K);
    if (gain && S > 1 && g.alpha == 1.f) {
      DLM_TRY(gemm_partials(g, s), what);
      DLM_TRY(resid_norm(p.kpart, S, R, p.x, d, gain, c.rms_eps, p.xn, s), "residual + rmsnorm");
      return DLM_OK;
    }
    DLM_TRY(gemm(g, EPI_RESID_F32, s), what);
    if (gain) DLM_TRY(rmsnorm(p.x, R, d, gain, c.rms_eps, p.xn, nullptr, nullptr, s), "rmsnorm");
    return DLM_OK;
  };
  const size_t lkv = layer_kv_elems(c, kv);
  dlm_status st;
  for (int l = 0; l < c.n_layers; ++l) {
    bf16_t* kc = static_cast<bf16_t*>(kv->k) + l * lkv;
    bf16_t* vc = static_cast<bf16_t*>(kv->v) + l * lkv;
    // p.xn holds RMSNorm(x) * attn_norm[l]: from embed_norm (layer 0) or the
    // previous layer's down projection
    GemmArgs g{};
    g.kpart = p.kpart;
    g.a = p.xn;
    g.w = m->wqkv[l];
    g.out = p.qkv;
    g.M = R;
    g.N = nq;
    g.K = d;
    g.lda = d;
    g.ldc = nq;
    // short products split over K sum their partials inside the RoPE + cache
    // write (the QKV timer then covers that kernel too)
    const int qs = gemm_ksplit(R, nq, d);
    if (qs > 1) {
      TimerScope t(DLM_TIMER_QKV, s, l == 0);
      DLM_TRY(gemm_partials(g, s), "gemm qkv");
      DLM_TRY(rope_kv(p.qkv, R, Lq, c.n_heads, c.n_kv_heads, c.head_dim, p.tab, kc, vc, prefix, pos_offset,
                      kv->capacity, s, p.kpart, qs),
              "rope_kv");
    } else {
      {
        TimerScope t(DLM_TIMER_QKV, s, l == 0);
        DLM_TRY(gemm(g, EPI_STORE_BF16, s), "gemm qkv");
      }
      DLM_TRY(rope_kv(p.qkv, R, Lq, c.n_heads, c.n_kv_heads, c.head_dim, p.tab, kc, vc, prefix, pos_offset,
                      kv->capacity, s),
              "rope_kv");
    }
    AttnArgs a{};
    a.q = p.qkv;
    a.ldq = nq;
    a.kc = kc;
    a.vc = vc;
    a.o = p.attn;
    a.prefix = prefix;
    a.pos_offset = pos_offset;
    a.B = B;
    a.Lq = Lq;
    a.H = c.n_heads;
    a.G = c.n_kv_heads;
    a.hd = c.head_dim;
    a.cap = kv->capacity;
    a.causal = causal;
    a.max_kv = max_kv;
    a.part_o = p.part_o;
    a.part_ml = p.part_ml;
    {
      TimerScope t(DLM_TIMER_ATTENTION, s, l == 0);
      DLM_TRY(attention(a, s), "attention");
    }
    g.a = p.attn;
    g.w = m->wo[l];
    g.out = p.x;
    g.N = d;
    g.K = qd;
    g.lda = qd;
    g.ldc = d;
    {
      TimerScope t(DLM_TIMER_O, s, l == 0);
      if ((st = resid_gemm(g, m->lora_on ? nullptr : m->ffn_norm[l], "gemm o")) != DLM_OK) return st;
    }
    if (m->lora_on) {  // x += scale * (o A^T) B^T, then the FFN norm
      GemmArgs la{};
      la.kpart = p.kpart;
      la.a = p.attn;
      la.w = m->lora_a[l];
      la.out = p.lora_t;
      la.M = R;
      la.N = m->lora_rank;
      la.K = qd;
      la.lda = qd;
      la.ldc = m->lora_rank;
      DLM_TRY(gemm(la, EPI_STORE_BF16, s), "gemm lora a");
      la.a = p.lora_t;
      la.w = m->lora_b[l];
      la.out = p.x;
      la.N = d;
      la.K = m->lora_rank;
      la.lda = m->lora_rank;
      la.ldc = d;
      la.alpha = m->lora_scale;
      if ((st = resid_gemm(la, m->ffn_norm[l], "gemm lora b")) != DLM_OK) return st;
    }
    g.a = p.xn;
    g.w = m->wgu[l];
    g.out = p.u;
    g.N = 2 * c.d_ffn;
    g.K = d;
    g.lda = d;
    g.ldc = c.d_ffn;
    {
      TimerScope t(DLM_TIMER_GATE_UP, s, l == 0);
      DLM_TRY(gemm(g, EPI_SWIGLU, s), "gemm gate/up");
    }
    g.a = p.u;
    g.w = m->wdown[l];
    g.out = p.x;
    g.N = d;
    g.K = c.d_ffn;
    g.lda = c.d_ffn;
    g.ldc = d;
    {
      // with the next layer's attention norm (the last layer's final norm is the caller's)
      TimerScope t(DLM_TIMER_DOWN, s, l == 0);
      const int S = gemm_ksplit(g.M, g.N, g.K);
      if (l + 1 == c.n_layers && defer_splits && S > 1) {
        DLM_TRY(gemm_partials(g, s), "gemm down");
        *defer_splits = S;
      } else if ((st = resid_gemm(g, l + 1 < c.n_layers ? m->attn_norm[l + 1] : nullptr, "gemm down")) !=
                 DLM_OK) {
        return st;
      }
    }
  }
  return DLM_OK;
}

// Final norm of the selected rows (all R if rows == null; skipped when the
// caller already normalised them into p.xn) and the fused head.
dlm_status run_head(const dlm_model* m, int R, const int* rows, const int* count, const int* out_rows, float* conf,
                    int32_t* argmax, float* logits, int32_t* flags, const PassBufs& p, hipStream_t s,
                    bool time_head, bool norm = true, float* entropy = nullptr) {
  const dlm_config& c = m->c;
  if (norm) DLM_TRY(rmsnorm(p.x, R, c.d_model, m->final_norm, c.rms_eps, p.xn, rows, count, s), "final norm");
  GemmArgs g{};
  g.a = p.xn;
  g.w = m->lm_head;
  g.M = R;
  g.N = c.vocab;
  g.K = c.d_model;
  g.lda = c.d_model;
  g.m_dev = count;
  g.partials = p.head_part;
  g.logits = logits;
  g.logit_rows = out_rows;
  g.mask_id = c.mask_id;
  g.nonfinite = flags;
  {
    TimerScope t(DLM_TIMER_LM_HEAD, s, time_head);
    DLM_TRY(gemm(g, EPI_HEAD, s), "lm head");
  }
  DLM_TRY(head_merge(p.head_part, c.vocab / gemm_head_tile_n(R), R, out_rows, count, conf, argmax, R, s, entropy),
          "head merge");
  return DLM_OK;
}

}  // namespace

extern "C" {

const char* dlm_status_string(dlm_status s) {
  switch (s) {
    case DLM_OK: return "ok";
    case DLM_ERR_INVALID_ARG: return "invalid argument";
    case DLM_ERR_SHAPE: return "bad shape";
    case DLM_ERR_CAPACITY: return "kv cache capacity exceeded";
    case DLM_ERR_UNSUPPORTED: return "unsupported shape";
    case DLM_ERR_HIP: return "hip launch error";
    case DLM_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* dlm_last_error(void) { return g_err; }

dlm_status dlm_set_kernel_timer(int32_t kernel, void* start_event, void* stop_event) {
  g_err[0] = 0;
  if (kernel < 0 || kernel >= DLM_TIMER_COUNT) return fail(DLM_ERR_INVALID_ARG, "unknown timer kernel %d", kernel);
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(DLM_ERR_INVALID_ARG, "start and stop events must both be given or both NULL");
  g_timer[kernel][0] = static_cast<hipEvent_t>(start_event);
  g_timer[kernel][1] = static_cast<hipEvent_t>(stop_event);
  return DLM_OK;
}

dlm_status dlm_model_create(const dlm_config* cfg, const dlm_weights* w, dlm_model** out) {
  g_err[0] = 0;
  if (!cfg || !w || !out) return fail(DLM_ERR_INVALID_ARG, "NULL config, weights or output handle");
  const dlm_config& c = *cfg;
  if (c.n_layers < 1 || c.d_model < 1 || c.n_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 || c.d_ffn < 1 ||
      c.vocab < 1)
    return fail(DLM_ERR_SHAPE, "all model sizes must be positive");
  if (c.head_dim != 32 && c.head_dim != 128) return fail(DLM_ERR_UNSUPPORTED, "head_dim %d (need 32 or 128)", c.head_dim);
  if (c.n_heads % c.n_kv_heads != 0) return fail(DLM_ERR_SHAPE, "n_heads %% n_kv_heads != 0");
  const int gs = c.n_heads / c.n_kv_heads;
  if (gs != 1 && gs != 2 && gs != 4) return fail(DLM_ERR_UNSUPPORTED, "query heads per KV head %d (need 1, 2 or 4)", gs);
  if (!gemm_k_ok(c.d_model) || !gemm_k_ok(static_cast<long>(c.n_heads) * c.head_dim) || !gemm_k_ok(c.d_ffn))
    return fail(DLM_ERR_UNSUPPORTED, "d_model, n_heads*head_dim and d_ffn must be multiples of 256 (or of 64 up to 256)");
  if (qkv_dim(c) % 128 || c.d_model % 128 || (2 * c.d_ffn) % 128 || c.vocab % 256)
    return fail(DLM_ERR_UNSUPPORTED, "(H+2G)*hd, d_model and 2*d_ffn must be multiples of 128, vocab of 256");
  if (c.d_model > 8192)  // the row kernels (embedding, residual + norm) run one thread per 8 columns
    return fail(DLM_ERR_UNSUPPORTED, "d_model %d > 8192", c.d_model);
  if (c.mask_id < 0 || c.mask_id >= c.vocab) return fail(DLM_ERR_INVALID_ARG, "mask_id %d outside [0, %d)", c.mask_id, c.vocab);
  if (!(std::isfinite(c.rope_base) && c.rope_base > 0.f)) return fail(DLM_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (!(std::isfinite(c.rms_eps) && c.rms_eps > 0.f)) return fail(DLM_ERR_INVALID_ARG, "rms_eps must be finite and > 0");
  const void* top[3] = {w->embed, w->final_norm, w->lm_head};
  for (const void* p : top)
    if (!p || !aligned16(p)) return fail(DLM_ERR_INVALID_ARG, "embed/final_norm/lm_head NULL or not 16-byte aligned");
  const void* const* arrs[6] = {w->attn_norm, w->wqkv, w->wo, w->ffn_norm, w->wgu, w->wdown};
  for (const void* const* a : arrs) {
    if (!a) return fail(DLM_ERR_INVALID_ARG, "a per-layer weight array is NULL");
    for (int l = 0; l < c.n_layers; ++l)
      if (!a[l] || !aligned16(a[l])) return fail(DLM_ERR_INVALID_ARG, "layer %d weight NULL or not 16-byte aligned", l);
  }
  dlm_model* m = new (std::nothrow) dlm_model();
  if (!m) return fail(DLM_ERR_INVALID_ARG, "out of host memory");
  m->c = c;
  m->embed = w->embed;
  m->final_norm = w->final_norm;
  m->lm_head = w->lm_head;
  m->attn_norm.assign(w->attn_norm, w->attn_norm + c.n_layers);
  m->wqkv.assign(w->wqkv, w->wqkv + c.n_layers);
  m->wo.assign(w->wo, w->wo + c.n_layers);
  m->ffn_norm.assign(w->ffn_norm, w->ffn_norm + c.n_layers);
  m->wgu.assign(w->wgu, w->wgu + c.n_layers);
  m->wdown.assign(w->wdown, w->wdown + c.n_layers);
  *out = m;
  return DLM_OK;
}

void dlm_model_destroy(dlm_model* m) { delete m; }

dlm_status dlm_model_set_lora(dlm_model* m, const void* const* a, const void* const* b, int32_t rank, float scale) {
  g_err[0] = 0;
  if (!m) return fail(DLM_ERR_INVALID_ARG, "model is NULL");
  if (!a && !b) {
    m->lora_a.clear();
    m->lora_b.clear();
    m->lora_rank = 0;
    m->lora_on = false;
    return DLM_OK;
  }
  if (!a || !b) return fail(DLM_ERR_INVALID_ARG, "adapter needs both A and B pointer arrays");
  if (rank < 128 || rank > DLM_MAX_LORA_RANK || rank % 128)
    return fail(DLM_ERR_UNSUPPORTED, "adapter rank %d must be a multiple of 128 up to %d", rank, DLM_MAX_LORA_RANK);
  if (!std::isfinite(scale)) return fail(DLM_ERR_INVALID_ARG, "adapter scale must be finite");
  for (int l = 0; l < m->c.n_layers; ++l)
    if (!a[l] || !b[l] || !aligned16(a[l]) || !aligned16(b[l]))
      return fail(DLM_ERR_INVALID_ARG, "adapter matrices of layer %d NULL or not 16-byte aligned", l);
  m->lora_a.assign(a, a + m->c.n_layers);
  m->lora_b.assign(b, b + m->c.n_layers);
  m->lora_rank = rank;
  m->lora_scale = scale;
  m->lora_on = false;
  return DLM_OK;
}

dlm_status dlm_model_enable_lora(dlm_model* m, int32_t on) {
  g_err[0] = 0;
  if (!m) return fail(DLM_ERR_INVALID_ARG, "model is NULL");
  if (on && m->lora_rank == 0) return fail(DLM_ERR_INVALID_ARG, "no adapter set (dlm_model_set_lora)");
  m->lora_on = on != 0;
  return DLM_OK;
}

size_t dlm_workspace_bytes(const dlm_model* m, int32_t max_rows, int32_t max_kv) {
  if (!m || max_rows < 1 || max_kv < 1) return 0;
  return carve(m->c, 0, max_rows, 0, 0, max_kv, true).bytes;
}

static dlm_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(DLM_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(DLM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(DLM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  return DLM_OK;
}

dlm_status dlm_prefill(const dlm_model* m, const dlm_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                       int32_t* prefix_len, int32_t* last_argmax, float* last_conf, int32_t* flags, void* ws,
                       size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dlm_status st = check_model(m);
  if (st != DLM_OK) return st;
  if ((st = check_kv(m, kv, B)) != DLM_OK) return st;
  if (T < 1) return fail(DLM_ERR_SHAPE, "prompt length %d < 1", T);
  if (T > kv->capacity) return fail(DLM_ERR_CAPACITY, "prompt length %d > capacity %d", T, kv->capacity);
  if (!tokens || !prefix_len || !aligned4(tokens) || !aligned4(prefix_len))
    return fail(DLM_ERR_INVALID_ARG, "tokens/prefix_len NULL or misaligned");
  if ((last_argmax == nullptr) != (last_conf == nullptr))
    return fail(DLM_ERR_INVALID_ARG, "last_argmax and last_conf must both be given or both NULL");
  // Passes of C positions: C = T if it fits, else the largest multiple of 32
  // that does.  Every pass (the shorter last one included, and every prefix
  // length a pass reads) is covered by the bound over B*C rows and T keys:
  // each buffer of a pass is no larger than its bound.
  int C = T;
  auto need = [&](int cc) { return carve(m->c, 0, B * cc, 0, 0, T, true).bytes; };
  if (!ws || ws_bytes < need(C)) {
    // the bound grows with the rows: binary search over multiples of 32
    int lo = 0, hi = T / 32;  // need(32 lo) fits (lo = 0: none yet), need(32 (hi + 1)) does not
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (ws_bytes >= need(32 * mid)) lo = mid;
      else hi = mid - 1;
    }
    C = 32 * lo;
    if (C < 32) return fail(DLM_ERR_WORKSPACE, "workspace %zu bytes cannot hold a 32-position pass (%zu)", ws_bytes,
                            need(std::min(T, 32)));
  }
  if ((st = check_ws(ws, ws_bytes, need(C))) != DLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int c0 = 0; c0 < T; c0 += C) {
    const int Lq = std::min(C, T - c0);
    const PassBufs p = carve(m->c, reinterpret_cast<uintptr_t>(ws), B * Lq, B, Lq, c0 + Lq, false);
    if ((st = run_layers(m, kv, tokens + c0, T, B, Lq, nullptr, c0, 1, c0 + Lq, flags, p, s)) != DLM_OK) return st;
    if (c0 + Lq == T && last_argmax) {
      DLM_TRY(strided_rows(p.rows, B, Lq - 1, Lq, s), "rows");
      // head over rows b*Lq + Lq - 1; results land at index b
      const dlm_config& cfg = m->c;
      DLM_TRY(rmsnorm(p.x, B, cfg.d_model, m->final_norm, cfg.rms_eps, p.xn, p.rows, nullptr, s), "final norm");
      GemmArgs g{};
      g.a = p.xn;
      g.w = m->lm_head;
      g.M = B;
      g.N = cfg.vocab;
      g.K = cfg.d_model;
      g.lda = cfg.d_model;
      g.partials = p.head_part;
      g.mask_id = cfg.mask_id;
      g.nonfinite = flags;
      DLM_TRY(gemm(g, EPI_HEAD, s), "lm head");
      DLM_TRY(head_merge(p.head_part, cfg.vocab / gemm_head_tile_n(B), B, nullptr, nullptr, last_conf, last_argmax, B,
                         s),
              "head merge");
    }
  }
  DLM_TRY(set_prefix(prefix_len, B, 0, T, s), "set prefix");
  return DLM_OK;
}

static dlm_status check_block_call(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len, int32_t max_prefix,
                                   const int32_t* canvas, int32_t B, int32_t L) {
  dlm_status st = check_model(m);
  if (st != DLM_OK) return st;
  if ((st = check_kv(m, kv, B)) != DLM_OK) return st;
  if (L < 1 || L > 64) return fail(DLM_ERR_SHAPE, "block length %d must be in [1, 64]", L);
  if (max_prefix < 0) return fail(DLM_ERR_INVALID_ARG, "max_prefix %d < 0", max_prefix);
  if (static_cast<long>(max_prefix) + L > kv->capacity)
    return fail(DLM_ERR_CAPACITY, "max_prefix %d + L %d > capacity %d", max_prefix, L, kv->capacity);
  if (!prefix_len || !canvas || !aligned4(prefix_len) || !aligned4(canvas))
    return fail(DLM_ERR_INVALID_ARG, "prefix_len/canvas NULL or misaligned");
  return DLM_OK;
}

dlm_status dlm_denoise_step(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len, int32_t max_prefix,
                            const int32_t* canvas, const uint8_t* masked, int32_t B, int32_t L, float* conf,
                            int32_t* argmax, float* logits, int32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  return dlm_denoise_step_ex(m, kv, prefix_len, max_prefix, canvas, masked, B, L, conf, argmax, nullptr, logits,
                             flags, ws, ws_bytes, stream);
}

dlm_status dlm_denoise_step_ex(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len, int32_t max_prefix,
                               const int32_t* canvas, const uint8_t* masked, int32_t B, int32_t L, float* conf,
                               int32_t* argmax, float* entropy, float* logits, int32_t* flags, void* ws,
                               size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dlm_status st = check_block_call(m, kv, prefix_len, max_prefix, canvas, B, L);
  if (st != DLM_OK) return st;
  if (!masked || !conf || !argmax || !aligned4(conf) || !aligned4(argmax))
    return fail(DLM_ERR_INVALID_ARG, "masked/conf/argmax NULL or misaligned");
  if (entropy && !aligned4(entropy)) return fail(DLM_ERR_INVALID_ARG, "entropy misaligned");
  if (logits && !aligned16(logits)) return fail(DLM_ERR_INVALID_ARG, "logits must be 16-byte aligned");
  const int R = B * L, max_kv = max_prefix + L;
  const size_t need = carve(m->c, 0, R, B, L, max_kv, false).bytes;
  if ((st = check_ws(ws, ws_bytes, need)) != DLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PassBufs p = carve(m->c, reinterpret_cast<uintptr_t>(ws), R, B, L, max_kv, false);
  // the last down projection's K-split partials are summed by the final norm,
  // for the masked rows only
  int splits = 0;
  if ((st = run_layers(m, kv, canvas, L, B, L, prefix_len, 0, 0, max_kv, flags, p, s, &splits)) != DLM_OK)
    return st;
  {
    TimerScope t(DLM_TIMER_FINAL_NORM, s);
    DLM_TRY(masked_norm(masked, R, p.x, m->c.d_model, m->final_norm, m->c.rms_eps, p.xn, p.rows, p.count, s,
                        p.kpart, splits),
            "masked rows + final norm");
  }
  return run_head(m, R, p.rows, p.count, p.rows, conf, argmax, logits, flags, p, s, true, false, entropy);
}

// ----------------------------------------------- allocation-free step ----
// The scratch of dlm_denoise_step_noalloc: one fixed array per GPU, in the code
// object's device memory.  In host code `scratch` names a host-side stand-in,
// not a device address: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[DLM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

dlm_status scratch_of_current_device(void** out) {
  int dev = -1;
  DLM_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DLM_ERR_HIP, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    DLM_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return fail(DLM_ERR_HIP, "scratch address %p unusable", p);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DLM_OK;
}
}  // namespace

dlm_status dlm_denoise_step_noalloc(const dlm_model* m, const dlm_kv* kv, const int32_t* prefix_len,
                                    int32_t max_prefix, const int32_t* canvas, const uint8_t* masked, int32_t B,
                                    int32_t L, float* conf, int32_t* argmax, float* entropy, float* logits,
                                    int32_t* flags, void* stream) {
  g_err[0] = 0;
  dlm_status st = check_block_call(m, kv, prefix_len, max_prefix, canvas, B, L);
  if (st != DLM_OK) return st;
  // the pass's exact workspace (the same carve dlm_denoise_step_ex makes),
  // checked against the fixed scratch before any device call
  const size_t need = carve(m->c, 0, B * L, B, L, max_prefix + L, false).bytes;
  if (need > DLM_NOALLOC_SCRATCH_BYTES)
    return fail(DLM_ERR_WORKSPACE, "this pass needs %zu bytes of scratch, the fixed scratch holds %zu", need,
                static_cast<size_t>(DLM_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != DLM_OK) return st;
  return dlm_denoise_step_ex(m, kv, prefix_len, max_prefix, canvas, masked, B, L, conf, argmax, entropy, logits,
                             flags, ws, DLM_NOALLOC_SCRATCH_BYTES, stream);
}

dlm_status dlm_commit(const float* conf, const int32_t* argmax, int32_t* canvas, uint8_t* masked, int32_t B,
                      int32_t L, const float* threshold, const int32_t* quota, int32_t* steps, int32_t max_steps,
                      int32_t* n_committed, int32_t* n_left, void* stream) {
  g_err[0] = 0;
  if (B < 1) return fail(DLM_ERR_SHAPE, "batch %d < 1", B);
  if (L < 1 || L > 64) return fail(DLM_ERR_SHAPE, "block length %d must be in [1, 64]", L);
  if (max_steps < 1) return fail(DLM_ERR_INVALID_ARG, "max_steps %d < 1", max_steps);
  const void* ps[] = {conf, argmax, canvas, threshold, quota, steps, n_committed, n_left};
  for (const void* p : ps)
    if (!p || !aligned4(p)) return fail(DLM_ERR_INVALID_ARG, "a commit buffer is NULL or misaligned");
  if (!masked) return fail(DLM_ERR_INVALID_ARG, "masked is NULL");
  DLM_TRY(dlm::commit(conf, argmax, canvas, masked, B, L, threshold, quota, steps, max_steps, n_committed, n_left,
                      static_cast<hipStream_t>(stream)),
          "commit");
  return DLM_OK;
}

dlm_status dlm_commit_ex(const float* conf, const int32_t* argmax, const float* entropy, int32_t* canvas,
                         uint8_t* masked, int32_t B, int32_t L, const float* threshold, const int32_t* quota,
                         int32_t* steps, int32_t max_steps, const dlm_commit_opts* opts, int32_t* n_committed,
                         int32_t* n_left, void* stream) {
  g_err[0] = 0;
  if (B < 1) return fail(DLM_ERR_SHAPE, "batch %d < 1", B);
  if (L < 1 || L > 64) return fail(DLM_ERR_SHAPE, "block length %d must be in [1, 64]", L);
  if (max_steps < 1) return fail(DLM_ERR_INVALID_ARG, "max_steps %d < 1", max_steps);
  if (!opts) return fail(DLM_ERR_INVALID_ARG, "opts is NULL");
  const void* ps[] = {conf, argmax, canvas, threshold, quota, steps, n_committed, n_left};
  for (const void* p : ps)
    if (!p || !aligned4(p)) return fail(DLM_ERR_INVALID_ARG, "a commit buffer is NULL or misaligned");
  if (!masked) return fail(DLM_ERR_INVALID_ARG, "masked is NULL");
  const dlm_commit_opts& o = *opts;
  if (o.rule < DLM_RULE_THRESHOLD || o.rule > DLM_RULE_ENTROPY) return fail(DLM_ERR_INVALID_ARG, "rule %d", o.rule);
  if (!std::isfinite(o.min_threshold) || !std::isfinite(o.scaling) || !std::isfinite(o.entropy_bound) ||
      !std::isfinite(o.stop_entropy))
    return fail(DLM_ERR_INVALID_ARG, "non-finite sampler parameter");
  if (o.max_transfer < 0 || o.stability_steps < 0)
    return fail(DLM_ERR_INVALID_ARG, "max_transfer %d / stability_steps %d < 0", o.max_transfer, o.stability_steps);
  if ((o.rule == DLM_RULE_ENTROPY || o.stability_steps > 0) && (!entropy || !aligned4(entropy)))
    return fail(DLM_ERR_INVALID_ARG, "the entropy rule and adaptive stopping need aligned entropies");
  if (o.stability_steps > 0 && (!o.prev_argmax || !o.stable || !aligned4(o.prev_argmax) || !aligned4(o.stable)))
    return fail(DLM_ERR_INVALID_ARG, "adaptive stopping needs prev_argmax and stable buffers");
  CommitOpts co;
  co.rule = o.rule;
  co.min_threshold = o.min_threshold;
  co.scaling = o.scaling;
  co.entropy_bound = o.entropy_bound;
  co.max_transfer = o.max_transfer;
  co.stability_steps = o.stability_steps;
  co.stop_entropy = o.stop_entropy;
  co.prev_argmax = o.prev_argmax;
  co.stable = o.stable;
  DLM_TRY(dlm::commit(conf, argmax, canvas, masked, B, L, threshold, quota, steps, max_steps, n_committed, n_left,
                      static_cast<hipStream_t>(stream), entropy, &co),
          "commit");
  return DLM_OK;
}

dlm_status dlm_append_block(const dlm_model* m, const dlm_kv* kv, int32_t* prefix_len, int32_t max_prefix,
                            const int32_t* block, int32_t B, int32_t L, int32_t* argmax_out, float* conf_out,
                            int32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dlm_status st = check_block_call(m, kv, prefix_len, max_prefix, block, B, L);
  if (st != DLM_OK) return st;
  if ((argmax_out == nullptr) != (conf_out == nullptr))
    return fail(DLM_ERR_INVALID_ARG, "argmax_out and conf_out must both be given or both NULL");
  const int R = B * L, max_kv = max_prefix + L;
  const size_t need = carve(m->c, 0, R, B, L, max_kv, false).bytes;
  if ((st = check_ws(ws, ws_bytes, need)) != DLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PassBufs p = carve(m->c, reinterpret_cast<uintptr_t>(ws), R, B, L, max_kv, false);
  if ((st = run_layers(m, kv, block, L, B, L, prefix_len, 0, 1, max_kv, flags, p, s)) != DLM_OK) return st;
  if (argmax_out) {
    if ((st = run_head(m, R, nullptr, nullptr, nullptr, conf_out, argmax_out, nullptr, flags, p, s, false)) != DLM_OK)
      return st;
  }
  DLM_TRY(set_prefix(prefix_len, B, 1, L, s), "advance prefix");
  return DLM_OK;
}

// ------------------------------------------------------------ ops ----

size_t dlm_op_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return align256(gemm_workspace_bytes(M, N, K));
}

dlm_status dlm_op_gemm(const void* a, const void* w, void* out, int32_t M, int32_t N, int32_t K, int32_t lda,
                       int32_t ldc, int32_t epilogue, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!a || !w || !out || !aligned16(a) || !aligned16(w) || !aligned16(out))
    return fail(DLM_ERR_INVALID_ARG, "a/w/out NULL or not 16-byte aligned");
  if (M < 1 || N < 1 || N % 128 || !gemm_k_ok(K)) return fail(DLM_ERR_SHAPE, "gemm shape M=%d N=%d K=%d", M, N, K);
  if (lda < K || lda % 8) return fail(DLM_ERR_SHAPE, "lda %d", lda);
  if (epilogue < 0 || epilogue > 2) return fail(DLM_ERR_INVALID_ARG, "epilogue %d", epilogue);
  const int cols = epilogue == DLM_EPI_SWIGLU ? N / 2 : N;
  if (ldc < cols || ldc % 8) return fail(DLM_ERR_SHAPE, "ldc %d", ldc);
  const size_t need = gemm_workspace_bytes(M, N, K);
  if (need > 0 && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256))
    return fail(DLM_ERR_WORKSPACE, "gemm needs %zu bytes of 256-byte aligned workspace, got %zu", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmArgs g{};
  g.kpart = static_cast<float*>(ws);
  g.a = a;
  g.w = w;
  g.out = out;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldc = ldc;
  DLM_TRY(gemm(g, static_cast<GemmEpilogue>(epilogue), s), "gemm");
  return DLM_OK;
}

dlm_status dlm_op_rmsnorm(const float* x, int32_t M, int32_t d, const void* gn, float eps, void* out, void* stream) {
  g_err[0] = 0;
  if (!x || !gn || !out || !aligned16(x) || !aligned16(gn) || !aligned16(out))
    return fail(DLM_ERR_INVALID_ARG, "x/g/out NULL or not 16-byte aligned");
  if (M < 1 || d < 8 || d % 8) return fail(DLM_ERR_SHAPE, "rmsnorm shape M=%d d=%d", M, d);
  if (!(std::isfinite(eps) && eps > 0.f)) return fail(DLM_ERR_INVALID_ARG, "eps");
  DLM_TRY(rmsnorm(x, M, d, gn, eps, out, nullptr, nullptr, static_cast<hipStream_t>(stream)), "rmsnorm");
  return DLM_OK;
}

size_t dlm_op_rope_workspace_bytes(int32_t B, int32_t Lq, int32_t hd) {
  if (B < 1 || Lq < 1 || hd < 2) return 0;
  return align256(static_cast<size_t>(B) * Lq * (hd / 2) * sizeof(float2));
}

dlm_status dlm_op_rope_kv(void* qkv, int32_t B, int32_t Lq, int32_t H, int32_t G, int32_t hd, float rope_base,
                          void* k_cache, void* v_cache, const int32_t* prefix, int32_t pos_offset, int32_t cap,
                          void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!qkv || !k_cache || !v_cache || !aligned16(qkv) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(DLM_ERR_INVALID_ARG, "qkv/k/v NULL or not 16-byte aligned");
  if (B < 1 || Lq < 1 || H < 1 || G < 1 || H % G || (hd != 32 && hd != 128) || cap < 16 || cap % 16)
    return fail(DLM_ERR_SHAPE, "rope shape");
  if (!(std::isfinite(rope_base) && rope_base > 0.f)) return fail(DLM_ERR_INVALID_ARG, "rope_base");
  dlm_status st = check_ws(ws, ws_bytes, dlm_op_rope_workspace_bytes(B, Lq, hd));
  if (st != DLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* tab = static_cast<float2*>(ws);
  DLM_TRY(rope_table(prefix, pos_offset, B, Lq, hd, rope_base, tab, s), "rope table");
  DLM_TRY(rope_kv(qkv, B * Lq, Lq, H, G, hd, tab, k_cache, v_cache, prefix, pos_offset, cap, s), "rope kv");
  return DLM_OK;
}

size_t dlm_op_attention_workspace_bytes(int32_t B, int32_t Lq, int32_t H, int32_t G, int32_t hd, int32_t max_kv) {
  if (B < 1 || Lq < 1 || H < 1 || G < 1 || max_kv < 1) return 0;
  AttnArgs a{};
  a.B = B;
  a.Lq = Lq;
  a.H = H;
  a.G = G;
  a.hd = hd;
  a.max_kv = max_kv;
  const int splits = attn_splits(a, nullptr);
  const size_t f = attn_partial_floats(splits, B * Lq, H, hd);
  return align256(f / (hd + 2) * hd * sizeof(float)) + align256(f / (hd + 2) * 2 * sizeof(float)) + 256;
}

dlm_status dlm_op_attention(const void* q, int32_t ldq, const void* k_cache, const void* v_cache, void* o,
                            const int32_t* prefix, int32_t pos_offset, int32_t B, int32_t Lq, int32_t H, int32_t G,
                            int32_t hd, int32_t cap, int32_t causal, int32_t max_kv, void* ws, size_t ws_bytes,
                            void* stream) {
  g_err[0] = 0;
  if (!q || !k_cache || !v_cache || !o || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(DLM_ERR_INVALID_ARG, "q/k/v/o NULL or not 16-byte aligned");
  if (B < 1 || Lq < 1 || H < 1 || G < 1 || H % G) return fail(DLM_ERR_SHAPE, "attention shape");
  if (hd != 32 && hd != 128) return fail(DLM_ERR_UNSUPPORTED, "head_dim %d", hd);
  const int gs = H / G;
  if (gs != 1 && gs != 2 && gs != 4) return fail(DLM_ERR_UNSUPPORTED, "group size %d", gs);
  if (ldq < H * hd || ldq % 8) return fail(DLM_ERR_SHAPE, "ldq %d", ldq);
  if (cap < 64 || cap % 64) return fail(DLM_ERR_SHAPE, "cap %d", cap);
  if (max_kv < Lq || max_kv > cap) return fail(DLM_ERR_CAPACITY, "max_kv %d outside [Lq, cap]", max_kv);
  dlm_status st = check_ws(ws, ws_bytes, dlm_op_attention_workspace_bytes(B, Lq, H, G, hd, max_kv));
  if (st != DLM_OK) return st;
  AttnArgs a{};
  a.q = q;
  a.ldq = ldq;
  a.kc = k_cache;
  a.vc = v_cache;
  a.o = o;
  a.prefix = prefix;
  a.pos_offset = pos_offset;
  a.B = B;
  a.Lq = Lq;
  a.H = H;
  a.G = G;
  a.hd = hd;
  a.cap = cap;
  a.causal = causal ? 1 : 0;
  a.max_kv = max_kv;
  const int splits = attn_splits(a, nullptr);
  const size_t f = attn_partial_floats(splits, B * Lq, H, hd);
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(f / (hd + 2) * hd * sizeof(float)));
  DLM_TRY(attention(a, static_cast<hipStream_t>(stream)), "attention");
  return DLM_OK;
}

size_t dlm_op_lm_head_workspace_bytes(int32_t R, int32_t V) {
  if (R < 1 || V < 128) return 0;
  return align256(static_cast<size_t>(V / gemm_head_tile_n(R)) * R * sizeof(float4));
}

dlm_status dlm_op_lm_head(const void* hidden, int32_t R, int32_t d, const void* head, int32_t V, int32_t mask_id,
                          float* conf, int32_t* argmax, float* entropy, float* logits, int32_t* flags, void* ws,
                          size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!hidden || !head || !conf || !argmax || !aligned16(hidden) || !aligned16(head) || !aligned4(conf) ||
      !aligned4(argmax))
    return fail(DLM_ERR_INVALID_ARG, "hidden/head/conf/argmax NULL or misaligned");
  if (logits && !aligned16(logits)) return fail(DLM_ERR_INVALID_ARG, "logits must be 16-byte aligned");
  if (entropy && !aligned4(entropy)) return fail(DLM_ERR_INVALID_ARG, "entropy misaligned");
  if (R < 1 || V < 256 || V % 256 || !gemm_k_ok(d)) return fail(DLM_ERR_SHAPE, "lm head shape R=%d V=%d d=%d", R, V, d);
  if (mask_id < 0 || mask_id >= V) return fail(DLM_ERR_INVALID_ARG, "mask_id %d", mask_id);
  dlm_status st = check_ws(ws, ws_bytes, dlm_op_lm_head_workspace_bytes(R, V));
  if (st != DLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmArgs g{};
  g.a = hidden;
  g.w = head;
  g.M = R;
  g.N = V;
  g.K = d;
  g.lda = d;
  g.partials = ws;
  g.logits = logits;
  g.mask_id = mask_id;
  g.nonfinite = flags;
  DLM_TRY(gemm(g, EPI_HEAD, s), "lm head");
  DLM_TRY(head_merge(ws, V / gemm_head_tile_n(R), R, nullptr, nullptr, conf, argmax, R, s, entropy), "head merge");
  return DLM_OK;
}

}  // extern "C"
