// Small kernels of the denoising path: commit/remask, embedding gather + RMSNorm
// (+ the RoPE table), RMSNorm, RoPE + KV-cache write, masked-row compaction +
// final RMSNorm, the cross-tile merge of the LM-head partials, and fills.
#include "dlm_device.h"
#include "dlm_internal.h"

namespace dlm {

// ------------------------------------------------------------ commit ----
// Commit rules, one wavefront per row (L <= 64), lane j = position j.
//
// Native (MLX-VLM Nemotron Labs Diffusion guide, sec. 5.2 native sampler and
// sec. 6; DiffusionGemma docs, BlockRefinementScheduler): A = masked positions
// with conf > tau.  Bounded (the guide's confidence_threshold_bound, sec. 5.2):
// conf >= tau, or conf >= min_threshold and conf >= 1 - scaling / (j + 2).
// Entropy bound (DiffusionGemma docs, EntropyBoundScheduler): masked positions
// in (entropy, position) order while the float32 running sum of their entropies
// stays <= the bound.  Then: on the last allowed step every remaining mask;
// otherwise A when |A| >= q = min(quota, #masked), else A plus the best-ranked
// others up to q; with max_transfer > 0 (the guide's --max-transfer-per-step,
// sec. 5.5) at most that many, the best-ranked.  Rank: (-conf, position), or
// (entropy, position) for the entropy rule.  Chosen positions take their argmax
// token and leave the mask; the others stay masked.
//
// Adaptive stopping (DiffusionGemma docs, adaptive stopping), before the rule:
// stable[b] counts consecutive steps whose argmax at every masked position
// equals prev_argmax; when it reaches stability_steps and the mean entropy of
// the masked positions (float32 sum in position order) is below stop_entropy,
// every remaining mask is committed.  prev_argmax takes this step's argmax.
// Rows with no mask left are frozen (no state changes).
// Lane i's value of v, i uniform (a scalar read, no LDS round trip).
__device__ __forceinline__ float lane_value(float v, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
}

__device__ __forceinline__ bool commit_better(bool by_entropy, float ci, float ei, int i, float cj, float ej, int j) {
  if (by_entropy) return ei < ej || (ei == ej && i < j);
  return ci > cj || (ci == cj && i < j);
}

__global__ void __launch_bounds__(256) k_commit(const float* __restrict__ conf,
                                                const int* __restrict__ argmax, int* __restrict__ canvas,
                                                uint8_t* __restrict__ masked, int B, int L,
                                                const float* __restrict__ tau,
                                                const int* __restrict__ quota, int* __restrict__ steps,
                                                int max_steps, int* __restrict__ n_committed,
                                                int* __restrict__ n_left, const float* __restrict__ entropy,
                                                CommitOpts o) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wavefront
  const size_t base = static_cast<size_t>(b) * L;
  const bool in = lane < L;
  // every input is loaded before any is used (one memory round trip)
  const bool mk = in && masked[base + lane] != 0;
  const float c = in ? conf[base + lane] : 0.f;
  const float e = (in && entropy) ? entropy[base + lane] : 0.f;
  const int st = steps[b];
  const int a = in ? argmax[base + lane] : 0;
  const float tb = tau[b];
  const int qb = quota[b];
  const bool adaptive = o.stability_steps > 0;
  const int prev = (adaptive && in) ? o.prev_argmax[base + lane] : 0;
  const int stable_in = adaptive ? o.stable[b] : 0;
  const unsigned long long mball = __ballot(mk);
  const int cnt = __popcll(mball);
  if (cnt == 0) {
    if (lane == 0) {
      n_committed[b] = 0;
      n_left[b] = 0;
    }
    return;
  }

  bool stop = false;
  if (adaptive) {
    const bool diff = mk && a != prev;
    const int stable = __any(diff) ? 0 : stable_in + 1;
    float total = 0.f;  // sequential, in position order
    for (int i = 0; i < L; ++i) {
      const float ei = lane_value(e, i);
      if ((mball >> i) & 1ull) total = total + ei;
    }
    const float mean = total / static_cast<float>(cnt);
    stop = stable >= o.stability_steps && mean < o.stop_entropy;
    if (mk) o.prev_argmax[base + lane] = a;
    if (lane == 0) o.stable[b] = stable;
  }

  const bool by_ent = o.rule == COMMIT_ENTROPY;
  bool chosen;
  int n;
  if (stop || st >= max_steps - 1) {
    chosen = mk;
    n = cnt;
  } else {
    bool inA;
    if (o.rule == COMMIT_BOUND) {
      inA = mk && (c >= tb || (c >= o.min_threshold && c >= 1.f - o.scaling / static_cast<float>(lane + 2)));
    } else if (o.rule == COMMIT_ENTROPY) {
      // rank among the masked positions by ascending entropy (the only rule
      // that needs every position's rank; the others rank only the positions
      // outside their qualifying set, below)
      int rank = 0;
      for (int i = 0; i < L; ++i) {
        const float ci = lane_value(c, i), ei = lane_value(e, i);
        const bool mi = (mball >> i) & 1ull;
        rank += (mi && commit_better(by_ent, ci, ei, i, c, e, lane)) ? 1 : 0;
      }
      // running sum of the entropies in rank order (float32, sequential)
      float total = 0.f, mine = 0.f;
      for (int r = 0; r < cnt; ++r) {
        const int src = __ffsll(static_cast<long long>(__ballot(mk && rank == r))) - 1;
        total = total + lane_value(e, src);
        if (rank == r) mine = total;
      }
      inA = mk && mine <= o.entropy_bound;
    } else {
      inA = mk && c > tb;
    }
    const unsigned long long aball = __ballot(inA);
    const int nA = __popcll(aball);
    const int q = min(qb, cnt);
    if (nA >= q) {
      chosen = inA;
      n = nA;
    } else {  // A plus the best-ranked others up to q
      int orank = 0;
      for (int i = 0; i < L; ++i) {
        const float ci = lane_value(c, i), ei = lane_value(e, i);
        const bool oi = ((mball & ~aball) >> i) & 1ull;
        orank += (oi && commit_better(by_ent, ci, ei, i, c, e, lane)) ? 1 : 0;
      }
      chosen = inA || (mk && orank < q - nA);
      n = q;
    }
    if (o.max_transfer > 0 && n > o.max_transfer) {
      const unsigned long long cball = __ballot(chosen);
      int crank = 0;
      for (int i = 0; i < L; ++i) {
        const float ci = lane_value(c, i), ei = lane_value(e, i);
        crank += (((cball >> i) & 1ull) && commit_better(by_ent, ci, ei, i, c, e, lane)) ? 1 : 0;
      }
      chosen = chosen && crank < o.max_transfer;
      n = o.max_transfer;
    }
  }
  if (chosen) {
    canvas[base + lane] = a;
    masked[base + lane] = 0;
  }
  if (lane == 0) {
    steps[b] = st + 1;
    n_committed[b] = n;
    n_left[b] = cnt - n;
  }
}

hipError_t commit(const float* conf, const int* argmax, int* canvas, uint8_t* masked, int B, int L,
                  const float* tau, const int* quota, int* steps, int max_steps, int* n_committed,
                  int* n_left, hipStream_t s, const float* entropy, const CommitOpts* opts) {
  const CommitOpts o = opts ? *opts : CommitOpts{};
  hipLaunchKernelGGL(k_commit, dim3((B + 3) / 4), dim3(256), 0, s, conf, argmax, canvas, masked, B, L,
                     tau, quota, steps, max_steps, n_committed, n_left, entropy, o);
  return hipGetLastError();
}

// ------------------------------------------------------------ RMSNorm ----
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) t += red[i];
  __syncthreads();
  return t;
}

// Sum over a workgroup of T threads (wave sums, then the waves in order).
template <int T>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < T / 64; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// Rotation angles for row m = b*Lq + j at absolute position p = prefix[b] + off + j:
// pair i of a head (components i and i + hd/2) turns by p * base^(-2i/hd).  The
// angle is formed in double precision (positions reach 1e5 and beyond), its
// cosine and sine are stored as fp32 and shared by every head and layer.
struct RopeSpec {
  const int* prefix;
  int off, Lq, half;
  double log_base;
  float2* tab;
  int total;  // rows * half entries (0: no table)
};

__device__ __forceinline__ void rope_entry(const RopeSpec& r, int e) {
  const int m = e / r.half, i = e % r.half;
  const int b = m / r.Lq, j = m % r.Lq;
  const double p = static_cast<double>((r.prefix ? r.prefix[b] : 0) + r.off + j);
  const double freq = exp(-2.0 * i / (2.0 * r.half) * r.log_base);
  double sn, cs;
  sincos(p * freq, &sn, &cs);
  r.tab[e] = make_float2(static_cast<float>(cs), static_cast<float>(sn));
}

// Blocks [0, M): x[m] = E[tok[m]] (fp32) and xn[m] = RMSNorm(x[m]) * g (bf16),
// RMSNorm being x / sqrt(mean(x^2) + eps) * g; out-of-range tokens read as
// zeros and are counted.  Blocks past M fill the RoPE table of the pass (one
// launch for both).
template <int T>
__global__ void __launch_bounds__(T) k_embed_norm(const int* __restrict__ tokens, int M, int Lq, int tok_ld,
                                                  const bf16_t* __restrict__ E, int V, int d,
                                                  const bf16_t* __restrict__ g, float eps,
                                                  float* __restrict__ x, bf16_t* __restrict__ xn,
                                                  int* __restrict__ bad, RopeSpec rope) {
  __shared__ float red[T / 64];
  const int m = blockIdx.x;
  if (m >= M) {
    const int e = (m - M) * T + threadIdx.x;
    if (e < rope.total) rope_entry(rope, e);
    return;
  }
  // one thread per 8 columns: the row stays in registers for the normalisation
  const int c = threadIdx.x;
  const bool on = c < d / 8;
  const int t = tokens[static_cast<size_t>(m / Lq) * tok_ld + m % Lq];
  const bool ok = t >= 0 && t < V;
  if (!ok && threadIdx.x == 0 && bad) atomicAdd(bad, 1);
  const bf16_t* row = E + static_cast<size_t>(ok ? t : 0) * d;
  float f[8], gg[8];
  float ss = 0.f;
  if (on) {
    unpack8(ok ? ld16(row + c * 8) : u32x4{0, 0, 0, 0}, f);
    unpack8(ld16(g + c * 8), gg);
    float* xo = x + static_cast<size_t>(m) * d + c * 8;
    *reinterpret_cast<float4*>(xo) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(xo + 4) = make_float4(f[4], f[5], f[6], f[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
  }
  const float rstd = rsqrtf(block_sum<T>(ss, red) / d + eps);
  if (!on) return;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i] * rstd * gg[2 * i], f[2 * i + 1] * rstd * gg[2 * i + 1]);
  st16(xn + static_cast<size_t>(m) * d + c * 8, o);
}

hipError_t embed_norm(const int* tokens, int M, int Lq, int tok_ld, const void* embed, int V, int d,
                      const void* gain, float eps, float* x, void* xn, int* bad_token, const int* prefix,
                      int pos_offset, int hd, float base, float2* tab, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d % 8 || d / 8 > 1024) return hipErrorInvalidValue;
  RopeSpec r{prefix, pos_offset, Lq, hd / 2, log(static_cast<double>(base)), tab, tab ? M * (hd / 2) : 0};
  auto go = [&](auto kern, int T) {
    hipLaunchKernelGGL(kern, dim3(M + (r.total + T - 1) / T), dim3(T), 0, s, tokens, M, Lq, tok_ld,
                       static_cast<const bf16_t*>(embed), V, d, static_cast<const bf16_t*>(gain), eps, x,
                       static_cast<bf16_t*>(xn), bad_token, r);
  };
  const int need = d / 8;
  if (need <= 64)
    go(k_embed_norm<64>, 64);
  else if (need <= 256)
    go(k_embed_norm<256>, 256);
  else if (need <= 512)
    go(k_embed_norm<512>, 512);
  else
    go(k_embed_norm<1024>, 1024);
  return hipGetLastError();
}

// xn[i] = RMSNorm(x[rows ? rows[i] : i]) * g; rows i >= *m_dev are skipped.
__global__ void __launch_bounds__(256) k_rmsnorm(const float* __restrict__ x, int d,
                                                 const bf16_t* __restrict__ g, float eps,
                                                 bf16_t* __restrict__ xn, const int* __restrict__ rows,
                                                 const int* __restrict__ m_dev) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  if (m_dev && i >= *m_dev) return;
  const int src = rows ? rows[i] : i;
  const float* xr = x + static_cast<size_t>(src) * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d / 4; c += 256) {
    const float4 v = reinterpret_cast<const float4*>(xr)[c];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  const float rstd = rsqrtf(block_sum_256(ss, red) / d + eps);
  for (int c = threadIdx.x; c < d / 8; c += 256) {
    const float4 v0 = reinterpret_cast<const float4*>(xr)[2 * c];
    const float4 v1 = reinterpret_cast<const float4*>(xr)[2 * c + 1];
    float gg[8];
    unpack8(ld16(g + c * 8), gg);
    u32x4 o;
    o[0] = pack_bf16x2(v0.x * rstd * gg[0], v0.y * rstd * gg[1]);
    o[1] = pack_bf16x2(v0.z * rstd * gg[2], v0.w * rstd * gg[3]);
    o[2] = pack_bf16x2(v1.x * rstd * gg[4], v1.y * rstd * gg[5]);
    o[3] = pack_bf16x2(v1.z * rstd * gg[6], v1.w * rstd * gg[7]);
    st16(xn + static_cast<size_t>(i) * d + c * 8, o);
  }
}

// Residual update from K-split partials fused with the next RMSNorm:
// x[m] += sum_s part[s][m] (split order), then xn[m] = RMSNorm(x[m]) * g.  One
// workgroup per row, one thread per 8 columns (d / 8 threads, at most 1024):
// every load of the row (the residual and its S partials) is issued at once and
// the updated row stays in registers for the normalisation.
template <int T>
__global__ void __launch_bounds__(T) k_resid_norm(const float* __restrict__ part, int S, int M,
                                                  float* __restrict__ x, int d, const bf16_t* __restrict__ g,
                                                  float eps, bf16_t* __restrict__ xn) {
  __shared__ float red[T / 64];
  const int m = blockIdx.x, c = threadIdx.x;
  const bool on = c < d / 8;
  const size_t plane = static_cast<size_t>(M) * d;
  float* xr = x + static_cast<size_t>(m) * d;
  const float* pr = part + static_cast<size_t>(m) * d;
  float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
  float ss = 0.f;
  // the gains are loaded with the row, not after the block sum: one memory round
  // trip per launch instead of two (the barrier inside block_sum would hold a
  // later load back)
  u32x4 graw = {0, 0, 0, 0};
  if (on) {
    graw = ld16(g + c * 8);
    v0 = reinterpret_cast<const float4*>(xr)[2 * c];
    v1 = reinterpret_cast<const float4*>(xr)[2 * c + 1];
    const float4 a0 = sum_planes(pr + 8 * c, plane, S);
    const float4 a1 = sum_planes(pr + 8 * c + 4, plane, S);
    v0.x += a0.x; v0.y += a0.y; v0.z += a0.z; v0.w += a0.w;
    v1.x += a1.x; v1.y += a1.y; v1.z += a1.z; v1.w += a1.w;
    reinterpret_cast<float4*>(xr)[2 * c] = v0;
    reinterpret_cast<float4*>(xr)[2 * c + 1] = v1;
    ss = v0.x * v0.x + v0.y * v0.y + v0.z * v0.z + v0.w * v0.w + v1.x * v1.x + v1.y * v1.y + v1.z * v1.z +
         v1.w * v1.w;
  }
  const float rstd = rsqrtf(block_sum<T>(ss, red) / d + eps);
  if (!on) return;
  float gg[8];
  unpack8(graw, gg);
  u32x4 o;
  o[0] = pack_bf16x2(v0.x * rstd * gg[0], v0.y * rstd * gg[1]);
  o[1] = pack_bf16x2(v0.z * rstd * gg[2], v0.w * rstd * gg[3]);
  o[2] = pack_bf16x2(v1.x * rstd * gg[4], v1.y * rstd * gg[5]);
  o[3] = pack_bf16x2(v1.z * rstd * gg[6], v1.w * rstd * gg[7]);
  st16(xn + static_cast<size_t>(m) * d + c * 8, o);
}

hipError_t resid_norm(const float* part, int S, int M, float* x, int d, const void* gain, float eps, void* xn,
                      hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (S < 1 || S > SPLIT_MAX || d % 8 || d / 8 > 1024) return hipErrorInvalidValue;
  auto go = [&](auto kern, int T) {
    hipLaunchKernelGGL(kern, dim3(M), dim3(T), 0, s, part, S, M, x, d, static_cast<const bf16_t*>(gain), eps,
                       static_cast<bf16_t*>(xn));
  };
  const int need = d / 8;
  if (need <= 64)
    go(k_resid_norm<64>, 64);
  else if (need <= 256)
    go(k_resid_norm<256>, 256);
  else if (need <= 512)
    go(k_resid_norm<512>, 512);
  else
    go(k_resid_norm<1024>, 1024);
  return hipGetLastError();
}

hipError_t rmsnorm(const float* x, int M, int d, const void* gain, float eps, void* xn, const int* rows,
                   const int* m_dev, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(256), 0, s, x, d, static_cast<const bf16_t*>(gain), eps,
                     static_cast<bf16_t*>(xn), rows, m_dev);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RoPE ----
__global__ void k_rope_table(RopeSpec r) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < r.total) rope_entry(r, e);
}

hipError_t rope_table(const int* prefix, int pos_offset, int B, int Lq, int hd, float base, float2* tab,
                      hipStream_t s) {
  RopeSpec r{prefix, pos_offset, Lq, hd / 2, log(static_cast<double>(base)), tab, B * Lq * (hd / 2)};
  if (r.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((r.total + 255) / 256), dim3(256), 0, s, r);
  return hipGetLastError();
}

// Rotate the query heads and write the rotated keys and the values of every row
// into the cache slot of its position.  qkv row layout: H query heads, then G
// key heads, then G value heads, each hd wide.  The row's values come either
// from bf16 qkv (rotated query heads are written back in place) or, with PART,
// from fp32 K-split partials [S][M][(H+2G)hd] summed in split order (the query
// heads are then written to qkv, rounded to bf16 once, after the rotation).
// K cache [B][G][cap][hd]; V cache [B][G][cap/16][hd][16] (blocks of 16
// positions, position fastest).
//
// One workgroup = 16 consecutive rows x one head.  Query and key heads: a thread
// takes four rotation pairs of one row.  Value heads: a thread takes 8 dims of
// one row, consecutive threads consecutive rows, so the 16 rows' values of one
// dim (consecutive positions of a batch row) are one contiguous run of the
// blocked V cache instead of 16 scattered 2-byte stores.
constexpr int RK_ROWS = 16;

template <bool PART>
__global__ void __launch_bounds__(256) k_rope_kv(bf16_t* __restrict__ qkv, const float* __restrict__ part, int S,
                                                 int M, int Lq, int H, int G, int hd,
                                                 const float2* __restrict__ tab, bf16_t* __restrict__ kc,
                                                 bf16_t* __restrict__ vc, const int* __restrict__ prefix,
                                                 int off, int cap) {
  const int h = blockIdx.y, t = threadIdx.x;
  const int half = hd / 2, quads = half / 4;
  const int nh = H + 2 * G;
  const size_t plane = static_cast<size_t>(M) * nh * hd;
  // four consecutive values of row m from column c
  auto load4 = [&](int m, int c, float* v) {
    if constexpr (PART) {
      const float4 acc = sum_planes(part + static_cast<size_t>(m) * nh * hd + c, plane, S);
      v[0] = acc.x; v[1] = acc.y; v[2] = acc.z; v[3] = acc.w;
    } else {
      const u32x2 u = *reinterpret_cast<const u32x2*>(qkv + static_cast<size_t>(m) * nh * hd + c);
      v[0] = __uint_as_float(u[0] << 16);
      v[1] = __uint_as_float(u[0] & 0xffff0000u);
      v[2] = __uint_as_float(u[1] << 16);
      v[3] = __uint_as_float(u[1] & 0xffff0000u);
    }
  };
  auto slot = [&](int m, int& b, int& pos) {
    b = m / Lq;
    pos = (prefix ? prefix[b] : 0) + off + m % Lq;
    return pos >= 0 && pos < cap;
  };
  if (h >= H + G) {  // value head: 8 dims of one row per thread, rows fastest
    const int r = t % RK_ROWS, c = t / RK_ROWS;
    const int m = blockIdx.x * RK_ROWS + r;
    if (m >= M || c >= hd / 8) return;
    int b, pos;
    if (!slot(m, b, pos)) return;
    float x[8];
    load4(m, h * hd + 8 * c, x);
    load4(m, h * hd + 8 * c + 4, x + 4);
    const int g = h - H - G;
    bf16_t* vb = vc + ((static_cast<size_t>(b) * G + g) * (cap / 16) + pos / 16) * hd * 16 + pos % 16;
#pragma unroll
    for (int u = 0; u < 8; ++u) vb[(8 * c + u) * 16] = f32_to_bf16(x[u]);
    return;
  }
  // query or key head: four rotation pairs of one row per thread
  const int r = t / quads, i0 = (t % quads) * 4;
  const int m = blockIdx.x * RK_ROWS + r;
  if (r >= RK_ROWS || m >= M) return;
  float x1[4], x2[4];
  load4(m, h * hd + i0, x1);
  load4(m, h * hd + i0 + half, x2);
  float y1[4], y2[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float2 cs = tab[static_cast<size_t>(m) * half + i0 + u];
    y1[u] = x1[u] * cs.x - x2[u] * cs.y;
    y2[u] = x2[u] * cs.x + x1[u] * cs.y;
  }
  const u32x2 olo = {pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
  const u32x2 ohi = {pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3])};
  if (h < H) {
    bf16_t* hp = qkv + static_cast<size_t>(m) * nh * hd + h * hd;
    *reinterpret_cast<u32x2*>(hp + i0) = olo;
    *reinterpret_cast<u32x2*>(hp + i0 + half) = ohi;
    return;
  }
  int b, pos;
  if (!slot(m, b, pos)) return;
  const int g = h - H;
  bf16_t* kp = kc + ((static_cast<size_t>(b) * G + g) * cap + pos) * hd;
  *reinterpret_cast<u32x2*>(kp + i0) = olo;
  *reinterpret_cast<u32x2*>(kp + i0 + half) = ohi;
}

hipError_t rope_kv(void* qkv, int M, int Lq, int H, int G, int hd, const float2* tab, void* kc, void* vc,
                   const int* prefix, int pos_offset, int cap, hipStream_t s, const float* part, int S) {
  if (M <= 0) return hipSuccess;
  if (part && (S < 1 || S > SPLIT_MAX)) return hipErrorInvalidValue;
  if (hd % 8 || RK_ROWS * (hd / 8) > 256) return hipErrorInvalidValue;
  const dim3 grid((M + RK_ROWS - 1) / RK_ROWS, H + 2 * G);
  if (part)
    hipLaunchKernelGGL(k_rope_kv<true>, grid, dim3(256), 0, s, static_cast<bf16_t*>(qkv), part, S, M, Lq, H, G,
                       hd, tab, static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), prefix, pos_offset, cap);
  else
    hipLaunchKernelGGL(k_rope_kv<false>, grid, dim3(256), 0, s, static_cast<bf16_t*>(qkv), nullptr, 1, M, Lq, H,
                       G, hd, tab, static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), prefix, pos_offset, cap);
  return hipGetLastError();
}

// ------------------------------------------------------ masked rows ----
// Masked-row compaction fused with the final RMSNorm: block m (one per canvas
// row) counts the masked rows before it; a masked row goes to slot `idx` of the
// compacted list (rows[idx] = m, xn[idx] = RMSNorm(x[m]) * g) and the last block
// writes the count.  Rows keep their canvas order.
__global__ void __launch_bounds__(256) k_masked_norm(const uint8_t* __restrict__ masked, int M,
                                                     const float* __restrict__ x, int d,
                                                     const bf16_t* __restrict__ g, float eps,
                                                     bf16_t* __restrict__ xn, int* __restrict__ rows,
                                                     int* __restrict__ count, const float* __restrict__ part,
                                                     int S) {
  __shared__ float red[4];
  // the row with the partials added (d <= 8192), read back for the normalisation
  __shared__ float4 sum_row[2048];
  const int m = blockIdx.x;
  float before = 0.f;
  for (int i = threadIdx.x; i < m; i += 256) before += masked[i] ? 1.f : 0.f;
  const int idx = static_cast<int>(block_sum_256(before, red));  // exact: at most M < 2^24
  const bool mine = masked[m] != 0;
  if (m == M - 1 && threadIdx.x == 0) count[0] = idx + (mine ? 1 : 0);
  if (!mine) return;
  if (threadIdx.x == 0) rows[idx] = m;
  const float* xr = x + static_cast<size_t>(m) * d;
  const float4* src = reinterpret_cast<const float4*>(xr);
  float ss = 0.f;
  if (S > 0) {
    const size_t plane = static_cast<size_t>(M) * d;
    const float* pr = part + static_cast<size_t>(m) * d;
    for (int c = threadIdx.x; c < d / 4; c += 256) {
      float4 v = src[c];
      const float4 a = sum_planes(pr + 4 * c, plane, S);
      v.x += a.x;
      v.y += a.y;
      v.z += a.z;
      v.w += a.w;
      sum_row[c] = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    src = sum_row;
  } else {
    for (int c = threadIdx.x; c < d / 4; c += 256) {
      const float4 v = src[c];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  // block_sum_256 synchronises the block: sum_row is complete after it (the
  // loop below reads quads that other threads wrote)
  const float rstd = rsqrtf(block_sum_256(ss, red) / d + eps);
  for (int c = threadIdx.x; c < d / 8; c += 256) {
    const float4 v0 = src[2 * c];
    const float4 v1 = src[2 * c + 1];
    float gg[8];
    unpack8(ld16(g + c * 8), gg);
    u32x4 o;
    o[0] = pack_bf16x2(v0.x * rstd * gg[0], v0.y * rstd * gg[1]);
    o[1] = pack_bf16x2(v0.z * rstd * gg[2], v0.w * rstd * gg[3]);
    o[2] = pack_bf16x2(v1.x * rstd * gg[4], v1.y * rstd * gg[5]);
    o[3] = pack_bf16x2(v1.z * rstd * gg[6], v1.w * rstd * gg[7]);
    st16(xn + static_cast<size_t>(idx) * d + c * 8, o);
  }
}

hipError_t masked_norm(const uint8_t* masked, int M, const float* x, int d, const void* gain, float eps, void* xn,
                       int* rows, int* count, hipStream_t s, const float* part, int S) {
  if (M <= 0) return hipSuccess;
  if (d > 8192 || S < 0 || S > SPLIT_MAX || (S > 0 && !part)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_masked_norm, dim3(M), dim3(256), 0, s, masked, M, x, d, static_cast<const bf16_t*>(gain), eps,
                     static_cast<bf16_t*>(xn), rows, count, part, S);
  return hipGetLastError();
}

// --------------------------------------------------------- head merge ----
// Per scored row: merge the per-vocab-tile (max, sum exp, argmax, sum exp*(l -
// max)) partials in a fixed order, then conf = 1 / sum_v exp(l_v - max), the
// argmax (lowest id on ties) and optionally the entropy ln(s) - t / s go to
// position rows[i] of the canvas.
//
// The partials are [tile][row] float4s, so one 128-byte line holds eight
// consecutive rows of a tile.  Workgroups go to the eight XCDs in turn; the
// grid is a multiple of 8 and workgroup b takes row (b % 8) * per + b / 8, so
// each XCD merges one contiguous run of rows and reads each line through its
// own L2 once (with rows in workgroup order every XCD fetched every line).
__device__ __forceinline__ MaxSumIdx msi_shfl_down(MaxSumIdx a, int w) {
  return MaxSumIdx{__shfl_down(a.m, w), __shfl_down(a.s, w), __shfl_down(a.idx, w), __shfl_down(a.t, w)};
}

__global__ void __launch_bounds__(256) k_head_merge(const float4* __restrict__ part, int n_tiles, int M,
                                                    int total_rows, const int* __restrict__ rows,
                                                    const int* __restrict__ m_dev, float* __restrict__ conf,
                                                    int* __restrict__ argmax, float* __restrict__ entropy) {
  __shared__ float sm[256], ss[256], st[256];
  __shared__ int si[256];
  const int per = gridDim.x / 8;
  const int i = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (i >= total_rows || (m_dev && i >= *m_dev)) return;  // uniform per workgroup
  MaxSumIdx acc{-INFINITY, 0.f, 0x7fffffff, 0.f};
  for (int t = threadIdx.x; t < n_tiles; t += 256) {
    const float4 p = part[static_cast<size_t>(t) * M + i];
    acc = msi_combine(acc, MaxSumIdx{p.x, p.y, __float_as_int(p.z), p.w});
  }
  // pairwise tree: thread t takes t + w for w = 128, 64 through LDS, then
  // w = 32 ... 1 within wavefront 0 by shuffles (the same pairs in the same
  // order)
  const int tid = threadIdx.x;
  sm[tid] = acc.m;
  ss[tid] = acc.s;
  st[tid] = acc.t;
  si[tid] = acc.idx;
  __syncthreads();
  if (tid < 128) {
    acc = msi_combine(acc, MaxSumIdx{sm[tid + 128], ss[tid + 128], si[tid + 128], st[tid + 128]});
    sm[tid] = acc.m;
    ss[tid] = acc.s;
    st[tid] = acc.t;
    si[tid] = acc.idx;
  }
  __syncthreads();
  if (tid >= 64) return;
  acc = msi_combine(acc, MaxSumIdx{sm[tid + 64], ss[tid + 64], si[tid + 64], st[tid + 64]});
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) {
    const MaxSumIdx o = msi_shfl_down(acc, w);
    acc = msi_combine(acc, o);  // lanes >= w hold values no lane reads later
  }
  if (tid == 0) {
    const int dst = rows ? rows[i] : i;
    conf[dst] = 1.0f / acc.s;
    argmax[dst] = acc.idx;
    if (entropy) entropy[dst] = logf(acc.s) - acc.t / acc.s;
  }
}

hipError_t head_merge(const void* partials, int n_tiles, int M, const int* rows, const int* m_dev,
                      float* conf, int* argmax, int total_rows, hipStream_t s, float* entropy) {
  if (total_rows <= 0) return hipSuccess;
  const int grid = (total_rows + 7) / 8 * 8;
  hipLaunchKernelGGL(k_head_merge, dim3(grid), dim3(256), 0, s, static_cast<const float4*>(partials), n_tiles, M,
                     total_rows, rows, m_dev, conf, argmax, entropy);
  return hipGetLastError();
}

// --------------------------------------------------------------- fills ----
__global__ void k_fill_i32(int* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void k_fill_f32(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void k_set_prefix(int* prefix, int B, int add, int value) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) prefix[b] = (add ? prefix[b] : 0) + value;
}

hipError_t fill_i32(int* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}
hipError_t fill_f32(float* p, int n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}
hipError_t set_prefix(int* prefix, int B, int add, int value, hipStream_t s) {
  hipLaunchKernelGGL(k_set_prefix, dim3((B + 255) / 256), dim3(256), 0, s, prefix, B, add, value);
  return hipGetLastError();
}
__global__ void k_strided_rows(int* rows, int n, int start, int stride) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) rows[i] = i * stride + start;
}
hipError_t strided_rows(int* rows, int n, int start, int stride, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_strided_rows, dim3((n + 255) / 256), dim3(256), 0, s, rows, n, start, stride);
  return hipGetLastError();
}

}  // namespace dlm
