// bf16 MFMA GEMMs of the denoising path, C = A[M][K] * W[N][K]^T with fp32
// accumulation, and their fused epilogues (bf16 store, residual add, SwiGLU,
// LM-head confidence partials).
//
// The products are computed transposed, D[n][m] = W * A^T, so that each lane of
// an MFMA result holds consecutive output columns of one row and stores them as
// one vector.
//
// Skinny tiling (M <= 64, one denoise canvas at batch 1-2): the weight matrix is
// read exactly once, streamed from HBM straight into MFMA operand registers
// (v_mfma_f32_16x16x32_bf16), K split over the wavefronts of a workgroup and
// summed through LDS -- no cross-workgroup reduction (whose release fence would
// write back the L2 of an XCD).
//
// Tiled (M > 64): 256 x 256 (LM head, eight wavefronts) or 128 x 128 (four)
// output tiles, 64-deep K stages double-buffered in LDS, each wavefront a block
// of v_mfma_f32_32x32x16_bf16 tiles.
#include <algorithm>

#include "dlm_device.h"
#include "dlm_internal.h"

namespace dlm {

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Reduce four logits of columns n0..n0+3 (one row) to a (max, sum exp, argmax) partial.
__device__ __forceinline__ MaxSumIdx head_quad(const float* v, int n0, int mask_id, bool& bad) {
  float x[4];
  MaxSumIdx r{-INFINITY, 0.f, 0x7fffffff};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    x[u] = v[u];
    if (n0 + u == mask_id) x[u] = -INFINITY;
    else if (!__builtin_isfinite(x[u])) bad = true;
    if (x[u] > r.m) {
      r.m = x[u];
      r.idx = n0 + u;
    }
  }
  if (r.m != -INFINITY) {
#pragma unroll
    for (int u = 0; u < 4; ++u) r.s += __expf(x[u] - r.m);
  }
  return r;
}

__device__ __forceinline__ MaxSumIdx msi_shfl_xor(MaxSumIdx a, int mask) {
  MaxSumIdx b;
  b.m = __shfl_xor(a.m, mask, WAVE);
  b.s = __shfl_xor(a.s, mask, WAVE);
  b.idx = __shfl_xor(a.idx, mask, WAVE);
  return msi_combine(a, b);
}

// Store four consecutive outputs (row m, columns n..n+3) according to the epilogue.
template <int EPI>
__device__ __forceinline__ void store_quad(const GemmArgs& g, int m, int n, const float* v) {
  if (EPI == EPI_STORE_BF16) {
    bf16_t* o = static_cast<bf16_t*>(g.out) + static_cast<size_t>(m) * g.ldc + n;
    *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else if (EPI == EPI_RESID_F32) {
    float* o = static_cast<float*>(g.out) + static_cast<size_t>(m) * g.ldc + n;
    float4 x = *reinterpret_cast<float4*>(o);
    x.x += v[0];
    x.y += v[1];
    x.z += v[2];
    x.w += v[3];
    *reinterpret_cast<float4*>(o) = x;
  }
}

// ======================================================= skinny tiling ====
// WAVES wavefronts per workgroup: NG groups of 16 weight rows times KP = WAVES/NG
// parts of K.  Each wavefront streams its 16 weight rows over its K part from
// HBM straight into MFMA operand registers (v_mfma_f32_16x16x32_bf16, weights as
// the 16 x 32 A operand, activations as the B operand), two batches of four
// 32-deep steps in flight; the K parts are summed through LDS in a fixed order.
constexpr int SK_U = 4;  // 32-deep steps per load batch

template <int MT, int EPI, int NG, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) k_gemm_skinny(GemmArgs g) {
  constexpr int KP = WAVES / NG;
  __shared__ float red[WAVES * MT * 4 * 64];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = w % NG, kp = w / NG;
  const int tile = blockIdx.x;
  const int n_w = (tile * NG + rg) * 16;
  const int M = g.m_dev ? min(g.M, *g.m_dev) : g.M;
  if (M <= 0) return;
  const int nsteps = g.K / 32;
  const int s_begin = kp * nsteps / KP, s_end = (kp + 1) * nsteps / KP;
  const bf16_t* wp = static_cast<const bf16_t*>(g.w) + static_cast<size_t>(n_w + (lane & 15)) * g.K + 8 * (lane >> 4);
  const bf16_t* ap[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = min(t * 16 + (lane & 15), M - 1);  // rows past M repeat the last row; discarded
    ap[t] = static_cast<const bf16_t*>(g.a) + static_cast<size_t>(r) * g.lda + 8 * (lane >> 4);
  }

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operand registers of the two load batches.  They are zeroed up front: the
  // loads and MFMAs below are guarded by the same step bound, but without
  // explicit initial values the compiled pipeline was seen to consume
  // registers left by earlier kernels (history-dependent garbage in the first
  // 16-row tile) on wavefronts whose K part ends inside a batch.
  u32x4 wa[SK_U], wb[SK_U], xa[SK_U][MT], xb[SK_U][MT];
#pragma unroll
  for (int u = 0; u < SK_U; ++u) {
    wa[u] = wb[u] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < MT; ++t) xa[u][t] = xb[u][t] = u32x4{0, 0, 0, 0};
  }
  // Loads are unconditional (steps past the end reload the last step, which is
  // in bounds and never multiplied) so that the wait before each batch's MFMAs
  // only covers that batch and the next batch stays in flight.
#define SK_LOAD(WV, XV, S0)                                              \
  _Pragma("unroll") for (int u = 0; u < SK_U; ++u) {                     \
    const int st = min((S0) + u, s_last);                                \
    WV[u] = ld16(wp + st * 32);                                          \
    _Pragma("unroll") for (int t = 0; t < MT; ++t) XV[u][t] = ld16(ap[t] + st * 32); \
  }
#define SK_COMP(WV, XV, S0)                                              \
  _Pragma("unroll") for (int u = 0; u < SK_U; ++u) {                     \
    if ((S0) + u < s_end) {                                              \
      _Pragma("unroll") for (int t = 0; t < MT; ++t)                     \
        acc[t] = mfma16x16x32(as_bf16x8(WV[u]), as_bf16x8(XV[u][t]), acc[t]); \
    }                                                                    \
  }
  const int s_last = max(s_end - 1, 0);
  if (s_begin < s_end) SK_LOAD(wa, xa, s_begin);
  for (int s = s_begin; s < s_end; s += 2 * SK_U) {
    SK_LOAD(wb, xb, s + SK_U);
    SK_COMP(wa, xa, s);
    SK_LOAD(wa, xa, s + 2 * SK_U);
    SK_COMP(wb, xb, s + SK_U);
  }
#undef SK_LOAD
#undef SK_COMP

  // lane holds D[n][m] for n = n_w + 4*(lane>>4) + r, m = t*16 + (lane & 15)
  if (KP > 1 || EPI == EPI_SWIGLU || EPI == EPI_HEAD) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((w * MT + t) * 4 + r) * 64 + lane] = acc[t][r];
    __syncthreads();
  }
  auto summed = [&](int group, int t, int r) {
    float v = 0.f;
    for (int k = 0; k < KP; ++k) v += red[(((k * NG + group) * MT + t) * 4 + r) * 64 + lane];
    return v;
  };

  if (EPI == EPI_STORE_BF16 || EPI == EPI_RESID_F32) {
    if (w >= NG) return;
    const int nq = n_w + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (KP > 1) ? summed(rg, t, r) : acc[t][r];
      if (m < M) store_quad<EPI>(g, m, nq, v);
    }
  } else if (EPI == EPI_SWIGLU) {
    // NG == 2: group 0 holds the 16 gate rows, group 1 the matching up rows
    if (w != 0) return;
    const int col = tile * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = silu_f(summed(0, t, r)) * summed(1, t, r);
      if (m < M) {
        bf16_t* o = static_cast<bf16_t*>(g.out) + static_cast<size_t>(m) * g.ldc + col;
        *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  } else if (EPI == EPI_HEAD) {
    // every wavefront reduces its own 16 vocab rows (summing the K parts), then
    // wavefront 0 merges the NG groups of the tile
    __shared__ float hm[NG * MT * 16], hs[NG * MT * 16];
    __shared__ int hi[NG * MT * 16];
    bool bad = false;
    if (w < NG) {
      const int nq = n_w + 4 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + (lane & 15);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (KP > 1) ? summed(rg, t, r) : acc[t][r];
        if (g.logits && m < M) {
          float* lo = g.logits + static_cast<size_t>(g.logit_rows ? g.logit_rows[m] : m) * g.N + nq;
          float4 o4 = make_float4(v[0], v[1], v[2], v[3]);
          if (nq <= g.mask_id && g.mask_id < nq + 4) (&o4.x)[g.mask_id - nq] = -INFINITY;
          *reinterpret_cast<float4*>(lo) = o4;
        }
        MaxSumIdx p = head_quad(v, nq, g.mask_id, bad);
        p = msi_shfl_xor(p, 16);
        p = msi_shfl_xor(p, 32);
        if (lane < 16) {
          hm[(rg * MT + t) * 16 + lane] = p.m;
          hs[(rg * MT + t) * 16 + lane] = p.s;
          hi[(rg * MT + t) * 16 + lane] = p.idx;
        }
      }
      if (__ballot(bad) && lane == 0 && g.nonfinite) atomicAdd(g.nonfinite, 1);
    }
    __syncthreads();
    if (threadIdx.x < MT * 16) {
      const int mm = threadIdx.x;  // = t*16 + row
      MaxSumIdx p{hm[mm], hs[mm], hi[mm]};
      for (int q = 1; q < NG; ++q) p = msi_combine(p, MaxSumIdx{hm[q * MT * 16 + mm], hs[q * MT * 16 + mm], hi[q * MT * 16 + mm]});
      if (mm < M)
        reinterpret_cast<float4*>(g.partials)[static_cast<size_t>(tile) * g.M + mm] =
            make_float4(p.m, p.s, __int_as_float(p.idx), 0.f);
    }
  }
}

// ======================================================== tiled GEMM ====
// BN x BM output tile (weights x activations) per workgroup of WN x WM
// wavefronts, each a (BN/WN) x (BM/WM) block of 32 x 32 MFMA tiles; 64-deep K
// stages double-buffered in LDS through registers; 16-byte chunks XOR-swizzled
// by row so the 32 rows of an MFMA operand read spread over the LDS banks.
// Tiles are ordered per XCD: workgroup i runs on XCD i % 8, so XCD x takes a
// contiguous range of tiles, activation tiles fastest, and the workgroups that
// share a weight tile share that XCD's L2.
constexpr int TL_BK = 64;

// 128-byte rows of 8 chunks; the LDS serves 16 lanes (256 bytes) per cycle, so
// the XOR key changes every second row: the 16 rows read by one quarter of an
// MFMA operand load land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * TL_BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

template <int EPI, int BN, int BM, int WN, int WM>
__global__ void __launch_bounds__(WN * WM * 64) k_gemm_tiled(GemmArgs g) {
  constexpr int T = WN * WM * 64;
  constexpr int TN = BN / WN / 32, TM = BM / WM / 32;
  constexpr int CPT = (BN + BM) * 8 / T;  // 16-byte chunks per thread per stage
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BN + BM) * TL_BK];

  const int nN = g.N / BN, nM = (g.M + BM - 1) / BM;
  const int total = nN * nM, per = (total + 7) / 8;
  const int tid_ = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tid_ >= total) return;
  const int n0 = (tid_ / nM) * BN, m0 = (tid_ % nM) * BM;
  const int M = g.m_dev ? min(g.M, *g.m_dev) : g.M;
  if (m0 >= M) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wn = w % WN, wm = w / WN;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* W = static_cast<const bf16_t*>(g.w);

  const int lc = threadIdx.x & 7, lr = threadIdx.x >> 3;  // chunk column, first row
  const bf16_t* src[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int row = lr + i * (T / 8);
    if (row < BN) {
      src[i] = W + static_cast<size_t>(n0 + row) * g.K + lc * 8;
    } else {
      const int m = min(m0 + row - BN, M - 1);  // rows past M repeat the last row; discarded
      src[i] = A + static_cast<size_t>(m) * g.lda + lc * 8;
    }
  }
  // Register staging: the next stage is loaded from memory while the current
  // one is multiplied out of LDS, then stored to the other LDS buffer.
  u32x4 st[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) st[i] = u32x4{0, 0, 0, 0};
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) st[i] = ld16(src[i] + kt * TL_BK);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) st16(&lds[buf][swz(lr + i * (T / 8), lc)], st[i]);
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = g.K / TL_BK;
  const int arow = lane & 31, ahalf = lane >> 5;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < TL_BK / 16; ++s) {
      bf16x8 fa[TN], fb[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) fa[i] = as_bf16x8(ld16(&lds[buf][swz(wn * TN * 32 + i * 32 + arow, 2 * s + ahalf)]));
#pragma unroll
      for (int j = 0; j < TM; ++j)
        fb[j] = as_bf16x8(ld16(&lds[buf][swz(BN + wm * TM * 32 + j * 32 + arow, 2 * s + ahalf)]));
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // lane holds D[n][m]: m = m0 + (wm*TM + j)*32 + (lane&31),
  // n = n0 + (wn*TN + i)*32 + 8*(r/4) + 4*(lane>>5) + r%4
  if (EPI == EPI_STORE_BF16 || EPI == EPI_RESID_F32) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + (wm * TM + j) * 32 + arow;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + i) * 32 + 8 * q + 4 * ahalf;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          store_quad<EPI>(g, m, n, v);
        }
      }
  } else if (EPI == EPI_SWIGLU) {
    // within a 32-row MFMA tile, rows 0..15 are gate rows and 16..31 the matching
    // up rows: register r (r < 8) pairs with register r + 8
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + (wm * TM + j) * 32 + arow;
        if (m >= M) continue;
        const int col0 = (n0 + (wn * TN + i) * 32) / 2;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = silu_f(acc[i][j][4 * q + u]) * acc[i][j][4 * q + u + 8];
          bf16_t* o = static_cast<bf16_t*>(g.out) + static_cast<size_t>(m) * g.ldc + col0 + 8 * q + 4 * ahalf;
          *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
  } else if (EPI == EPI_HEAD) {
    __shared__ float rm[WN * BM], rs[WN * BM];
    __shared__ int ri[WN * BM];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int ml = (wm * TM + j) * 32 + arow, m = m0 + ml;
      MaxSumIdx p{-INFINITY, 0.f, 0x7fffffff};
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + i) * 32 + 8 * q + 4 * ahalf;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (g.logits && m < M) {
            float4 o4 = make_float4(v[0], v[1], v[2], v[3]);
            if (n <= g.mask_id && g.mask_id < n + 4) (&o4.x)[g.mask_id - n] = -INFINITY;
            *reinterpret_cast<float4*>(g.logits + static_cast<size_t>(g.logit_rows ? g.logit_rows[m] : m) * g.N + n) = o4;
          }
          p = msi_combine(p, head_quad(v, n, g.mask_id, bad));
        }
      p = msi_shfl_xor(p, 32);
      if (ahalf == 0) {
        rm[wn * BM + ml] = p.m;
        rs[wn * BM + ml] = p.s;
        ri[wn * BM + ml] = p.idx;
      }
    }
    if (__ballot(bad) && lane == 0 && g.nonfinite) atomicAdd(g.nonfinite, 1);
    __syncthreads();
    for (int ml = threadIdx.x; ml < BM; ml += T) {
      const int m = m0 + ml;
      MaxSumIdx p{rm[ml], rs[ml], ri[ml]};
#pragma unroll
      for (int q = 1; q < WN; ++q) p = msi_combine(p, MaxSumIdx{rm[q * BM + ml], rs[q * BM + ml], ri[q * BM + ml]});
      if (m < M)
        reinterpret_cast<float4*>(g.partials)[static_cast<size_t>(n0 / BN) * g.M + m] =
            make_float4(p.m, p.s, __int_as_float(p.idx), 0.f);
    }
  }
}

// ============================================================== host ====
// LM-head vocabulary columns per partial record: 64 (skinny) or 256 (tiled).
int gemm_head_tile_n(int M) { return M <= 64 ? 64 : 256; }

template <int EPI, int BN, int BM, int WN, int WM>
static void launch_tiled(const GemmArgs& g, hipStream_t s) {
  const int total = (g.N / BN) * ((g.M + BM - 1) / BM);
  const int per = (total + 7) / 8;
  hipLaunchKernelGGL((k_gemm_tiled<EPI, BN, BM, WN, WM>), dim3(8 * per), dim3(WN * WM * 64), 0, s, g);
}

template <int MT, int EPI>
static void launch_skinny(const GemmArgs& g, hipStream_t s) {
  if constexpr (EPI == EPI_HEAD) {
    hipLaunchKernelGGL((k_gemm_skinny<MT, EPI, 4, 4>), dim3(g.N / 64), dim3(256), 0, s, g);
  } else if constexpr (EPI == EPI_SWIGLU) {
    hipLaunchKernelGGL((k_gemm_skinny<MT, EPI, 2, 4>), dim3(g.N / 32), dim3(256), 0, s, g);
  } else if (g.N / 16 < 512) {
    hipLaunchKernelGGL((k_gemm_skinny<MT, EPI, 1, 8>), dim3(g.N / 16), dim3(512), 0, s, g);
  } else {
    hipLaunchKernelGGL((k_gemm_skinny<MT, EPI, 1, 4>), dim3(g.N / 16), dim3(256), 0, s, g);
  }
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 64) {
    if (g.M <= 16)
      launch_skinny<1, EPI>(g, s);
    else if (g.M <= 32)
      launch_skinny<2, EPI>(g, s);
    else
      launch_skinny<4, EPI>(g, s);
  } else {
    // 256 x 256 tiles where they still give at least one wave of workgroups
    // (the LM head, the SwiGLU gate/up projection); 128 x 128 otherwise
    if (EPI == EPI_HEAD || (g.N / 256) * ((g.M + 255) / 256) >= 256)
      launch_tiled<EPI, 256, 256, 4, 2>(g, s);
    else
      launch_tiled<EPI, 128, 128, 2, 2>(g, s);
  }
  return hipGetLastError();
}

hipError_t gemm(const GemmArgs& g, GemmEpilogue epi, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE_BF16: return launch_epi<EPI_STORE_BF16>(g, s);
    case EPI_RESID_F32: return launch_epi<EPI_RESID_F32>(g, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(g, s);
    case EPI_HEAD: return launch_epi<EPI_HEAD>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dlm
