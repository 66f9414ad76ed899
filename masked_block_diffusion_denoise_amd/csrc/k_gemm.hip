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
// (v_mfma_f32_16x16x32_bf16); the activation chunk is staged in LDS and shared
// by the four wavefronts of a workgroup; K may be split across workgroups, the
// last workgroup of a column tile sums the partials in a fixed order and runs
// the epilogue.
//
// Tiled (M > 64): 128 x 128 output tile per 256-thread workgroup, 64-deep K
// stages double-buffered in LDS (XOR-swizzled 16-byte chunks), each wavefront a
// 64 x 64 sub-tile of v_mfma_f32_32x32x16_bf16.
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
constexpr int SK_ROWS = 64;   // weight rows (output columns) per workgroup
constexpr int SK_KC = 256;    // K chunk staged per iteration

template <int MT, int EPI>
__global__ void __launch_bounds__(256) k_gemm_skinny(GemmArgs g, int ks_len) {
  constexpr int MR = MT * 16;
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][MR * SK_KC];
  __shared__ float red[512 * MT];  // epilogue exchange (SwiGLU: 2*MT*256, head: 12*MR)

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int ks = blockIdx.y, KS = gridDim.y;
  const int n_w = tile * SK_ROWS + w * 16;  // first weight row of this wavefront
  const int M = g.m_dev ? min(g.M, *g.m_dev) : g.M;
  if (M <= 0) return;
  const int k_begin = ks * ks_len;
  const int kc = min(SK_KC, ks_len);
  const int n_chunks = ks_len / kc;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* W = static_cast<const bf16_t*>(g.w);

  const bf16_t* wrow = W + static_cast<size_t>(n_w + (lane & 15)) * g.K + k_begin + 8 * (lane >> 4);
  const int steps = kc / 32;  // 32-deep MFMA steps per chunk (<= 8)

  u32x4 wcur[8], wnxt[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (s < steps) wcur[s] = ld16(wrow + s * 32);

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage activation chunk c into LDS buffer c & 1
  auto stage = [&](int c) {
    bf16_t* dst = xs[c & 1];
    const int cpr = kc / 8;  // 16-byte chunks per row
    for (int e = threadIdx.x; e < MR * cpr; e += 256) {
      const int r = e / cpr, ch = e % cpr;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (r < M) v = ld16(A + static_cast<size_t>(r) * g.lda + k_begin + c * kc + ch * 8);
      st16(dst + r * kc + ch * 8, v);
    }
  };

  stage(0);
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    if (c + 1 < n_chunks) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s < steps) wnxt[s] = ld16(wrow + (c + 1) * kc + s * 32);
      stage(c + 1);
    }
    const bf16_t* xb = xs[c & 1];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < steps) {
        const bf16x8 a = as_bf16x8(wcur[s]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const bf16x8 b = as_bf16x8(ld16(xb + (t * 16 + (lane & 15)) * kc + s * 32 + 8 * (lane >> 4)));
          acc[t] = mfma16x16x32(a, b, acc[t]);
        }
      }
    }
    __syncthreads();
    if (c + 1 < n_chunks) {
#pragma unroll
      for (int s = 0; s < 8; ++s) wcur[s] = wnxt[s];
    }
  }

  // lane holds D[n][m] for n = n_w + 4*(lane>>4) + r, m = t*16 + (lane & 15)
  const int nq = n_w + 4 * (lane >> 4);
  if (KS > 1) {
    float* ws = g.splitk_ws + static_cast<size_t>(ks) * g.M * g.N;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      if (m < M) *reinterpret_cast<float4*>(ws + static_cast<size_t>(m) * g.N + nq) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    }
    __threadfence();
    __syncthreads();
    __shared__ int last;
    if (threadIdx.x == 0) last = (atomicAdd(g.splitk_cnt + tile, 1) == KS - 1);
    __syncthreads();
    if (!last) return;
    __threadfence();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < M) {
        for (int k2 = 0; k2 < KS; ++k2) {
          const float4 p = *reinterpret_cast<const float4*>(
              g.splitk_ws + (static_cast<size_t>(k2) * g.M + m) * g.N + nq);
          s4.x += p.x;
          s4.y += p.y;
          s4.z += p.z;
          s4.w += p.w;
        }
      }
      acc[t] = f32x4{s4.x, s4.y, s4.z, s4.w};
    }
    if (threadIdx.x == 0) g.splitk_cnt[tile] = 0;
  }

  if (EPI == EPI_STORE_BF16 || EPI == EPI_RESID_F32) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      float v[4] = {acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
      if (m < M) store_quad<EPI>(g, m, nq, v);
    }
  } else if (EPI == EPI_SWIGLU) {
    // wavefronts 0,2 hold gate rows, 1,3 the matching up rows (16-row interleave)
    if (w & 1) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((w >> 1) * MT + t) * 256 + r * 64 + lane] = acc[t][r];
    }
    __syncthreads();
    if (!(w & 1)) {
      const int col = (tile * SK_ROWS + w * 16) / 2 + 4 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + (lane & 15);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu_f(acc[t][r]) * red[((w >> 1) * MT + t) * 256 + r * 64 + lane];
        if (m < M) {
          bf16_t* o = static_cast<bf16_t*>(g.out) + static_cast<size_t>(m) * g.ldc + col;
          *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
  } else if (EPI == EPI_HEAD) {
    bool bad = false;
    MaxSumIdx part[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      float v[4] = {acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
      if (g.logits && m < M) {
        float* lo = g.logits + static_cast<size_t>(g.logit_rows ? g.logit_rows[m] : m) * g.N + nq;
        float4 o4 = make_float4(v[0], v[1], v[2], v[3]);
        if (nq <= g.mask_id && g.mask_id < nq + 4) (&o4.x)[g.mask_id - nq] = -INFINITY;
        *reinterpret_cast<float4*>(lo) = o4;
      }
      MaxSumIdx p = head_quad(v, nq, g.mask_id, bad);
      p = msi_shfl_xor(p, 16);
      p = msi_shfl_xor(p, 32);
      part[t] = p;
    }
    if (__ballot(bad && true) && lane == 0 && g.nonfinite) atomicAdd(g.nonfinite, 1);
    float* rm = red;
    float* rs = red + 4 * MR;
    int* ri = reinterpret_cast<int*>(red + 8 * MR);
    if (lane < 16) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        rm[w * MR + t * 16 + lane] = part[t].m;
        rs[w * MR + t * 16 + lane] = part[t].s;
        ri[w * MR + t * 16 + lane] = part[t].idx;
      }
    }
    __syncthreads();
    if (threadIdx.x < MR) {
      const int m = threadIdx.x;
      MaxSumIdx p{rm[m], rs[m], ri[m]};
      for (int ww = 1; ww < 4; ++ww) p = msi_combine(p, MaxSumIdx{rm[ww * MR + m], rs[ww * MR + m], ri[ww * MR + m]});
      if (m < M)
        reinterpret_cast<float4*>(g.partials)[static_cast<size_t>(tile) * g.M + m] =
            make_float4(p.m, p.s, __int_as_float(p.idx), 0.f);
    }
  }
}

// ======================================================== tiled GEMM ====
constexpr int TL_BN = 128, TL_BM = 128, TL_BK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * TL_BK + ((chunk ^ (row & 7)) << 3); }

template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_tiled(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t ws_[2][TL_BN * TL_BK];
  __shared__ __attribute__((aligned(16))) bf16_t xs_[2][TL_BM * TL_BK];
  __shared__ float red[2 * TL_BM * 3];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wn = w >> 1, wm = w & 1;  // 2 x 2 wavefronts, each 64 (n) x 64 (m)
  const int n0 = blockIdx.x * TL_BN, m0 = blockIdx.y * TL_BM;
  const int M = g.m_dev ? min(g.M, *g.m_dev) : g.M;
  if (m0 >= M) return;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* W = static_cast<const bf16_t*>(g.w);

  // global -> register staging: thread covers rows t/8 + 32 i, 16-byte chunk t % 8
  const int lr = threadIdx.x >> 3, lc = threadIdx.x & 7;
  u32x4 wr[4], xr[4];
  auto gload = [&](int kt) {
    const int k = kt * TL_BK + lc * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wr[i] = ld16(W + static_cast<size_t>(n0 + lr + 32 * i) * g.K + k);
      const int m = m0 + lr + 32 * i;
      xr[i] = (m < M) ? ld16(A + static_cast<size_t>(m) * g.lda + k) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&ws_[buf][swz(lr + 32 * i, lc)], wr[i]);
      st16(&xs_[buf][swz(lr + 32 * i, lc)], xr[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = g.K / TL_BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int arow = lane & 31, ahalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < TL_BK / 16; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rn = wn * 64 + i * 32 + arow;
        a[i] = as_bf16x8(ld16(&ws_[buf][swz(rn, 2 * s + ahalf)]));
        const int rm = wm * 64 + i * 32 + arow;
        b[i] = as_bf16x8(ld16(&xs_[buf][swz(rm, 2 * s + ahalf)]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // lane holds D[n][m]: m = m0 + wm*64 + j*32 + (lane&31),
  // n = n0 + wn*64 + i*32 + 8*(r/4) + 4*(lane>>5) + r%4
  if (EPI == EPI_STORE_BF16 || EPI == EPI_RESID_F32) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * 64 + j * 32 + arow;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * 64 + i * 32 + 8 * q + 4 * ahalf;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          store_quad<EPI>(g, m, n, v);
        }
      }
  } else if (EPI == EPI_SWIGLU) {
    // within a 32-row MFMA tile, rows 0..15 are gate rows and 16..31 the matching
    // up rows: register r (r < 8) pairs with register r + 8
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * 64 + j * 32 + arow;
        if (m >= M) continue;
        const int col0 = (n0 + wn * 64 + i * 32) / 2;
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
    bool bad = false;
    MaxSumIdx part[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * 64 + j * 32 + arow;
      MaxSumIdx p{-INFINITY, 0.f, 0x7fffffff};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * 64 + i * 32 + 8 * q + 4 * ahalf;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (g.logits && m < M) {
            float4 o4 = make_float4(v[0], v[1], v[2], v[3]);
            if (n <= g.mask_id && g.mask_id < n + 4) (&o4.x)[g.mask_id - n] = -INFINITY;
            *reinterpret_cast<float4*>(g.logits + static_cast<size_t>(g.logit_rows ? g.logit_rows[m] : m) * g.N + n) = o4;
          }
          p = msi_combine(p, head_quad(v, n, g.mask_id, bad));
        }
      part[j] = msi_shfl_xor(p, 32);
    }
    if (__ballot(bad && true) && lane == 0 && g.nonfinite) atomicAdd(g.nonfinite, 1);
    float* rm = red;
    float* rs = red + 2 * TL_BM;
    int* ri = reinterpret_cast<int*>(red + 4 * TL_BM);
    if (lane < 32) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ml = wm * 64 + j * 32 + lane;
        rm[wn * TL_BM + ml] = part[j].m;
        rs[wn * TL_BM + ml] = part[j].s;
        ri[wn * TL_BM + ml] = part[j].idx;
      }
    }
    __syncthreads();
    if (threadIdx.x < TL_BM) {
      const int ml = threadIdx.x, m = m0 + ml;
      MaxSumIdx p = msi_combine(MaxSumIdx{rm[ml], rs[ml], ri[ml]},
                                MaxSumIdx{rm[TL_BM + ml], rs[TL_BM + ml], ri[TL_BM + ml]});
      if (m < M)
        reinterpret_cast<float4*>(g.partials)[static_cast<size_t>(blockIdx.x) * g.M + m] =
            make_float4(p.m, p.s, __int_as_float(p.idx), 0.f);
    }
  }
}

// ============================================================== host ====
static int skinny_ks(int M, int N, int K, int epi) {
  if (epi == EPI_HEAD) return 1;
  const int tiles = N / SK_ROWS;
  int ks = 1;
  while (tiles * ks < 512 && ks < 16) {
    const int nk = ks * 2;
    if (K % nk != 0) break;
    const int len = K / nk;
    if (len < SK_KC || len % SK_KC != 0) break;
    ks = nk;
  }
  (void)M;
  return ks;
}

size_t gemm_splitk_ws_floats(int M, int N, int K) {
  if (M > 64) return 0;
  size_t best = 0;
  for (int e = 0; e < 3; ++e) {
    const int ks = skinny_ks(M, N, K, e);
    if (ks > 1) best = std::max(best, static_cast<size_t>(ks) * M * N);
  }
  return best;
}

int gemm_head_tile_n(int M) { return M <= 64 ? SK_ROWS : TL_BN; }

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 64) {
    const int ks = skinny_ks(g.M, g.N, g.K, EPI);
    const int len = g.K / ks;
    dim3 grid(g.N / SK_ROWS, ks);
    if (g.M <= 16)
      hipLaunchKernelGGL((k_gemm_skinny<1, EPI>), grid, dim3(256), 0, s, g, len);
    else if (g.M <= 32)
      hipLaunchKernelGGL((k_gemm_skinny<2, EPI>), grid, dim3(256), 0, s, g, len);
    else
      hipLaunchKernelGGL((k_gemm_skinny<4, EPI>), grid, dim3(256), 0, s, g, len);
  } else {
    dim3 grid(g.N / TL_BN, (g.M + TL_BM - 1) / TL_BM);
    hipLaunchKernelGGL((k_gemm_tiled<EPI>), grid, dim3(256), 0, s, g);
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
