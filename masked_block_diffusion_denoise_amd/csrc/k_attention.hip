// Block attention for the denoising step and for causal passes (prefill, the
// post-block append), with grouped-query heads and split-KV partials.
//
// A canvas block reads every cached prefix key and every key of its own block,
// bidirectionally; the prefix never reads the block (Modern LLMs, Module 12,
// sec. 14; MLX-VLM Nemotron Labs Diffusion guide, sec. 6).  Because the block's
// own keys/values are written to the cache slots right after the prefix before
// this kernel runs, the denoise pass is plain unmasked attention over keys
// [0, P_b + L) and the causal pass masks keys after the query's position.
//
// One workgroup = one (row b, KV head g, block of 32 queries, key split); its
// wavefronts are the query heads of the group.  Per 32-key tile:
//   S^T[key][query] = K_tile * Q^T      (v_mfma_f32_32x32x16_bf16, Q in registers)
//   online softmax per query (each lane owns one query column)
//   O^T[d][query] += V_tile^T * P^T     (P reused from the S registers as bf16)
// K rows are staged in LDS in a permuted order (bits 2 and 3 of the key index
// swapped) so that the S accumulator registers of a lane line up with eight
// consecutive keys -- the layout of the V cache, which stores blocks of 16 keys
// with the key index fastest ([cap/16][hd][16]).  So the V operand is one
// 16-byte LDS read per MFMA and no transpose is needed anywhere.
#include <algorithm>

#include "dlm_device.h"
#include "dlm_internal.h"

namespace dlm {

constexpr int KT = 32;          // keys per tile
constexpr int MIN_CHUNK = 128;  // minimum keys per split

// K rows in LDS: 16-byte chunks XOR-swizzled by the row so that the 32 rows read
// by one MFMA operand load spread over the banks.
__device__ __forceinline__ int kswz(int row, int chunk, int chunks) {
  const int mask = chunks >= 8 ? 7 : chunks - 1;
  return row * chunks * 8 + ((chunk ^ (row & mask)) << 3);
}

template <int HD, int GS>
__global__ void __launch_bounds__(GS * 64) k_attn(AttnArgs a, int chunk_len) {
  constexpr int KCH = HD / 8;  // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) bf16_t ks[KT * HD];
  __shared__ __attribute__((aligned(16))) bf16_t vs[KT * HD];  // [2][HD][16]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int split = blockIdx.x, qb = blockIdx.y;
  const int b = blockIdx.z / a.G, g = blockIdx.z % a.G;
  const int h = g * GS + w;
  const int p0 = (a.prefix ? a.prefix[b] : 0) + a.pos_offset;
  const int kv_len = min(p0 + a.Lq, a.cap);  // never read past the cache
  const int jq = qb * 32 + (lane & 31);  // this lane's query (block-relative)
  const int half = lane >> 5;

  int kbeg = split * chunk_len;
  int kend = min(kv_len, kbeg + chunk_len);
  if (a.causal) kend = min(kend, p0 + min(qb * 32 + 32, a.Lq));

  const int splits = gridDim.x;
  const size_t mrow = static_cast<size_t>(b) * a.Lq + jq;  // output row

  // queries, this lane's column: d = s*16 + 8*half .. +8
  bf16x8 qf[HD / 16];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + mrow * a.ldq + h * HD + 8 * half;
#pragma unroll
    for (int s = 0; s < HD / 16; ++s)
      qf[s] = as_bf16x8(jq < a.Lq ? ld16(qp + s * 16) : u32x4{0, 0, 0, 0});
  }

  f32x16 o[HD / 32];
#pragma unroll
  for (int c = 0; c < HD / 32; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[c][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = 1.4426950408889634f / sqrtf(static_cast<float>(HD));  // log2(e)/sqrt(hd)
  const int qpos = p0 + jq;

  const bf16_t* kc = static_cast<const bf16_t*>(a.kc) + (static_cast<size_t>(b) * a.G + g) * a.cap * HD;
  const bf16_t* vc = static_cast<const bf16_t*>(a.vc) + (static_cast<size_t>(b) * a.G + g) * a.cap * HD;

  // staging: K tile = KT*KCH chunks, V tile = 2*HD*2 chunks (16 B each)
  constexpr int NKC = KT * KCH, NVC = 2 * HD * 2;
  constexpr int PER = (NKC + NVC + GS * 64 - 1) / (GS * 64);
  u32x4 st[PER];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * GS * 64;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (e < NKC) {
        const int row = e / KCH, ch = e % KCH;
        const int key = k0 + row;
        if (key < kend) v = ld16(kc + static_cast<size_t>(key) * HD + ch * 8);
      } else if (e < NKC + NVC) {
        const int f = e - NKC;  // [blk][d][half]
        const int blk = f / (HD * 2), d = (f / 2) % HD, hh = f & 1;
        const int key0 = k0 + blk * 16 + hh * 8;
        if (key0 < kend) {
          v = ld16(vc + (static_cast<size_t>(k0 / 16 + blk) * HD + d) * 16 + hh * 8);
          const int valid = kend - key0;  // zero keys past the end (stale slots)
          if (valid < 8) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              uint32_t x = v[u];
              if (2 * u >= valid) x &= 0xffff0000u;
              if (2 * u + 1 >= valid) x &= 0x0000ffffu;
              v[u] = x;
            }
          }
        }
      }
      st[i] = v;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * GS * 64;
      if (e < NKC) {
        const int row = e / KCH, ch = e % KCH;
        st16(&ks[kswz(row, ch, KCH)], st[i]);
      } else if (e < NKC + NVC) {
        st16(&vs[(e - NKC) * 8], st[i]);
      }
    }
  };

  // physical key row read by this lane in the S product (bits 2 and 3 swapped)
  const int ar = lane & 31;
  const int krow = (ar & ~12) | ((ar & 4) << 1) | ((ar & 8) >> 1);

  if (kbeg < kend) {
    gload(kbeg);
    lstore();
    __syncthreads();
    for (int k0 = kbeg; k0 < kend; k0 += KT) {
      const bool more = k0 + KT < kend;
      if (more) gload(k0 + KT);

      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        const bf16x8 kf = as_bf16x8(ld16(&ks[kswz(krow, 2 * s + half, KCH)]));
        sacc = mfma32x32x16(kf, qf[s], sacc);
      }
      // register r holds key k0 + 16*(r/8) + 8*half + (r%8)
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 16 * (r >> 3) + 8 * half + (r & 7);
        float sv = sacc[r] * scale;
        if (key >= kend || (a.causal && key > qpos)) sv = -INFINITY;
        sacc[r] = sv;
        mloc = fmaxf(mloc, sv);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, WAVE));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[r] - m_use);
        sacc[r] = p;
        lsum += p;
      }
      lsum += __shfl_xor(lsum, 32, WAVE);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < HD / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
      bf16x8 pb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(sacc[8 * c + 2 * e], sacc[8 * c + 2 * e + 1]);
        pb[c] = as_bf16x8(u);
      }
#pragma unroll
      for (int dc = 0; dc < HD / 32; ++dc)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 vf = as_bf16x8(ld16(&vs[((c * HD) + dc * 32 + ar) * 16 + 8 * half]));
          o[dc] = mfma32x32x16(vf, pb[c], o[dc]);
        }
      __syncthreads();
      if (more) {
        lstore();
        __syncthreads();
      }
    }
  }

  // lane holds O^T[d][query]: d = dc*32 + 8*(r/4) + 4*half + r%4
  if (jq >= a.Lq) return;
  if (splits == 1) {
    const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
    bf16_t* op = static_cast<bf16_t*>(a.o) + mrow * (a.H * HD) + h * HD + 4 * half;
#pragma unroll
    for (int dc = 0; dc < HD / 32; ++dc)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2*>(op + dc * 32 + 8 * q) =
            u32x2{pack_bf16x2(o[dc][4 * q] * inv, o[dc][4 * q + 1] * inv),
                  pack_bf16x2(o[dc][4 * q + 2] * inv, o[dc][4 * q + 3] * inv)};
  } else {
    const size_t rows = static_cast<size_t>(a.B) * a.Lq;
    const size_t base = (static_cast<size_t>(split) * rows + mrow) * a.H + h;
    float* po = a.part_o + base * HD + 4 * half;
#pragma unroll
    for (int dc = 0; dc < HD / 32; ++dc)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(po + dc * 32 + 8 * q) =
            make_float4(o[dc][4 * q], o[dc][4 * q + 1], o[dc][4 * q + 2], o[dc][4 * q + 3]);
    if (half == 0) *reinterpret_cast<float2*>(a.part_ml + base * 2) = make_float2(m_run, l_run);
  }
}

// Merge split partials: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int HD>
__global__ void __launch_bounds__(256) k_attn_merge(AttnArgs a, int splits) {
  constexpr int PER_BLK = 256 / HD;
  const int rows = a.B * a.Lq;
  const int pair = blockIdx.x * PER_BLK + threadIdx.x / HD;  // (row, head)
  const int d = threadIdx.x % HD;
  if (pair >= rows * a.H) return;
  const int mrow = pair / a.H, h = pair % a.H;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s)
    mx = fmaxf(mx, a.part_ml[((static_cast<size_t>(s) * rows + mrow) * a.H + h) * 2]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float l = 0.f, acc = 0.f;
  for (int s = 0; s < splits; ++s) {
    const size_t base = (static_cast<size_t>(s) * rows + mrow) * a.H + h;
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + base * 2);
    const float wgt = (ml.y > 0.f) ? exp2f(ml.x - mu) : 0.f;
    l += wgt * ml.y;
    if (wgt != 0.f) acc += wgt * a.part_o[base * HD + d];
  }
  static_cast<bf16_t*>(a.o)[static_cast<size_t>(mrow) * a.H * HD + h * HD + d] =
      f32_to_bf16(l > 0.f ? acc / l : 0.f);
}

int attn_splits(const AttnArgs& a, int* chunk_out) {
  const int qblocks = (a.Lq + 31) / 32;
  const long base = static_cast<long>(qblocks) * a.B * a.G;
  int splits = static_cast<int>((512 + base - 1) / base);
  const int max_splits = (a.max_kv + MIN_CHUNK - 1) / MIN_CHUNK;
  splits = std::max(1, std::min(splits, max_splits));
  int chunk = (a.max_kv + splits - 1) / splits;
  chunk = (chunk + KT - 1) / KT * KT;
  splits = (a.max_kv + chunk - 1) / chunk;
  if (chunk_out) *chunk_out = chunk;
  return splits;
}

size_t attn_partial_floats(int splits, int rows, int H, int hd) {
  if (splits <= 1) return 0;
  return static_cast<size_t>(splits) * rows * H * (hd + 2);
}

template <int HD, int GS>
static hipError_t launch(const AttnArgs& a, hipStream_t s) {
  int chunk = 0;
  const int splits = attn_splits(a, &chunk);
  dim3 grid(splits, (a.Lq + 31) / 32, a.B * a.G);
  hipLaunchKernelGGL((k_attn<HD, GS>), grid, dim3(GS * 64), 0, s, a, chunk);
  if (splits > 1) {
    const int pairs = a.B * a.Lq * a.H;
    const int per = 256 / HD;
    hipLaunchKernelGGL((k_attn_merge<HD>), dim3((pairs + per - 1) / per), dim3(256), 0, s, a, splits);
  }
  return hipGetLastError();
}

hipError_t attention(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.Lq <= 0) return hipSuccess;
  const int gs = a.H / a.G;
  if (a.hd == 128 && gs == 4) return launch<128, 4>(a, s);
  if (a.hd == 128 && gs == 1) return launch<128, 1>(a, s);
  if (a.hd == 128 && gs == 2) return launch<128, 2>(a, s);
  if (a.hd == 32 && gs == 2) return launch<32, 2>(a, s);
  if (a.hd == 32 && gs == 4) return launch<32, 4>(a, s);
  if (a.hd == 32 && gs == 1) return launch<32, 1>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dlm
