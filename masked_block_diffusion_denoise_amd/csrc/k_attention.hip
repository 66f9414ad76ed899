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
// One workgroup = one (row b, KV head g, block of 32 queries, key range); its
// wavefronts are the query heads of the group, which share every K/V tile.
// Per 32-key tile:
//   S^T[key][query] = K_tile * Q^T      (v_mfma_f32_32x32x16_bf16, Q in registers)
//   online softmax per query (each lane owns one query column)
//   O^T[d][query] += V_tile^T * P^T     (P reused from the S registers as bf16)
// K rows are read in a permuted order (bits 2 and 3 of the key index swapped)
// so that the S accumulator registers of a lane line up with eight consecutive
// keys -- the layout of the V cache, which stores blocks of 16 keys with the key
// index fastest ([cap/16][hd][16]).  So the V operand is one 16-byte LDS read per
// MFMA and no transpose is needed anywhere.
//
// K/V tiles stream through a ring of LDS stages of two tiles each, filled by
// direct global-to-LDS loads (global_load_lds_dwordx4), one wait + barrier per
// stage: two stages (one in flight), or three (two in flight) for long key
// ranges with one workgroup per CU.  With SPR a stage's loads are issued one
// tile at a time between the batches of the S product rather than all at once
// after the barrier.  The two tiles
// of a stage are computed together (one softmax update over 64 keys), which
// gives each wavefront independent MFMA chains to overlap -- with one or two
// wavefronts per SIMD, a single tile's dependent chain (S product, softmax,
// P*V) left the matrix unit idle most of the time.  Fragments are read in
// inline asm that waits for its own reads (the compiler cannot tell the ring
// stages apart and would otherwise drain every load before each read).
#include <algorithm>

#include "dlm_device.h"
#include "dlm_internal.h"

namespace dlm {

constexpr int KT = 32;          // keys per tile
// Minimum keys per split (4 tiles).  Short prefixes at batch 1 are latency-
// bound: shorter splits shorten each workgroup's chain of dependent tiles (the
// 8B-class model over a ~1024-position prefix: 4.074 -> 4.023 ms per denoise
// step with 128 instead of 256; 64 measured the same as 128).
constexpr int MIN_CHUNK = 128;
// Launch shape: up to 512 workgroups (two per CU, each with its 64 KB ring), so
// that the other workgroup on a CU hides the latency of a stage's dependent
// chain (one workgroup per CU with a deeper ring measured up to 25% slower at
// batch 4 over a 65536-position prefix, and no faster at batch 1); key splits
// are only made for that second workgroup while they stay long (attn_splits).
constexpr int TARGET_WG = 512;
constexpr int SUB = 2;  // 32-key tiles per ring stage
constexpr float RESCALE = 8.f;  // lazy-rescale threshold (log2 units)

__device__ __forceinline__ uint32_t att_lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// NT: cache policy non-temporal (evicted first), for large K/V streams (the
// launch picks it above 64 MB per launch)
template <bool NT>
__device__ __forceinline__ void att_load_lds16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, NT ? 2 : 0);
}

template <int N>
__device__ __forceinline__ void att_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(N) : "memory");
}

// K rows in LDS: row r (key k0 + r) holds its 16-byte chunks XOR-swizzled.  The
// LDS serves 16 lanes x 16 bytes per cycle; the 16 rows one quarter of an
// operand read touches must land in 16 distinct 16-byte bank groups: with
// 256-byte rows (hd 128) the chunk is XOR-ed with the row's low 4 bits, with
// 64-byte rows (hd 32, four rows per 256 bytes) with row bits 2-3.
template <int HD>
__device__ __forceinline__ int kxor(int row) {
  return HD >= 128 ? (row & 15) : ((row >> 2) & 3);
}

// V rows ([blk][d] of 2 x 16 bytes): the two halves of row d are swapped when
// bit 3 of d is set, so the 16 consecutive d one read quarter touches cover all
// 16 bank groups.
__device__ __forceinline__ int vxor(int vrow) { return (vrow >> 3) & 1; }

// Fragment reads (each waits for its own reads before returning).
template <int N>
__device__ __forceinline__ void lds_read_n(const uint32_t (&addr)[N], u32x4 (&f)[N]);

template <>
__device__ __forceinline__ void lds_read_n<8>(const uint32_t (&a)[8], u32x4 (&f)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]), "=&v"(f[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_n<4>(const uint32_t (&a)[4], u32x4 (&f)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_n<1>(const uint32_t (&a)[1], u32x4 (&f)[1]) {
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(f[0]) : "v"(a[0]) : "memory");
}

template <>
__device__ __forceinline__ void lds_read_n<2>(const uint32_t (&a)[2], u32x4 (&f)[2]) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(f[0]), "=&v"(f[1])
               : "v"(a[0]), "v"(a[1])
               : "memory");
}

// Four products on two accumulators (c0 += a0 b0, c1 += a1 b0, c0 += a2 b1,
// c1 += a3 b1), with four fragment reads (n0..n3 <- [d0..d3]) issued first and
// waited for at the end, so that they land under the products.
__device__ __forceinline__ void att_quad(f32x16& c0, f32x16& c1, const u32x4& a0, const u32x4& a1, const u32x4& a2,
                                         const u32x4& a3, const u32x4& b0, const u32x4& b1, u32x4& n0, u32x4& n1,
                                         u32x4& n2, u32x4& n3, uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
  asm volatile(
      "ds_read_b128 %2, %12\n\t"
      "ds_read_b128 %3, %13\n\t"
      "ds_read_b128 %4, %14\n\t"
      "ds_read_b128 %5, %15\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %10, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %7, %10, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %8, %11, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %9, %11, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "+v"(c0), "+v"(c1), "=&v"(n0), "=&v"(n1), "=&v"(n2), "=&v"(n3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(d0), "v"(d1), "v"(d2), "v"(d3)
      : "memory");
}

template <int HD, int GS, bool NT, int NB, bool SPR>
__global__ void __launch_bounds__(GS * 64) k_attn(AttnArgs a, int chunk_len) {
  constexpr int KCH = HD / 8;              // 16-byte chunks per key row
  constexpr int TILE_K = KT * HD * 2;      // bytes of a K tile (= bytes of a V tile)
  constexpr int TILE = 2 * TILE_K;         // one 32-key tile: K, then V
  constexpr int STAGE = SUB * TILE;        // one ring stage: SUB tiles
  constexpr int TBLK = TILE / 1024 / GS;   // 1 KB load blocks per wavefront per tile
  static_assert((TILE / 1024) % GS == 0 && TBLK >= 1, "a tile must split evenly over the wavefronts");
  constexpr int NS = HD / 16;              // 16-deep steps of the S product
  constexpr int ND = HD / 32;              // 32-row blocks of the output
  static_assert(NB == 2 || NB == 3, "two or three ring stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NB * STAGE];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, qb = blockIdx.y;
  const int b = blockIdx.z / a.G, g = blockIdx.z % a.G;
  const int h = g * GS + w;
  // uniform over the workgroup (kept in scalar registers, so the per-stage
  // tests below are scalar branches)
  const int p0 = __builtin_amdgcn_readfirstlane((a.prefix ? a.prefix[b] : 0) + a.pos_offset);
  const int kv_len = min(p0 + a.Lq, a.cap);  // never read past the cache
  const int jq = qb * 32 + (lane & 31);      // this lane's query (block-relative)
  const int half = lane >> 5;

  const int kbeg = split * chunk_len;
  int kend = min(kv_len, kbeg + chunk_len);
  if (a.causal) kend = min(kend, p0 + min(qb * 32 + 32, a.Lq));
  const int ntiles = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;
  const int nst = (ntiles + SUB - 1) / SUB;  // ring stages

  const int splits = gridDim.x;
  const size_t mrow = static_cast<size_t>(b) * a.Lq + jq;  // output row

  // queries, this lane's column: d = s*16 + 8*half .. +8
  bf16x8 qf[NS];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + mrow * a.ldq + h * HD + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(jq < a.Lq ? ld16(qp + s * 16) : u32x4{0, 0, 0, 0});
  }

  f32x16 o[ND];
#pragma unroll
  for (int c = 0; c < ND; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[c][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = 1.4426950408889634f / sqrtf(static_cast<float>(HD));  // log2(e)/sqrt(hd)
  const int qpos = p0 + jq;

  const size_t head_off = (static_cast<size_t>(b) * a.G + g) * a.cap * HD;
  const bf16_t* kc = static_cast<const bf16_t*>(a.kc) + head_off;
  const bf16_t* vc = static_cast<const bf16_t*>(a.vc) + head_off;

  // Load block q of a tile, lane l -> 16-byte slot 64q + l of the tile.  K
  // blocks (q < TILE/2048): slot -> (row, physical chunk) -> logical chunk of
  // key k0 + row.  V blocks: the V tile is contiguous in the blocked cache
  // layout ([2][HD][16] keys from k0), slot -> (vrow, physical half) -> logical
  // half.  Both tile bases sit at element k0*HD of their cache.
  const bf16_t* src[TBLK];
#pragma unroll
  for (int i = 0; i < TBLK; ++i) {
    const int q = w * TBLK + i;
    if (q < TILE / 2048) {
      const int slot = q * 64 + lane;
      const int row = slot / KCH, pc = slot % KCH;
      src[i] = kc + row * HD + (pc ^ kxor<HD>(row)) * 8;
    } else {
      const int slot = (q - TILE / 2048) * 64 + lane;
      const int vrow = slot >> 1, ph = slot & 1;
      src[i] = vc + vrow * 16 + (ph ^ vxor(vrow)) * 8;
    }
  }
  // tile u of stage st: tile st*SUB + u of this workgroup's key range; a tile
  // past the range is not loaded (its keys are masked and its values zeroed)
  auto issue_tile = [&](int st, int u) {
    const int t = st * SUB + u;
    if (t < ntiles) {
      uint8_t* dst = lds + (st % NB) * STAGE + u * TILE + w * TBLK * 1024;
      const size_t off = static_cast<size_t>(kbeg + t * KT) * HD;
#pragma unroll
      for (int i = 0; i < TBLK; ++i) att_load_lds16<NT>(src[i] + off, dst + i * 1024);
    }
  };

  // fragment offsets within a tile
  const int ar = lane & 31;
  const int krow = (ar & ~12) | ((ar & 4) << 1) | ((ar & 8) >> 1);  // bits 2 and 3 swapped
  uint32_t koff[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) koff[s] = krow * HD * 2 + (((2 * s + half) ^ kxor<HD>(krow)) << 4);
  // V row d = dc*32 + ar of block c; the bank swizzle only depends on ar
  const uint32_t voff = TILE_K + ar * 32 + ((half ^ vxor(ar)) << 4);
  const uint32_t lbase = att_lds_addr(lds);

#pragma unroll
  for (int p = 0; p < NB - 1; ++p)
#pragma unroll
    for (int u = 0; u < SUB; ++u)
      if (p < nst) issue_tile(p, u);
  for (int st = 0; st < nst; ++st) {
    // stage st has landed once at most stage st + 1's loads (three stages) are
    // outstanding; the barrier also retires stage st - 1, whose buffer this
    // stage refills with stage st + NB - 1
    if (NB == 3 && st + 1 < nst) {
      if (ntiles - (st + 1) * SUB >= SUB)
        att_wait_barrier<SUB * TBLK>();
      else
        att_wait_barrier<TBLK>();
    } else {
      att_wait_barrier<0>();
    }
    const bool more = st + NB - 1 < nst;
    if (!SPR && more) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) issue_tile(st + NB - 1, u);
    }
    const int k0 = kbeg + st * SUB * KT;
    const uint32_t sb = lbase + (st % NB) * STAGE;
    // The stage that reaches past the range (the last one): cache slots past the
    // row's end may hold anything (also NaN), and a tile past the range was not
    // loaded, so their values are zeroed in LDS -- a zero probability alone
    // would still give 0 * NaN.  No load is in flight on the last stage.
    const bool tail = k0 + SUB * KT > kend;
    if (tail) {
      uint8_t* st_lds = lds + (st % NB) * STAGE;
      const int first = max(0, kend - k0);  // first stage key past the range
      for (int i = threadIdx.x; i < (SUB * KT - first) * HD; i += GS * 64) {
        const int kk = first + i / HD, d = i % HD;      // stage key, value dim
        const int u = kk / KT, c = (kk % KT) / 16, vrow = c * HD + d;
        const int ph = ((kk % 16) / 8) ^ vxor(vrow);  // physical 16-byte half
        *reinterpret_cast<uint16_t*>(st_lds + u * TILE + TILE_K + (vrow * 2 + ph) * 16 + (kk % 8) * 2) = 0;
      }
      __syncthreads();
    }

    f32x16 sacc[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[u][r] = 0.f;
    // hd 128: each batch of fragment reads is issued under the previous batch's
    // products (att_quad), and the first batch of V fragments under the second
    // half of the S product, so that the P*V products start from registers
    // right after the softmax.  Batch 32 over 4096 positions 114.9 -> 109.2 us,
    // batch 4 over 65536 196.7 -> 192.7 us (interleaved, outputs identical).
    constexpr bool PIPE = HD == 128 && SUB == 2;
    u32x4 vf0[8];  // first batch of V fragments (pipelined form)
    if constexpr (PIPE) {
      auto qv = [&](int s) { return __builtin_bit_cast(u32x4, qf[s]); };
      uint32_t ka[8];
      u32x4 kf0[8], kf1[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[u * 4 + s] = sb + u * TILE + koff[s];
      lds_read_n<8>(ka, kf0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[u * 4 + s] = sb + u * TILE + koff[4 + s];
      att_quad(sacc[0], sacc[1], kf0[0], kf0[4], kf0[1], kf0[5], qv(0), qv(1), kf1[0], kf1[1], kf1[2], kf1[3], ka[0], ka[1],
               ka[2], ka[3]);
      att_quad(sacc[0], sacc[1], kf0[2], kf0[6], kf0[3], kf0[7], qv(2), qv(3), kf1[4], kf1[5], kf1[6], kf1[7], ka[4], ka[5],
               ka[6], ka[7]);
      if (SPR && more) issue_tile(st + NB - 1, 0);
      uint32_t va[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dd = 0; dd < 2; ++dd)
#pragma unroll
          for (int c = 0; c < 2; ++c) va[(u * 2 + dd) * 2 + c] = sb + u * TILE + voff + c * (HD * 32) + dd * 1024;
      att_quad(sacc[0], sacc[1], kf1[0], kf1[4], kf1[1], kf1[5], qv(4), qv(5), vf0[0], vf0[1], vf0[2], vf0[3], va[0], va[1],
               va[2], va[3]);
      att_quad(sacc[0], sacc[1], kf1[2], kf1[6], kf1[3], kf1[7], qv(6), qv(7), vf0[4], vf0[5], vf0[6], vf0[7], va[4], va[5],
               va[6], va[7]);
      if (SPR && more) issue_tile(st + NB - 1, 1);
    } else {
      // S of the SUB tiles: one accumulation chain per tile, the chains
      // interleaved so that consecutive MFMAs are independent; fragment reads in
      // batches of KB steps per tile (register pressure)
      constexpr int KB = NS >= 8 ? NS / 2 : NS;
      static_assert(NS % KB == 0, "whole batches of K fragments");
#pragma unroll
      for (int hs = 0; hs < NS; hs += KB) {
        uint32_t ka[SUB * KB];
        u32x4 kf[SUB * KB];
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int s = 0; s < KB; ++s) ka[u * KB + s] = sb + u * TILE + koff[hs + s];
        lds_read_n<SUB * KB>(ka, kf);
#pragma unroll
        for (int s = 0; s < KB; ++s)
#pragma unroll
          for (int u = 0; u < SUB; ++u) sacc[u] = mfma32x32x16(as_bf16x8(kf[u * KB + s]), qf[hs + s], sacc[u]);
        // one tile of stage st + NB - 1 after each batch of the S product
        if (SPR && more && hs / KB < SUB) issue_tile(st + NB - 1, hs / KB);
      }
      if (SPR && more) {
#pragma unroll
        for (int u = NS / KB; u < SUB; ++u) issue_tile(st + NB - 1, u);
      }
    }
    // register r of tile u holds key k0 + u*KT + 16*(r/8) + 8*half + (r%8).
    // Only the last stage of the range and causal passes need a mask.
    // A key is masked when it is past the range or (causal) after the query:
    // key >= min(kend, qpos + 1), one compare against a per-lane limit.  The
    // empty asm keeps the masking behind its branch (if-converted, it would run
    // on every stage).
    if (tail || a.causal) {
      asm volatile("");
      const int lim = (a.causal ? min(kend, qpos + 1) : kend) - (k0 + 8 * half);
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (u * KT + 16 * (r >> 3) + (r & 7) >= lim) sacc[u][r] = -INFINITY;
    }
    // this lane's maximum over its half of the stage's keys (lanes l and l^32
    // hold the two halves of one query)
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[u][r]);
    mloc *= scale;
    // Lazy rescaling: the exponent reference m_run only moves when some query of
    // the wavefront sees a score more than 2^RESCALE above it (then all lanes
    // rescale together); otherwise p <= 2^RESCALE and the output accumulators
    // are not touched.  o / l is unchanged by the choice.  The two halves of a
    // query keep the same m_run: the test is over the whole wavefront, and the
    // new reference takes the maximum over both halves.
    if (__any(mloc > m_run + RESCALE)) {
      const float m_new = fmaxf(m_run, fmaxf(mloc, __shfl_xor(mloc, 32, WAVE)));
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < ND; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    // l_run is this lane's half of the query's sum; the halves are added at the end
    float lsum = 0.f;
    bf16x8 pb[SUB][2];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[u][r], scale, -m_use));
        sacc[u][r] = p;
        lsum += p;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = pack_bf16x2(sacc[u][8 * c + 2 * e], sacc[u][8 * c + 2 * e + 1]);
        pb[u][c] = as_bf16x8(x);
      }
    }
    l_run += lsum;
    if constexpr (PIPE) {
      // O^T += V^T P^T: output blocks 0-1 from vf0, reading blocks 2-3's V
      // fragments under those products, then blocks 2-3
      auto pv = [&](int u, int c) { return __builtin_bit_cast(u32x4, pb[u][c]); };
      uint32_t va[8];
      u32x4 vf1[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dd = 0; dd < 2; ++dd)
#pragma unroll
          for (int c = 0; c < 2; ++c) va[(u * 2 + dd) * 2 + c] = sb + u * TILE + voff + c * (HD * 32) + (2 + dd) * 1024;
      att_quad(o[0], o[1], vf0[0], vf0[2], vf0[1], vf0[3], pv(0, 0), pv(0, 1), vf1[0], vf1[1], vf1[2], vf1[3], va[0], va[1],
               va[2], va[3]);
      att_quad(o[0], o[1], vf0[4], vf0[6], vf0[5], vf0[7], pv(1, 0), pv(1, 1), vf1[4], vf1[5], vf1[6], vf1[7], va[4], va[5],
               va[6], va[7]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int dd = 0; dd < 2; ++dd)
            o[2 + dd] = mfma32x32x16(as_bf16x8(vf1[(u * 2 + dd) * 2 + c]), pb[u][c], o[2 + dd]);
    } else {
      // O^T += V^T P^T; consecutive MFMAs go to different output blocks
      constexpr int DH = ND > 1 ? ND / 2 : 1;  // output blocks per batch of V reads
#pragma unroll
      for (int d0 = 0; d0 < ND; d0 += DH) {
        uint32_t va[SUB * 2 * DH];
        u32x4 vf[SUB * 2 * DH];
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int dd = 0; dd < DH; ++dd)
#pragma unroll
            for (int c = 0; c < 2; ++c)
              va[(u * DH + dd) * 2 + c] = sb + u * TILE + voff + c * (HD * 32) + (d0 + dd) * 1024;
        lds_read_n<SUB * 2 * DH>(va, vf);
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dd = 0; dd < DH; ++dd)
              o[d0 + dd] = mfma32x32x16(as_bf16x8(vf[(u * DH + dd) * 2 + c]), pb[u][c], o[d0 + dd]);
      }
    }
  }

  l_run += __shfl_xor(l_run, 32, WAVE);
  // lane holds O^T[d][query]: d = dc*32 + 8*(r/4) + 4*half + r%4
  if (jq >= a.Lq) return;
  if (splits == 1) {
    const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
    bf16_t* op = static_cast<bf16_t*>(a.o) + mrow * (a.H * HD) + h * HD + 4 * half;
#pragma unroll
    for (int dc = 0; dc < ND; ++dc)
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
    for (int dc = 0; dc < ND; ++dc)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(po + dc * 32 + 8 * q) =
            make_float4(o[dc][4 * q], o[dc][4 * q + 1], o[dc][4 * q + 2], o[dc][4 * q + 3]);
    if (half == 0) *reinterpret_cast<float2*>(a.part_ml + base * 2) = make_float2(m_run, l_run);
  }
}

// Merge split partials: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wavefront per (row, head): lane s holds split s's (m, l); each lane sums
// HD/64 (or one) output dims over the splits in split order (every split's
// partial is written, an empty one as zeros with weight 0).  The partials of the
// first 16 splits are loaded together with the (m, l) pairs, since they do not
// depend on them, so up to 16 splits take one memory round trip instead of
// three; further splits follow 16 at a time.
template <int HD>
__global__ void __launch_bounds__(256) k_attn_merge(AttnArgs a, int splits) {
  const int rows = a.B * a.Lq;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, head)
  const int lane = threadIdx.x & 63;
  if (pair >= rows * a.H) return;
  const int mrow = pair / a.H, h = pair % a.H;
  auto at = [&](int s) { return (static_cast<size_t>(s) * rows + mrow) * a.H + h; };
  constexpr int PER = HD >= 64 ? HD / 64 : 1;
  constexpr int B16 = 16;
  const int d0 = min(lane * PER, HD - PER);  // lanes past HD (HD < 64) duplicate the last dims, not stored
  float v[B16][PER];
  auto load = [&](int s0) {
#pragma unroll
    for (int k = 0; k < B16; ++k) {
      const float* po = a.part_o + at(min(s0 + k, splits - 1)) * HD + d0;
#pragma unroll
      for (int e = 0; e < PER; ++e) v[k][e] = po[e];
    }
  };
  load(0);
  float2 ml = make_float2(-INFINITY, 0.f);
  if (lane < splits) ml = *reinterpret_cast<const float2*>(a.part_ml + at(lane) * 2);
  float mx = ml.y > 0.f ? ml.x : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, WAVE));
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  const float wgt = (ml.y > 0.f) ? __builtin_amdgcn_exp2f(ml.x - mu) : 0.f;
  const float l = wave_sum(wgt * ml.y);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < splits; s0 += B16) {
    if (s0 > 0) load(s0);
#pragma unroll
    for (int k = 0; k < B16; ++k) {
      const float ws = __shfl(wgt, min(s0 + k, 63), WAVE);
      if (s0 + k < splits)
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += ws * v[k][e];
    }
  }
  if (lane * PER < HD) {
    bf16_t* op = static_cast<bf16_t*>(a.o) + static_cast<size_t>(mrow) * a.H * HD + h * HD + d0;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = f32_to_bf16(l > 0.f ? acc[e] / l : 0.f);
  }
}

// Key splits: enough (row, group, query block, split) workgroups for about one
// per CU, each split at least MIN_CHUNK keys; two per CU (about TARGET_WG in
// all) only while every split keeps at least LONG_CHUNK keys.  A split costs a
// pass over fp32 partials (written here, read by the merge): with ~2000 keys
// per split (batch 32 over 4096 positions) that outweighs the second workgroup
// (133 vs 109-123 us unsplit); with ~4000 (batch 4 over 65536) it does not
// (212 vs 224 us with one workgroup per CU).  At most 64 splits (one merge
// lane each).
constexpr int LONG_CHUNK = 3072;

int attn_splits(const AttnArgs& a, int* chunk_out) {
  const int qblocks = (a.Lq + 31) / 32;
  const long base = static_cast<long>(qblocks) * a.B * a.G;
  const int max_splits = std::max(1, std::min(a.max_kv / MIN_CHUNK, 64));
  auto want = [&](long wgs) { return static_cast<int>(std::min<long>(max_splits, std::max<long>(1, (wgs + base - 1) / base))); };
  int splits = want(TARGET_WG / 2);
  const int two = want(TARGET_WG);
  if (two > splits && a.max_kv / two >= LONG_CHUNK) splits = two;
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

size_t attn_partial_floats_bound(int R, int H, int G, int hd, int max_kv) {
  // splits <= min(ceil(max target / G), max_kv / MIN_CHUNK, 64) for any B, Lq with B*Lq <= R
  const int s = std::max(1, std::min({(TARGET_WG + G - 1) / G, max_kv / MIN_CHUNK, 64}));
  return attn_partial_floats(s, R, H, hd);
}

template <int HD, int GS>
static hipError_t launch(const AttnArgs& a, hipStream_t s) {
  int chunk = 0;
  const int splits = attn_splits(a, &chunk);
  const int qblocks = (a.Lq + 31) / 32;
  dim3 grid(splits, qblocks, a.B * a.G);
  // Large K/V streams of one launch (over 64 MB, a quarter of the 256 MB
  // last-level cache: their layers' K/V together cannot stay cached from one
  // denoise step to the next) load non-temporally and leave the cached data of
  // the rest of the step alone.  8B-class full model: batch 4 over 65536
  // positions (1 GB per layer) 12.25 -> 11.79 ms per denoise step, batch 32
  // over ~1100 (150 MB) 19.04 -> 18.93 ms.  Small K/V stay cacheable: the
  // denoise steps of a block re-read the same prefix (batch 1 over 4096
  // positions, 17 MB, was slower with non-temporal loads).
  const double kv_bytes = 2.0 * a.B * a.G * static_cast<double>(a.max_kv) * HD * 2;
  // Ring depth and load schedule by launch shape (interleaved medians against
  // two stages issued at once after each barrier; outputs identical):
  // - at most one workgroup per CU and >= 2048 keys per workgroup: three
  //   stages, loads spread (batch 32 over 4096 positions 107.4 -> 102.4 us;
  //   three stages issued at once measured 150 us);
  // - two workgroups per CU: two stages each, loads spread (batch 4 over 65536
  //   positions 198.3 -> 190.2 us);
  // - otherwise two stages issued at once (short key ranges: batch 1 over 4096
  //   positions, 160 keys per split, and batch 8 were ~0.4 us slower deeper).
  const long wgs = static_cast<long>(grid.x) * grid.y * grid.z;
  const int mode = wgs > 256 ? 1 : (chunk >= 2048 ? 2 : 0);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(GS * 64), 0, s, a, chunk); };
  if (kv_bytes > 64.0 * (1 << 20)) {
    if (mode == 2) go(k_attn<HD, GS, true, 3, true>);
    else if (mode == 1) go(k_attn<HD, GS, true, 2, true>);
    else go(k_attn<HD, GS, true, 2, false>);
  } else {
    if (mode == 2) go(k_attn<HD, GS, false, 3, true>);
    else if (mode == 1) go(k_attn<HD, GS, false, 2, true>);
    else go(k_attn<HD, GS, false, 2, false>);
  }
  if (splits > 1) {
    const int pairs = a.B * a.Lq * a.H;
    hipLaunchKernelGGL((k_attn_merge<HD>), dim3((pairs + 3) / 4), dim3(256), 0, s, a, splits);
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
