// bf16 MFMA GEMMs of the denoising path, C = A[M][K] * W[N][K]^T with fp32
// accumulation, and their fused epilogues (bf16 store, residual add, SwiGLU,
// LM-head confidence partials).
//
// The products are computed transposed, D[n][m] = W * A^T, so that each lane of
// an MFMA result holds consecutive output columns of one row and stores them as
// one vector.
//
// One tiled kernel for every shape: 256 x 256, 256 x 320 (LM head, rows split
// evenly on the device), 256 x 128, 192 x 128, 256 x 64, 256 x 32, 128 x 128,
// 128 x 64 or 128 x 32 output tiles, 32- or 64-deep K stages in a ring of LDS
// buffers filled by direct global-to-LDS loads, each wavefront a block of
// v_mfma_f32_32x32x16_bf16 tiles.  Short products (one canvas at batch 1-2) are HBM-bound: their
// activation rows are loaded once per workgroup and shared from LDS, their
// weights (read once) with non-temporal loads, and when there are too few
// weight tiles to fill the chip K is split over workgroups, the fp32 partials
// summed in a fixed order by a second kernel or by the caller's next step (no
// cross-workgroup atomics or fences).
#include <algorithm>

#include "dlm_device.h"
#include "dlm_internal.h"

namespace dlm {

// g * sigmoid(g) with the hardware reciprocal (1 ulp; the product is stored as
// bf16) instead of an IEEE division: exp(-g) -> inf for g << 0 gives g * 0.
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

__device__ __forceinline__ MaxSumIdx msi_shfl_xor(MaxSumIdx a, int mask) {
  MaxSumIdx b;
  b.m = __shfl_xor(a.m, mask, WAVE);
  b.s = __shfl_xor(a.s, mask, WAVE);
  b.idx = __shfl_xor(a.idx, mask, WAVE);
  b.t = __shfl_xor(a.t, mask, WAVE);
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
    x.x += g.alpha * v[0];
    x.y += g.alpha * v[1];
    x.z += g.alpha * v[2];
    x.w += g.alpha * v[3];
    *reinterpret_cast<float4*>(o) = x;
  }
}

// ======================================================== tiled GEMM ====
// BN x BM output tile (weights x activations) per workgroup of WN x WM
// wavefronts, each a (BN/WN) x (BM/WM) block of 32 x 32 MFMA tiles.
//
// K runs in BK-deep stages through a ring of NBUF LDS buffers filled by direct
// global-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land at
// the instruction's LDS base + 16 * lane), so NBUF - 1 stages are in flight
// while one is multiplied, without staging registers.  One wait + barrier per
// stage: it makes the stage visible to every wavefront and retires the buffer
// that the next load refills.  Operand fragments are read from LDS in inline
// asm that waits for its own reads, so the compiler's conservative wait for
// LDS DMA (it cannot tell the ring buffers apart) is never inserted.
//
// Tiles are ordered per XCD: workgroup i runs on XCD i % 8, so XCD x takes a
// contiguous range of tiles, activation tiles fastest, and the workgroups that
// share a weight tile share that XCD's L2.
constexpr int TL_BK = 32;                 // K per stage of the default tiles

// Byte offset of 16-byte chunk c of row `row` in a stage region of BK-deep
// rows (BK*2 bytes: 4 or 8 chunks).  The LDS serves 16 lanes (256 bytes) per
// cycle; XOR-ing the chunk with the row's index among the rows that share a
// 256-byte bank line's position (row / rows-per-256-bytes) sends the 16 rows of
// one quarter of an MFMA operand read to 16 distinct 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  constexpr int ROW = BK * 2, CH = BK / 8, RP = 256 / ROW;
  return row * ROW + ((c ^ ((row / RP) & (CH - 1))) << 4);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// One 16-byte direct global-to-LDS load per lane: lane l's bytes land at
// lds_dst + 16 l (lds_dst must be the same for the whole wavefront).
__device__ __forceinline__ void load_lds16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}
// The same marked non-temporal (cache policy NT): lines that are read once are
// evicted first, so they do not push out cached data of later kernels.
__device__ __forceinline__ void load_lds16_nt(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 2);
}

// Wait until at most N of this wavefront's vector-memory operations are
// outstanding, then join the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(N) : "memory");
}

// Fragment reads of one 16-deep step: TN weight fragments at a + D i and TM
// activation fragments at b + D j (consecutive 32-row blocks, D bytes apart),
// each one ds_read_b128 per lane; the asm waits for its reads before returning.
template <int TN, int TM, int D>
__device__ __forceinline__ void lds_frags(uint32_t a, uint32_t b, u32x4 (&fa)[TN], u32x4 (&fb)[TM]);

template <int D>
__device__ __forceinline__ void lds_frags_2_4(uint32_t a, uint32_t b, u32x4 (&fa)[2], u32x4 (&fb)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:%8\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "ds_read_b128 %4, %7 offset:%9\n\t"
      "ds_read_b128 %5, %7 offset:%10\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fb[0]), "=&v"(fb[1]), "=&v"(fb[2]), "=&v"(fb[3])
      : "v"(a), "v"(b), "i"(D), "i"(2 * D), "i"(3 * D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void lds_frags_2_5(uint32_t a, uint32_t b, u32x4 (&fa)[2], u32x4 (&fb)[5]) {
  asm volatile(
      "ds_read_b128 %0, %7\n\t"
      "ds_read_b128 %1, %7 offset:%9\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %8 offset:%9\n\t"
      "ds_read_b128 %4, %8 offset:%10\n\t"
      "ds_read_b128 %5, %8 offset:%11\n\t"
      "ds_read_b128 %6, %8 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fb[0]), "=&v"(fb[1]), "=&v"(fb[2]), "=&v"(fb[3]), "=&v"(fb[4])
      : "v"(a), "v"(b), "i"(D), "i"(2 * D), "i"(3 * D), "i"(4 * D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void lds_frags_2_2(uint32_t a, uint32_t b, u32x4 (&fa)[2], u32x4 (&fb)[2]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %5\n\t"
      "ds_read_b128 %3, %5 offset:%6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fb[0]), "=&v"(fb[1])
      : "v"(a), "v"(b), "i"(D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void lds_frags_1_2(uint32_t a, uint32_t b, u32x4 (&fa)[1], u32x4 (&fb)[2]) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b128 %2, %4 offset:%5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fb[0]), "=&v"(fb[1])
      : "v"(a), "v"(b), "i"(D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void lds_frags_2_1(uint32_t a, uint32_t b, u32x4 (&fa)[2], u32x4 (&fb)[1]) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %3 offset:%5\n\t"
      "ds_read_b128 %2, %4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fb[0])
      : "v"(a), "v"(b), "i"(D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void lds_frags_3_2(uint32_t a, uint32_t b, u32x4 (&fa)[3], u32x4 (&fb)[2]) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:%7\n\t"
      "ds_read_b128 %2, %5 offset:%8\n\t"
      "ds_read_b128 %3, %6\n\t"
      "ds_read_b128 %4, %6 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fb[0]), "=&v"(fb[1])
      : "v"(a), "v"(b), "i"(D), "i"(2 * D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void lds_frags_1_1(uint32_t a, uint32_t b, u32x4 (&fa)[1], u32x4 (&fb)[1]) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa[0]), "=&v"(fb[0])
      : "v"(a), "v"(b)
      : "memory");
}

template <int TN, int TM, int D>
__device__ __forceinline__ void lds_frags(uint32_t a, uint32_t b, u32x4 (&fa)[TN], u32x4 (&fb)[TM]) {
  if constexpr (TN == 3 && TM == 2)
    lds_frags_3_2<D>(a, b, fa, fb);
  else if constexpr (TN == 2 && TM == 1)
    lds_frags_2_1<D>(a, b, fa, fb);
  else if constexpr (TN == 2 && TM == 4)
    lds_frags_2_4<D>(a, b, fa, fb);
  else if constexpr (TN == 2 && TM == 5)
    lds_frags_2_5<D>(a, b, fa, fb);
  else if constexpr (TN == 2 && TM == 2)
    lds_frags_2_2<D>(a, b, fa, fb);
  else if constexpr (TN == 1 && TM == 2)
    lds_frags_1_2<D>(a, b, fa, fb);
  else if constexpr (TN == 1 && TM == 1)
    lds_frags_1_1<D>(a, b, fa, fb);
  else
    static_assert(TN < 0, "no fragment reader for this wavefront tile");
}

// One 16-deep step of a 2 x 4-fragment wavefront tile: the next step's six
// fragment reads (weights at a + D i, activations at b + D j) are issued first
// and land under this step's eight products; the asm waits for the reads
// before returning, so na/nb are complete when it ends.
template <int D>
__device__ __forceinline__ void step_2_4(uint32_t a, uint32_t b, const u32x4 (&fa)[2], const u32x4 (&fb)[4],
                                         u32x4 (&na)[2], u32x4 (&nb)[4], f32x16 (&acc)[2][4]) {
  asm volatile(
      "ds_read_b128 %8, %20\n\t"
      "ds_read_b128 %9, %20 offset:%22\n\t"
      "ds_read_b128 %10, %21\n\t"
      "ds_read_b128 %11, %21 offset:%22\n\t"
      "ds_read_b128 %12, %21 offset:%23\n\t"
      "ds_read_b128 %13, %21 offset:%24\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %14, %16, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %14, %17, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %14, %18, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %14, %19, %3\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %15, %16, %4\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %15, %17, %5\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %15, %18, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %15, %19, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]), "+v"(acc[1][0]), "+v"(acc[1][1]),
        "+v"(acc[1][2]), "+v"(acc[1][3]), "=&v"(na[0]), "=&v"(na[1]), "=&v"(nb[0]), "=&v"(nb[1]), "=&v"(nb[2]),
        "=&v"(nb[3])
      : "v"(fa[0]), "v"(fa[1]), "v"(fb[0]), "v"(fb[1]), "v"(fb[2]), "v"(fb[3]), "v"(a), "v"(b), "i"(D), "i"(2 * D),
        "i"(3 * D)
      : "memory");
}

// The same for the 3 x 2 and 2 x 2 wavefront tiles of the 4-wavefront tiles.
template <int D>
__device__ __forceinline__ void step_3_2(uint32_t a, uint32_t b, const u32x4 (&fa)[3], const u32x4 (&fb)[2],
                                         u32x4 (&na)[3], u32x4 (&nb)[2], f32x16 (&acc)[3][2]) {
  asm volatile(
      "ds_read_b128 %6, %16\n\t"
      "ds_read_b128 %7, %16 offset:%18\n\t"
      "ds_read_b128 %8, %16 offset:%19\n\t"
      "ds_read_b128 %9, %17\n\t"
      "ds_read_b128 %10, %17 offset:%18\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %11, %14, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %11, %15, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %12, %14, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %12, %15, %3\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %13, %14, %4\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %13, %15, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[2][0]), "+v"(acc[2][1]),
        "=&v"(na[0]), "=&v"(na[1]), "=&v"(na[2]), "=&v"(nb[0]), "=&v"(nb[1])
      : "v"(fa[0]), "v"(fa[1]), "v"(fa[2]), "v"(fb[0]), "v"(fb[1]), "v"(a), "v"(b), "i"(D), "i"(2 * D)
      : "memory");
}

template <int D>
__device__ __forceinline__ void step_2_2(uint32_t a, uint32_t b, const u32x4 (&fa)[2], const u32x4 (&fb)[2],
                                         u32x4 (&na)[2], u32x4 (&nb)[2], f32x16 (&acc)[2][2]) {
  asm volatile(
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %12 offset:%14\n\t"
      "ds_read_b128 %6, %13\n\t"
      "ds_read_b128 %7, %13 offset:%14\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %8, %10, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %8, %11, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %9, %10, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %9, %11, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]), "=&v"(na[0]), "=&v"(na[1]),
        "=&v"(nb[0]), "=&v"(nb[1])
      : "v"(fa[0]), "v"(fa[1]), "v"(fb[0]), "v"(fb[1]), "v"(a), "v"(b), "i"(D)
      : "memory");
}

template <int TN, int TM, int D>
__device__ __forceinline__ void step_pipe(uint32_t a, uint32_t b, const u32x4 (&fa)[TN], const u32x4 (&fb)[TM],
                                          u32x4 (&na)[TN], u32x4 (&nb)[TM], f32x16 (&acc)[TN][TM]) {
  if constexpr (TN == 3 && TM == 2)
    step_3_2<D>(a, b, fa, fb, na, nb, acc);
  else if constexpr (TN == 2 && TM == 2)
    step_2_2<D>(a, b, fa, fb, na, nb, acc);
  else
    static_assert(TN < 0, "no pipelined step for this wavefront tile");
}

// The 4-wavefront tiles with 128 or more rows (one wavefront per SIMD) run a
// pipelined ring (see gemm_tile) wherever all of a wavefront's fragments are
// live.
template <int T, int BM, int TN, int TM>
constexpr bool pipe_ring() {
  return T == 256 && BM >= 128 && ((TN == 3 && TM == 2) || (TN == 2 && TM == 2));
}

// The 8-wavefront 256 x 256 tiles with 64-deep stages run a split ring (see
// gemm_tile): weights in two 32 KB buffers, activations in three.
template <int T, int BN, int BM, int NBUF, int BK>
constexpr bool split_ring() {
  return T == 512 && BN == 256 && BM == 256 && NBUF == 2 && BK == 64;
}

// With DYN the live rows (the device row count) are split evenly, in 32-row
// units, over the fewest tiles of at most BM rows, so that a count just past a
// multiple of the tile height does not cost one more pass over the weights;
// tiles past that number exit.
template <int T, int BN, int BM, int NBUF, int BK>
struct TileLds {
  static constexpr int BYTES = split_ring<T, BN, BM, NBUF, BK>() ? 5 * BN * BK * 2 : NBUF * (BN + BM) * BK * 2;
};

template <int EPI, int BN, int BM, int WN, int WM, int NBUF, int BK, bool DYN>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, uint8_t* lds) {
  constexpr int T = WN * WM * 64;
  constexpr int TN = BN / WN / 32, TM = BM / WM / 32;
  constexpr int ROW = BK * 2, CH = BK / 8;         // bytes and 16-byte chunks per stage row
  constexpr int STAGE = (BN + BM) * ROW;          // bytes per stage
  constexpr int BLK = STAGE / 1024 / (T / 64);    // 1-KB load blocks per wavefront per stage
  static_assert(STAGE % (1024 * (T / 64)) == 0, "stage must split into 1 KB blocks per wavefront");
  static_assert(BN % (1024 / ROW) == 0, "a 1 KB block must not straddle the weight/activation regions");
  static_assert(NBUF >= 2 && NBUF <= 6, "wait ladder covers up to four later stages");

  // tile = (weight tile, K range, activation tile), activation tiles fastest.
  // The grid is sized for M rows; the tiles are laid out for the live rows, so
  // that with a smaller device row count every XCD's live tiles come first in
  // its dispatch order and the surplus workgroups exit at the end (interleaved
  // idle workgroups measured ~1.6x slower).
  const int S = EPI == EPI_SPLITK ? g.ksplit : 1;
  const int live_rows = g.m_dev ? min(g.M, *g.m_dev) : g.M;
  const int nt = (live_rows + BM - 1) / BM;  // row tiles
  const int total = g.N / BN * S * nt, per = (total + 7) / 8;
  if (static_cast<int>(blockIdx.x / 8) >= per) return;
  const int tid_ = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tid_ >= total) return;
  int n0 = (tid_ / (nt * S)) * BN, split = (tid_ / nt) % S, mi = tid_ % nt;
  if (g.weights_fastest) {  // weight tiles fastest, then row tiles, then K ranges
    const int nn = g.N / BN;
    n0 = (tid_ % nn) * BN;
    mi = (tid_ / nn) % nt;
    split = tid_ / (nn * nt);
  }
  // this tile's rows are [m0, M)
  int m0 = mi * BM, M = live_rows;
  if constexpr (DYN) {
    const int rows = ((live_rows + nt - 1) / nt + 31) & ~31;
    m0 = mi * rows;
    M = min(live_rows, m0 + rows);
  }
  if (m0 >= M) return;

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = w % WN, wm = w / WN;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* W = static_cast<const bf16_t*>(g.w);

  // Load block q = w*BLK + b of a stage is 1 KB of whole rows; lane l fills the
  // 16-byte slot 64q + l, i.e. a physical chunk of one row of its region, and so
  // reads the logical chunk that the swizzle puts there.
  const bf16_t* src[BLK];
#pragma unroll
  for (int b = 0; b < BLK; ++b) {
    const int slot = (w * BLK + b) * 64 + lane;
    const int row = slot / CH;
    const int c = (slot % CH) ^ ((row / (256 / ROW)) & (CH - 1));
    if (row < BN) {
      src[b] = W + static_cast<size_t>(n0 + row) * g.K + c * 8;
    } else {
      const int m = min(m0 + row - BN, M - 1);  // rows past M repeat the last row; discarded
      src[b] = A + static_cast<size_t>(m) * g.lda + c * 8;
    }
  }
  // this workgroup's stages: [k_lo, k_lo + nk) of the K / 32 stages
  const int k_lo = split * (g.K / BK) / S;
  const int nk = (split + 1) * (g.K / BK) / S - k_lo;
  // Products of short row counts (one canvas at batch 1-2: the split layer
  // projections and the LM head) read every weight exactly once: those weight
  // loads are non-temporal, which keeps them from pushing out data the rest of
  // the step reuses (8B-class full model at batch 1: 4.32 -> 4.27 ms per denoise
  // step over a 1024-position prefix, 4.49 -> 4.31 over 4096, for the split
  // projections; 0.193 -> 0.165 ms for the head).  Only with 64-deep stages: a
  // 32-deep stage reads half of each 128-byte weight line, and an early-evicted
  // line is fetched again for the other half (the head took 0.266 ms).  The
  // batch-32 tiles reuse weight tiles across row tiles and keep normal loads.
  constexpr bool NT_W = (EPI == EPI_SPLITK || EPI == EPI_HEAD) && BM <= 64 && BK == 64;
  auto issue = [&](int kt) {  // kt counts this workgroup's stages from 0
    uint8_t* dst = lds + (kt % NBUF) * STAGE + w * BLK * 1024;
#pragma unroll
    for (int b = 0; b < BLK; ++b) {
      if (NT_W && (w * BLK + b) * 1024 / ROW < BN)  // a weight block
        load_lds16_nt(src[b] + (k_lo + kt) * BK, dst + b * 1024);
      else
        load_lds16(src[b] + (k_lo + kt) * BK, dst + b * 1024);
    }
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int arow = lane & 31, ahalf = lane >> 5;
  // fragment offsets within a stage for its 16-deep steps (chunk 2s + ahalf);
  // the swizzle key repeats every 32 rows, so consecutive 32-row blocks sit
  // 32 rows apart
  constexpr int NSTEP = BK / 16;
  uint32_t fa_off[NSTEP], fb_off[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    fa_off[s] = swz<BK>(wn * TN * 32 + arow, 2 * s + ahalf);
    fb_off[s] = BN * ROW + swz<BK>(wm * TM * 32 + arow, 2 * s + ahalf);
  }
  const uint32_t lbase = lds_addr(lds);
  constexpr bool SPLIT = split_ring<T, BN, BM, NBUF, BK>();
  constexpr bool PIPE = pipe_ring<T, BM, TN, TM>();
  // Activation fragments (32 rows each) past the live rows (the ragged last row
  // tile, e.g. the masked rows of the LM head) are not multiplied; a wavefront
  // with none left still loads its share of every stage and joins every
  // barrier, but skips its reads too.  In the split ring a wavefront multiplies
  // all of its fragments or none (a branch per product there cost more than the
  // products it saves).
  const int live = SPLIT ? (M > m0 + wm * TM * 32 ? TM : 0) : min(TM, max(0, (M - (m0 + wm * TM * 32) + 31) / 32));

  if constexpr (SPLIT) {
    // Split ring.  Loading a stage holds a wavefront at its DMA instructions
    // until the address unit has taken them, so a stage loaded by all eight
    // wavefronts at once leaves the matrix units idle for that time.  Here the
    // two wavefronts of each SIMD (w and w + 4) load at different times:
    // wavefronts 0-3 load the stage's weight half into a 2-deep ring at
    // [0, 2 HALF) right after the barrier, then multiply; wavefronts 4-7 (the
    // workgroup's waves go to the CU's four SIMDs in turn, so w and w + 4 share one)
    // multiply first and then load the activation half two stages ahead into a
    // 3-deep ring at [2 HALF, 5 HALF).  So one wavefront of a SIMD multiplies
    // while the other loads.  The products of each 16-deep step are issued with
    // the next step's fragment reads in flight (step_2_4).  Batch-32 gate/up
    // (1024 x 28672 x 4096): 0.257 -> 0.231 ms; LM head, 496 rows: 0.535 ->
    // 0.479 ms; down (K split): 0.126 -> 0.115 ms.
    constexpr int HALF = BN * ROW;
    static_assert(BLK == 8 && 4 * BLK * 1024 == HALF, "wavefronts 0-3 load exactly the weight half");
    static_assert(TN == 2 && TM == 4, "step_2_4 wavefront tiles");
    const bool early = w < 4;
    auto issue_half = [&](int kt) {
      uint8_t* dst = early ? lds + (kt & 1) * HALF + w * BLK * 1024 : lds + (2 + kt % 3) * HALF + (w - 4) * BLK * 1024;
#pragma unroll
      for (int b = 0; b < BLK; ++b) load_lds16(src[b] + (k_lo + kt) * BK, dst + b * 1024);
    };
    if (nk > 0) issue_half(0);
    if (!early && nk > 1) issue_half(1);
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt has landed: weights are the only loads in flight of 0-3;
      // 4-7 may keep stage kt + 1's activations in flight
      if (!early && kt + 1 < nk)
        wait_vm_barrier<BLK>();
      else
        wait_vm_barrier<0>();
      if (early && kt + 1 < nk) issue_half(kt + 1);
      if (live != 0) {
        // fb_off includes the weight region's HALF; the activation buffer of
        // stage kt starts at (2 + kt % 3) HALF
        const uint32_t sw = lbase + (kt & 1) * HALF, sa = lbase + (1 + kt % 3) * HALF;
        u32x4 fa[TN], fb[TM];
        lds_frags<TN, TM, 32 * ROW>(sw + fa_off[0], sa + fb_off[0], fa, fb);
#pragma unroll
        for (int s = 0; s + 1 < NSTEP; ++s) {
          u32x4 na[TN], nb[TM];
          step_2_4<32 * ROW>(sw + fa_off[s + 1], sa + fb_off[s + 1], fa, fb, na, nb, acc);
#pragma unroll
          for (int i = 0; i < TN; ++i) fa[i] = na[i];
#pragma unroll
          for (int j = 0; j < TM; ++j) fb[j] = nb[j];
        }
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) acc[i][j] = mfma32x32x16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j]);
      }
      // stage kt + 2 refills the activation buffer of stage kt - 1, which every
      // wavefront finished before this stage's barrier
      if (!early && kt + 2 < nk) issue_half(kt + 2);
    }
  } else {
    // Plain ring: every wavefront issues its share of stage kt + NBUF - 1 right
    // after the barrier, then multiplies stage kt step by step.
    auto plain_ring = [&]() {
#pragma unroll
      for (int p = 0; p < NBUF - 1; ++p)
        if (p < nk) issue(p);
      for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once at most the later stages' loads are outstanding
        const int later = min(nk - 1 - kt, NBUF - 2);
        if (later >= 4)
          wait_vm_barrier<4 * BLK>();
        else if (later == 3)
          wait_vm_barrier<3 * BLK>();
        else if (later == 2)
          wait_vm_barrier<2 * BLK>();
        else if (later == 1)
          wait_vm_barrier<BLK>();
        else
          wait_vm_barrier<0>();
        if (kt + NBUF - 1 < nk) issue(kt + NBUF - 1);
        if (live == 0) continue;
        const uint32_t sb = lbase + (kt % NBUF) * STAGE;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
          u32x4 fa[TN], fb[TM];
          lds_frags<TN, TM, 32 * ROW>(sb + fa_off[s], sb + fb_off[s], fa, fb);
#pragma unroll
          for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
              if (j < live) acc[i][j] = mfma32x32x16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j]);
        }
      }
    };
    if constexpr (PIPE) {
      static_assert(NBUF <= 4, "wait ladder of the pipelined ring covers two later stages");
      if (live == TM) {
        // Pipelined ring (one wavefront per SIMD, so nothing else on the SIMD
        // fills its stalls): each 16-deep step's products run with the next
        // step's fragment reads in flight (step_pipe), and the wavefront's
        // share of stage kt + NBUF - 1 is issued in pieces after each step's
        // products instead of all at once after the barrier.  With three
        // buffers (two stages in flight) on the batch-32 QKV (1024 x 6144 x
        // 4096, 192 x 128 tiles) and O (1024 x 4096 x 4096, 128 x 128) products:
        // 68.6 -> 62.7 us and 54.2 -> 50.8 us; with four (160 and 128 KB of
        // LDS) a further 64.6 -> 62.7 us and 52.1 -> 49.1 us.
#pragma unroll
        for (int p = 0; p < NBUF - 1; ++p)
          if (p < nk) issue(p);
        for (int kt = 0; kt < nk; ++kt) {
          const int later = min(nk - 1 - kt, NBUF - 2);
          if (later >= 2)
            wait_vm_barrier<2 * BLK>();
          else if (later == 1)
            wait_vm_barrier<BLK>();
          else
            wait_vm_barrier<0>();
          const bool more = kt + NBUF - 1 < nk;
          uint8_t* dst = lds + ((kt + NBUF - 1) % NBUF) * STAGE + w * BLK * 1024;
          const int koff = (k_lo + kt + NBUF - 1) * BK;
          const uint32_t sb = lbase + (kt % NBUF) * STAGE;
          u32x4 fa[TN], fb[TM];
          lds_frags<TN, TM, 32 * ROW>(sb + fa_off[0], sb + fb_off[0], fa, fb);
#pragma unroll
          for (int s = 0; s < NSTEP; ++s) {
            if (s + 1 < NSTEP) {
              u32x4 na[TN], nb[TM];
              step_pipe<TN, TM, 32 * ROW>(sb + fa_off[s + 1], sb + fb_off[s + 1], fa, fb, na, nb, acc);
#pragma unroll
              for (int i = 0; i < TN; ++i) fa[i] = na[i];
#pragma unroll
              for (int j = 0; j < TM; ++j) fb[j] = nb[j];
            } else {
#pragma unroll
              for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j) acc[i][j] = mfma32x32x16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j]);
            }
            if (more) {
#pragma unroll
              for (int b = s * BLK / NSTEP; b < (s + 1) * BLK / NSTEP; ++b) load_lds16(src[b] + koff, dst + b * 1024);
            }
          }
        }
      } else {
        plain_ring();
      }
    } else {
      plain_ring();
    }
  }

  // lane holds D[n][m]: m = m0 + (wm*TM + j)*32 + (lane&31),
  // n = n0 + (wn*TN + i)*32 + 8*(r/4) + 4*(lane>>5) + r%4
  if (EPI == EPI_SPLITK) {
    float* part = g.kpart + static_cast<size_t>(split) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + (wm * TM + j) * 32 + arow;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + i) * 32 + 8 * q + 4 * ahalf;
          *reinterpret_cast<float4*>(part + static_cast<size_t>(m) * g.N + n) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
  } else if (EPI == EPI_STORE_BF16 || EPI == EPI_RESID_F32) {
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
    // per (wavefront column, row) partials in the LDS of the ring, free once
    // every wavefront has left the main loop
    static_assert(4 * WN * BM * sizeof(float) <= NBUF * STAGE, "head partials must fit in the ring");
    __syncthreads();
    float* rm = reinterpret_cast<float*>(lds);
    float* rs = rm + WN * BM;
    float* rt = rs + WN * BM;
    int* ri = reinterpret_cast<int*>(rt + WN * BM);
    // Per row, two passes over the lane's TN x 16 logits: their max, then the
    // sums of exp2((x - max) log2 e) and of that times (x - max) log2 e, and the
    // lowest column holding the max.  The mask id's column (in at most one tile
    // of the vocabulary) is pinned to -1e30 first, so that it adds exactly
    // nothing and never holds the max.  A non-finite logit makes a sum NaN
    // (NaN and +inf through the exponential, -inf through 0 x -inf), which is
    // what flags the row.  Register r of fragment i holds column
    // nb + 32 i + 8 (r / 4) + r % 4.
    constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
    const int nb = n0 + wn * TN * 32 + 4 * ahalf;
    const bool mask_here = g.mask_id >= n0 && g.mask_id < n0 + BN;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int ml = (wm * TM + j) * 32 + arow, m = m0 + ml;
      if (g.logits && m < M) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = nb + 32 * i + 8 * q;
            float4 o4 = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            const int mk = g.mask_id - n;  // the mask id's lane of the quad, if any (selects, no indexing)
            o4.x = mk == 0 ? -INFINITY : o4.x;
            o4.y = mk == 1 ? -INFINITY : o4.y;
            o4.z = mk == 2 ? -INFINITY : o4.z;
            o4.w = mk == 3 ? -INFINITY : o4.w;
            *reinterpret_cast<float4*>(g.logits + static_cast<size_t>(g.logit_rows ? g.logit_rows[m] : m) * g.N + n) = o4;
          }
      }
      if (mask_here) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (nb + 32 * i + 8 * (r / 4) + r % 4 == g.mask_id) acc[i][j][r] = -1e30f;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      const float m2 = mx * LOG2E;
      float sum = 0.f, t2 = 0.f;
      int loc = -1;
#pragma unroll
      for (int i = TN - 1; i >= 0; --i)  // columns downwards: the last match is the lowest
#pragma unroll
        for (int r = 15; r >= 0; --r) {
          const float x = acc[i][j][r], d2 = fmaf(x, LOG2E, -m2), e = __builtin_amdgcn_exp2f(d2);
          sum += e;
          t2 = fmaf(e, d2, t2);
          loc = x == mx ? 32 * i + 8 * (r / 4) + r % 4 : loc;
        }
      bad |= !__builtin_isfinite(sum) || !__builtin_isfinite(t2);
      MaxSumIdx p{mx, sum, loc < 0 ? 0x7fffffff : nb + loc, t2 * LN2};
      p = msi_shfl_xor(p, 32);
      if (ahalf == 0) {
        rm[wn * BM + ml] = p.m;
        rs[wn * BM + ml] = p.s;
        rt[wn * BM + ml] = p.t;
        ri[wn * BM + ml] = p.idx;
      }
    }
    if (__ballot(bad) && lane == 0 && g.nonfinite) atomicAdd(g.nonfinite, 1);
    __syncthreads();
    for (int ml = threadIdx.x; ml < BM; ml += T) {
      const int m = m0 + ml;
      MaxSumIdx p{rm[ml], rs[ml], ri[ml], rt[ml]};
#pragma unroll
      for (int q = 1; q < WN; ++q)
        p = msi_combine(p, MaxSumIdx{rm[q * BM + ml], rs[q * BM + ml], ri[q * BM + ml], rt[q * BM + ml]});
      if (m < M)
        reinterpret_cast<float4*>(g.partials)[static_cast<size_t>(n0 / BN) * g.M + m] =
            make_float4(p.m, p.s, __int_as_float(p.idx), p.t);
    }
  }
}

template <int EPI, int BN, int BM, int WN, int WM, int NBUF, int BK, bool DYN>
__global__ void __launch_bounds__(WN * WM * 64) k_gemm_tiled(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[TileLds<WN * WM * 64, BN, BM, NBUF, BK>::BYTES];
  gemm_tile<EPI, BN, BM, WN, WM, NBUF, BK, DYN>(g, lds);
}

// The LM head over many scored rows, whose count only the device knows: every
// row tile is one more pass of the 1 GB of weights through LDS, so the launch
// takes 256-row tiles or the fewest tiles of up to 320 rows with the rows split
// evenly, whichever needs fewer (256-row tiles on a tie; e.g. 530 rows: two
// tiles of 288 rows instead of three of 256).  Both tile bodies live in this
// one kernel behind a branch on the count (the grid is sized for 256-row
// tiles, the larger count), which replaces a second launch that only read the
// count and exited (~4 us per step).
constexpr int HEAD_BM_MAX = 320;
__global__ void __launch_bounds__(512) k_gemm_head_rows(GemmArgs g) {
  constexpr int L256 = TileLds<512, 256, 256, 2, 64>::BYTES, L320 = TileLds<512, 256, HEAD_BM_MAX, 2, 64>::BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L256 > L320 ? L256 : L320];
  const int live = g.m_dev ? min(g.M, *g.m_dev) : g.M;
  if ((live + 255) / 256 <= (live + HEAD_BM_MAX - 1) / HEAD_BM_MAX)
    gemm_tile<EPI_HEAD, 256, 256, 4, 2, 2, 64, false>(g, lds);
  else
    gemm_tile<EPI_HEAD, 256, HEAD_BM_MAX, 4, 2, 2, 64, true>(g, lds);
}

// Sum of the K-split partials in split order (deterministic), then the
// epilogue; one thread per 4 output columns of one row.
template <int EPI>
__global__ void __launch_bounds__(256) k_splitk_reduce(GemmArgs g) {
  const int cols = EPI == EPI_SWIGLU ? g.N / 2 : g.N;
  const int q4 = cols / 4;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= g.M * q4) return;
  const int m = t / q4, c = (t % q4) * 4;
  const size_t plane = static_cast<size_t>(g.M) * g.N;
  const float* row = g.kpart + static_cast<size_t>(m) * g.N;
  if (EPI == EPI_SWIGLU) {
    // output column c of a 16-column group reads gate row 32*(c/16) + c%16 and
    // the up row 16 further (gate/up rows interleaved by 16)
    const int n = 32 * (c / 16) + c % 16;
    const float4 gs = sum_planes(row + n, plane, g.ksplit), us = sum_planes(row + n + 16, plane, g.ksplit);
    bf16_t* o = static_cast<bf16_t*>(g.out) + static_cast<size_t>(m) * g.ldc + c;
    *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(silu_f(gs.x) * us.x, silu_f(gs.y) * us.y),
                                         pack_bf16x2(silu_f(gs.z) * us.z, silu_f(gs.w) * us.w)};
  } else {
    const float4 a = sum_planes(row + c, plane, g.ksplit);
    float v[4] = {a.x, a.y, a.z, a.w};
    store_quad<EPI>(g, m, c, v);
  }
}

// ============================================================== host ====
// LM-head vocabulary columns per partial record (the tiled kernels' BN).
int gemm_head_tile_n(int) { return 256; }

// Short products (M <= 64 rows: one canvas at batch 1-2) stream their weights
// once through 128 x 64 tiles (256 x 64 with many weight rows, below).  With
// too few weight tiles to fill the chip, K is split so that several hundred
// workgroups stream disjoint weight slices; each K range stays at least 16
// stages deep and at most 8 splits are made, since every split adds an fp32
// partial plane to write and reduce (measured best: 8 splits for 32-48 tiles).
constexpr int SK_BN = 128, SK_BM = 64;

// Long-K products with few 256 x 256 tiles (the down projection at batch 32:
// 64 tiles, K = 14336) split K so that about one 256 x 256 workgroup per CU
// runs, instead of 128 x 128 tiles that move twice the bytes per flop
// (168 -> 145 us).  Other products with few 128 x 128 tiles (QKV and O at
// batch 4: 48 and 32 tiles) split K over 128 x 128 tiles to about 256
// workgroups, each K range at least 8 stages (O at 256 rows: 46 -> 25 us).
constexpr int LK_MIN_K = 8192, FEW_TILES = 128;

static bool long_k_split(int M, int N, int K) {
  return M > SK_BM && N % 256 == 0 && K >= LK_MIN_K && (N / 256) * ((M + 255) / 256) < 256;
}

static int tiles128(int M, int N) { return (N / 128) * ((M + 127) / 128); }

// Short products with many weight rows (the SwiGLU gate/up at batch 1: 28672)
// stream through 256 x 64 tiles with 64-deep stages, two buffers and
// non-temporal weights, the LM head's short tile, K split for about 512
// workgroups: gate/up at 32 rows 51 -> 48 us, at one row 45 -> 40 us; the
// 8B-class full-model batch-1 step 4.17 -> 4.07 ms.
static bool short_wide(int N) { return N % 256 == 0 && N / SK_BN >= 128; }

int gemm_ksplit(int M, int N, int K) {
  if (long_k_split(M, N, K)) {
    const int tiles = (N / 256) * ((M + 255) / 256);
    return std::max(1, std::min({(256 + tiles - 1) / tiles, K / (16 * 64), SPLIT_MAX}));
  }
  if (M > SK_BM) {
    const int t = tiles128(M, N);
    if (t >= FEW_TILES) return 1;
    return std::max(1, std::min({(256 + t - 1) / t, K / (8 * 64), SPLIT_MAX}));
  }
  if (short_wide(N)) {
    const int t = N / 256;
    return std::max(1, std::min({(512 + t - 1) / t, K / (16 * 64), SPLIT_MAX}));
  }
  const int tiles = N / SK_BN;
  const int want = (640 + tiles - 1) / tiles;
  return std::max(1, std::min({want, K / (16 * TL_BK), SPLIT_MAX}));
}


size_t gemm_workspace_bytes(int M, int N, int K) {
  const int S = gemm_ksplit(M, N, K);
  return S > 1 ? static_cast<size_t>(S) * M * N * sizeof(float) : 0;
}

template <int EPI, int BN, int BM, int WN, int WM, int NBUF, int BK = TL_BK, bool DYN = false>
static void launch_tiled(const GemmArgs& g, hipStream_t s) {
  const int S = EPI == EPI_SPLITK ? g.ksplit : 1;
  const int total = (g.N / BN) * S * ((g.M + BM - 1) / BM);
  const int per = (total + 7) / 8;
  hipLaunchKernelGGL((k_gemm_tiled<EPI, BN, BM, WN, WM, NBUF, BK, DYN>), dim3(8 * per), dim3(WN * WM * 64), 0, s,
                     g);
}

// the partial-product launch of a split product (tile by shape)
static void launch_partials(const GemmArgs& h, hipStream_t s) {
  if (long_k_split(h.M, h.N, h.K)) {
    // Each XCD takes every weight tile of one K range for two row tiles, so the
    // row tiles' activations (1.8 MB each) stay in its L2 while the weights
    // stream past, instead of every XCD streaming all activations of every K
    // range (the down projection at batch 32: 149 -> 143 us).
    GemmArgs w = h;
    w.weights_fastest = 1;
    launch_tiled<EPI_SPLITK, 256, 256, 4, 2, 2, 64>(w, s);
  } else if (h.M > SK_BM) {
    launch_tiled<EPI_SPLITK, 128, 128, 2, 2, 3, 64>(h, s);
  } else if (short_wide(h.N)) {
    // one canvas (up to 32 rows): 32-row tiles, a tenth fewer bytes per stage
    // through LDS (this and the 128 x 32 tile below measured 0.2-0.4 us faster
    // on each of the four batch-1 projections, e.g. gate/up 52.6 -> 52.2 us)
    if (h.M <= 32)
      launch_tiled<EPI_SPLITK, 256, 32, 4, 1, 2, 64>(h, s);
    else
      launch_tiled<EPI_SPLITK, 256, 64, 4, 1, 2, 64>(h, s);
  } else if (h.M <= 32) {
    launch_tiled<EPI_SPLITK, SK_BN, 32, 4, 1, 3, 64>(h, s);
  } else {
    launch_tiled<EPI_SPLITK, SK_BN, SK_BM, 4, 1, 3, 64>(h, s);
  }
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  if constexpr (EPI == EPI_HEAD) {
    // The head streams 1 GB of weights: at up to 128 scored rows it is HBM-bound,
    // and short tiles whose activation rows every wavefront shares from LDS, two
    // workgroups per CU, keep the most bytes in flight.  Above that, every row
    // tile is one more pass of the weights through LDS, and the scored-row count
    // is known only on the device: one launch picks 256-row tiles or tiles of
    // up to 320 rows split evenly, whichever needs fewer (k_gemm_head_rows).
    if (g.M <= 32) {
      // one 32-row fragment per wavefront: a tenth fewer bytes per stage through
      // LDS than the 64-row tile (batch 1: 0.158 -> 0.156 ms)
      launch_tiled<EPI, 256, 32, 4, 1, 2, 64>(g, s);
    } else if (g.M <= 64) {
      // 64-deep stages, two buffers, non-temporal weights: 165 us (32-deep stages
      // with normal loads: 193 us with 4 buffers, 202 with 3, 212 with 6)
      launch_tiled<EPI, 256, 64, 4, 1, 2, 64>(g, s);
    } else if (g.M <= 128) {
      launch_tiled<EPI, 256, 128, 4, 2, 3>(g, s);
    } else if (g.M <= 256) {
      launch_tiled<EPI, 256, 256, 4, 2, 2, 64>(g, s);
    } else {
      // grid for 256-row tiles over the host bound (the larger of the two tilings)
      const int per = ((g.N / 256) * ((g.M + 255) / 256) + 7) / 8;
      hipLaunchKernelGGL(k_gemm_head_rows, dim3(8 * per), dim3(512), 0, s, g);
    }
  } else if (gemm_ksplit(g.M, g.N, g.K) > 1) {
    if (!g.kpart) return hipErrorInvalidValue;
    GemmArgs h = g;
    h.ksplit = gemm_ksplit(g.M, g.N, g.K);
    launch_partials(h, s);
    const int cols = EPI == EPI_SWIGLU ? g.N / 2 : g.N;
    hipLaunchKernelGGL((k_splitk_reduce<EPI>), dim3((g.M * (cols / 4) + 255) / 256), dim3(256), 0, s, h);
  } else if (g.M <= SK_BM) {
    launch_tiled<EPI, SK_BN, SK_BM, 4, 1, 3, 64>(g, s);
  } else {
    // 256 x 256 tiles where they still give at least one wave of workgroups
    // (the SwiGLU gate/up projection); else with at most one 128 x 128 tile per
    // CU (down, O projections at batch 32) one workgroup per CU with a deeper
    // ring of 64-deep stages; else 192 x 128 tiles where they come to at most
    // one per CU (QKV at batch 32: 6144 / 192 x 8 = 256 tiles, 80 -> 68 us
    // against two 256 x 128 tiles per CU); else 256 x 128 tiles, two per CU
    // with 32-deep stages (a third fewer bytes per flop than 128 x 128)
    const int t128 = (g.N / 128) * ((g.M + 127) / 128);
    if (g.N % 256 == 0 && (g.N / 256) * ((g.M + 255) / 256) >= 256)
      launch_tiled<EPI, 256, 256, 4, 2, 2, 64>(g, s);
    else if (t128 <= 256 && g.M > 128)  // several row tiles: MFMA-bound (O at 1024 rows 55 -> 52 us)
      launch_tiled<EPI, 128, 128, 2, 2, 4, 64>(g, s);
    else if (t128 <= 256)  // one row tile: HBM-bound, deeper ring (gate/up at 128 rows: 58 vs 74 us
      // with two buffers; four against three 63.6 -> 62.4 us)
      launch_tiled<EPI, 128, 128, 2, 2, 4, 64>(g, s);
    else if (g.N % 192 == 0 && (g.N / 192) * ((g.M + 127) / 128) <= 256)
      launch_tiled<EPI, 192, 128, 2, 2, 4, 64>(g, s);
    else if (g.N % 256 == 0)
      launch_tiled<EPI, 256, 128, 4, 2, 3>(g, s);
    else
      launch_tiled<EPI, 128, 128, 2, 2, 4>(g, s);
  }
  return hipGetLastError();
}

hipError_t gemm_partials(const GemmArgs& g, hipStream_t s) {
  const int S = gemm_ksplit(g.M, g.N, g.K);
  if (g.M <= 0 || S <= 1 || !g.kpart) return hipErrorInvalidValue;
  GemmArgs h = g;
  h.ksplit = S;
  launch_partials(h, s);
  return hipGetLastError();
}

hipError_t gemm(const GemmArgs& g, GemmEpilogue epi, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE_BF16: return launch_epi<EPI_STORE_BF16>(g, s);
    case EPI_RESID_F32: return launch_epi<EPI_RESID_F32>(g, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(g, s);
    case EPI_HEAD: return launch_epi<EPI_HEAD>(g, s);
    case EPI_SPLITK: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace dlm
