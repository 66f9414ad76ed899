// Device-side helpers shared by the libdlm kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlm {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hw_f32x2 __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 per pair on
// gfx950); NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(hw_f32x2{lo, hi}, hw_bf16x2));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xffffu); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum of S <= SPLIT_MAX fp32 partial planes at p, p + plane, ... (split order).
// Every load is issued before the first add, so the S reads overlap instead of
// each waiting for the previous sum (S is uniform across the wavefront).
constexpr int SPLIT_MAX = 8;
__device__ __forceinline__ float4 sum_planes(const float* p, size_t plane, int S) {
  float4 a[SPLIT_MAX];
#pragma unroll
  for (int k = 0; k < SPLIT_MAX; ++k)
    if (k < S) a[k] = *reinterpret_cast<const float4*>(p + k * plane);
  float4 acc = a[0];
#pragma unroll
  for (int k = 1; k < SPLIT_MAX; ++k)
    if (k < S) {
      acc.x += a[k].x;
      acc.y += a[k].y;
      acc.z += a[k].z;
      acc.w += a[k].w;
    }
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Online-softmax / argmax partial: running max m, s = sum of exp(l - m), index
// of the max, and t = sum of exp(l - m) * (l - m), so that the entropy of the
// softmax is ln(s) - t / s.
struct MaxSumIdx {
  float m;
  float s;
  int idx;
  float t;
};

// Combine two partials: the max, its lowest index on ties, and the rescaled sum.
__device__ __forceinline__ MaxSumIdx msi_combine(MaxSumIdx a, MaxSumIdx b) {
  MaxSumIdx r;
  if (a.m > b.m || (a.m == b.m && a.idx < b.idx)) {
    r.m = a.m;
    r.idx = a.idx;
  } else {
    r.m = b.m;
    r.idx = b.idx;
  }
  // rescale each side to the new max: exp(l - M) = exp(m - M) exp(l - m), and
  // exp(l - M)(l - M) = exp(m - M) [exp(l - m)(l - m) + (m - M) exp(l - m)]
  float sa = 0.f, ta = 0.f, sb = 0.f, tb = 0.f;
  if (a.s != 0.f) {
    const float e = __expf(a.m - r.m);
    sa = a.s * e;
    ta = (a.t + (a.m - r.m) * a.s) * e;
  }
  if (b.s != 0.f) {
    const float e = __expf(b.m - r.m);
    sb = b.s * e;
    tb = (b.t + (b.m - r.m) * b.s) * e;
  }
  r.s = sa + sb;
  r.t = ta + tb;
  return r;
}

}  // namespace dlm
