// Device-side helpers for the gfx950 kernels: vector types, bf16 packing,
// and the cell decode (Equation 3 of the DanLing NestedTensor paper inverted).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16 bytes of storage seen as VEC elements.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  bf16x8 v;
  __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
  __device__ __forceinline__ void set(int i, float x) { v[i] = (bf16)x; }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  f32x4 v;
  __device__ __forceinline__ float get(int i) const { return v[i]; }
  __device__ __forceinline__ void set(int i, float x) { v[i] = x; }
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T* p) {
  Vec16<T> r;
  r.v = *reinterpret_cast<const decltype(r.v)*>(p);
  return r;
}
template <typename T>
__device__ __forceinline__ void store16(T* p, const Vec16<T>& x) {
  *reinterpret_cast<decltype(x.v)*>(p) = x.v;
}

// Index i in [lo, hi) with off[i] <= t < off[i + 1], for a non-decreasing
// offset array with off[lo] <= t < off[hi]. Empty segments (repeated
// offsets) are never returned.
__device__ __forceinline__ int find_segment(const int64_t* __restrict__ off, int lo, int hi,
                                            int64_t t) {
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Decoded pair cell: sample i, pair row r, pair column c, the row singles'
// offset eta_i, the column singles' offset mu_i, and M_i, the cells per pair
// row (N_i for square pairs, whose mu is eta).
struct Cell {
  int i;
  int64_t r, c, eta, mu, m;
};

// Packed cell t -> (sample, row, col): the sample is found from the pair
// offsets, then t - o_i = r * M_i + c (Equation 3, row-major within the
// sample's N_i x M_i block).
__device__ __forceinline__ Cell decode_cell(const int64_t* __restrict__ pair_offsets,
                                            const int64_t* __restrict__ single_offsets,
                                            const int64_t* __restrict__ col_offsets,
                                            const int32_t* __restrict__ col_lengths, int B,
                                            int64_t t) {
  Cell x;
  x.i = find_segment(pair_offsets, 0, B, t);
  x.m = col_lengths[x.i];
  x.eta = single_offsets[x.i];
  x.mu = col_offsets[x.i];
  const int64_t local = t - pair_offsets[x.i];
  if (x.m <= 65535 && local <= 0xffffffffLL) {  // 32-bit division suffices
    const uint32_t l32 = (uint32_t)local, m32 = (uint32_t)x.m;
    const uint32_t q = l32 / m32;
    x.r = q;
    x.c = l32 - q * m32;
  } else {
    x.r = local / x.m;
    x.c = local - x.r * x.m;
  }
  return x;
}

}  // namespace nt
