// Column mean over packed pair rows (DanLing NestedTensor, Equation 4 and the
// mean of Equation 1's third line), M_i cells per row (N_i for square pairs):
//   m[eta_i + r, :] = (1 / M_i) * sum_{c < M_i} z[o_i + r M_i + c, :].
// With `mean` false the sum is returned undivided: the row operand's
// gradient of the broadcast (Equation 1's first line differentiated).
// HBM-read bound. Deterministic: each row is summed by one wave or one
// workgroup in a fixed order (no atomics).
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;

// A pair state above kStreamBytes is read with nontemporal loads: on
// long_square_x4 (459.5 MB) the column mean then takes 68.5 us instead of
// 80.6 us; on a pair state that fits the cache (near_uniform_x4, 242 MB)
// cached loads are 5% faster.

// 16 bytes at p; STREAM: a nontemporal load
template <typename T, bool STREAM>
__device__ __forceinline__ Vec16<T> load_row16(const T* p) {
  if constexpr (STREAM) {
    Vec16<T> r;
    r.v = __builtin_nontemporal_load(reinterpret_cast<const decltype(r.v)*>(p));
    return r;
  } else {
    return load16(p);
  }
}

// Sum of the 16-byte vectors at cells c0, c0 + step, ... < n of one pair row.
template <typename T, bool STREAM>
__device__ __forceinline__ void row_partial(float (&acc)[Vec16<T>::N], const T* row_base,
                                            int64_t c0, int64_t n, int64_t step, int c_z) {
  constexpr int VEC = Vec16<T>::N;
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  int64_t c = c0;
  for (; c + (kUnroll - 1) * step < n; c += kUnroll * step) {
    Vec16<T> v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_row16<T, STREAM>(row_base + (c + u * step) * c_z);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += v[u].get(e);
  }
  for (; c < n; c += step) {
    const Vec16<T> v = load_row16<T, STREAM>(row_base + c * c_z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += v.get(e);
  }
}

// A cell's c_z values are sl slices of G feature vectors (G a power of two
// <= 64; sl = 1 unless c_z / VEC is not one, as for the S slices of the
// non-leading layout). Lane (f, cl) of a wave holds vector f of a slice of
// every (64/G)-th cell; a butterfly over the cell-lane bits sums the lanes
// that share f. The slices of a row are summed one after another.
template <typename T, int G, bool STREAM>
__global__ __launch_bounds__(kThreads) void k_reduce_pow2(
    const T* __restrict__ z, float* __restrict__ m, const int64_t* __restrict__ item_offsets,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ col_lengths, int B,
    int c_z, int sl, bool mean) {
  constexpr int VEC = Vec16<T>::N;
  constexpr int CLW = 64 / G;
  __shared__ float part[kWaves][G * VEC];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int f = lane % G, cl = lane / G;
  const int64_t item = blockIdx.x;
  const int i = find_segment(item_offsets, 0, B, item);
  const int64_t rows = lengths[i];   // N_i
  const int64_t n = col_lengths[i];  // M_i, cells per row and the divisor
  const int64_t eta = single_offsets[i];
  const int64_t o = pair_offsets[i];
  const int64_t j = item - item_offsets[i];
  const float nf = mean ? (float)n : 1.f;  // dividing by 1 is exact
  float acc[VEC];
  if (n >= kLongRow) {
    // one row, every wave takes a share of its cells
    const int64_t r = j;
    for (int sc = 0; sc < sl; ++sc) {
      const int fo = (sc * G + f) * VEC;  // the lane's first value in the cell
      row_partial<T, STREAM>(acc, z + (o + r * n) * c_z + fo, wave * CLW + cl, n, kWaves * CLW,
                             c_z);
#pragma unroll
      for (int off = G; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
      if (cl == 0) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) part[wave][f * VEC + e] = acc[e];
      }
      __syncthreads();
      if (wave == 0 && cl == 0) {
        Vec16<float> out[VEC / 4];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float s = part[0][f * VEC + e];
#pragma unroll
          for (int w = 1; w < kWaves; ++w) s += part[w][f * VEC + e];
          out[e / 4].set(e % 4, s / nf);
        }
        float* dst = m + (eta + r) * c_z + fo;
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) store16(dst + 4 * q, out[q]);
      }
      __syncthreads();  // part is written again for the next slice
    }
  } else {
    // a group of whole rows; each wave reduces its own rows
    const int64_t R = rows_per_item(n);
    const int64_t r0 = j * R;
    const int64_t r1 = r0 + R < rows ? r0 + R : rows;
    for (int64_t r = r0 + wave; r < r1; r += kWaves) {
      for (int sc = 0; sc < sl; ++sc) {
        const int fo = (sc * G + f) * VEC;
        row_partial<T, STREAM>(acc, z + (o + r * n) * c_z + fo, cl, n, CLW, c_z);
#pragma unroll
        for (int off = G; off < 64; off <<= 1)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
        if (cl == 0) {
          float* dst = m + (eta + r) * c_z + fo;
#pragma unroll
          for (int q = 0; q < VEC / 4; ++q) {
            Vec16<float> out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out.set(e, acc[4 * q + e] / nf);
            store16(dst + 4 * q, out);
          }
        }
      }
    }
  }
}

// Any width: one thread per (pair row, 16-byte feature vector), summing the
// row's cells in order.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_reduce_generic(
    const T* __restrict__ z, float* __restrict__ m, const int64_t* __restrict__ row_splits,
    const int32_t* __restrict__ row_sample, const int32_t* __restrict__ col_lengths, int64_t T_rows,
    int c_z, int G, bool mean) {
  constexpr int VEC = Vec16<T>::N;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= T_rows * G) return;
  const int64_t g = idx / G;
  const int f = (int)(idx - g * G);
  const int64_t n = col_lengths[row_sample[g]];
  const float nf = mean ? (float)n : 1.f;
  float acc[VEC];
  row_partial<T, false>(acc, z + row_splits[g] * c_z + f * VEC, 0, n, 1, c_z);
  float* dst = m + g * c_z + f * VEC;
#pragma unroll
  for (int q = 0; q < VEC / 4; ++q) {
    Vec16<float> out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out.set(e, acc[4 * q + e] / nf);
    store16(dst + 4 * q, out);
  }
}

template <typename T, int G>
hipError_t launch_pow2(const nt_partition& p, const void* z, float* m, int c_z, int sl,
                       bool mean, hipStream_t stream) {
  const bool stream_z = p.cells * c_z * (int64_t)sizeof(T) > kStreamBytes;
  auto kern = stream_z ? k_reduce_pow2<T, G, true> : k_reduce_pow2<T, G, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.n_items), dim3(kThreads), 0, stream,
                     static_cast<const T*>(z), m, p.item_offsets, p.pair_offsets,
                     p.single_offsets, p.lengths, p.col_lengths, p.B, c_z, sl, mean);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const nt_partition& p, const void* z, float* m, int c_z, bool mean,
                    hipStream_t stream) {
  const int vecs = c_z / Vec16<T>::N;  // feature vectors per cell
  // the slices: the largest power of two <= 64 that divides vecs, at least 4
  int G = 64;
  while (G > 4 && vecs % G != 0) G >>= 1;
  if (vecs % G == 0) {
    const int sl = vecs / G;
    switch (G) {
      case 4: return launch_pow2<T, 4>(p, z, m, c_z, sl, mean, stream);
      case 8: return launch_pow2<T, 8>(p, z, m, c_z, sl, mean, stream);
      case 16: return launch_pow2<T, 16>(p, z, m, c_z, sl, mean, stream);
      case 32: return launch_pow2<T, 32>(p, z, m, c_z, sl, mean, stream);
      case 64: return launch_pow2<T, 64>(p, z, m, c_z, sl, mean, stream);
      default: break;
    }
  }
  switch (vecs) {
    case 1: return launch_pow2<T, 1>(p, z, m, c_z, 1, mean, stream);
    case 2: return launch_pow2<T, 2>(p, z, m, c_z, 1, mean, stream);
    default: break;
  }
  const int G1 = vecs;
  const int64_t total = p.T * G1;
  hipLaunchKernelGGL(k_reduce_generic<T>, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, static_cast<const T*>(z), m, p.row_splits,
                     p.row_sample, p.col_lengths, p.T, c_z, G1, mean);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const nt_partition& p, const void* z, float* m, int c_z, nt_dtype dtype,
                         hipStream_t stream, bool mean) {
  if (p.T == 0) return hipSuccess;
  if (dtype == NT_BF16) return launch_t<bf16>(p, z, m, c_z, mean, stream);
  return launch_t<float>(p, z, m, c_z, mean, stream);
}

}  // namespace nt
