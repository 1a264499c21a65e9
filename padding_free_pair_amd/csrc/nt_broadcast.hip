// Pair broadcast (DanLing NestedTensor, Equation 1 first line; Section 3.2
// "Creating axes through broadcasting"):
//   z[o_i + r M_i + c, :] = a[eta_i + r, :] + b[mu_i + c, :]
// (M_i = N_i and mu = eta for square pairs).
// HBM-write bound: each cell writes c_z elements, a and b are L2 resident.
//
// Batches of at most kTiledSamples samples take k_broadcast_tiled: a
// workgroup owns a tile of kTileRows pair rows x C pair columns of one sample
// and loads the tile's C column singles once into registers, then walks its
// rows (one row single each), so the L2 reads are (kTileRows + C) rows for
// kTileRows x C cells written instead of two rows per cell. Tiles are
// numbered sample by sample, row tiles outer; each workgroup finds its
// sample from an in-workgroup scan of the per-sample tile counts.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kThreads = 256;
constexpr int kSteps = 8;  // cells each thread visits

// VEC consecutive elements of TI widened to fp32.
template <typename TI, int VEC>
__device__ __forceinline__ void load_vec(const TI* p, float (&v)[VEC]) {
  constexpr int PER = Vec16<TI>::N;
#pragma unroll
  for (int q = 0; q < VEC / PER; ++q) {
    const Vec16<TI> x = load16(p + q * PER);
#pragma unroll
    for (int e = 0; e < PER; ++e) v[q * PER + e] = x.get(e);
  }
}

// Thread (f, cl) owns 16-byte output vector f of every CL-th cell of the
// workgroup's chunk of CL * kSteps consecutive cells. The cell decode is done
// once per thread and then advanced by CL cells at a time. TI is the type of
// a and b (T, or fp32 projections for a bf16 pair state: the sum is formed
// in fp32 and rounded once, as in the fused transition).
template <typename TI, typename T>
__global__ __launch_bounds__(kThreads) void k_broadcast(
    const TI* __restrict__ a, const TI* __restrict__ b, T* __restrict__ z,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths, int B,
    int64_t cells, int c_z, int G, int CL) {
  constexpr int VEC = Vec16<T>::N;
  const int tid = threadIdx.x;
  const int f = tid % G;
  const int cl = tid / G;
  if (cl >= CL) return;
  int64_t t = (int64_t)blockIdx.x * CL * kSteps + cl;
  if (t >= cells) return;
  Cell x = decode_cell(pair_offsets, single_offsets, col_offsets, col_lengths, B, t);
  int64_t end = pair_offsets[x.i + 1];  // first cell past the sample
  const int64_t fo = (int64_t)f * VEC;
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    float va[VEC], vb[VEC];
    load_vec<TI, VEC>(a + (x.eta + x.r) * c_z + fo, va);
    load_vec<TI, VEC>(b + (x.mu + x.c) * c_z + fo, vb);
    Vec16<T> out;
#pragma unroll
    for (int e = 0; e < VEC; ++e) out.set(e, va[e] + vb[e]);
    store16(z + t * c_z + fo, out);
    t += CL;
    if (k + 1 == kSteps || t >= cells) break;
    x.c += CL;
    if (x.c >= x.m) {
      if (x.m > CL && t < end) {  // at most one wrap into the next row
        x.c -= x.m;
        x.r += 1;
      } else {
        x = decode_cell(pair_offsets, single_offsets, col_offsets, col_lengths, B, t);
        end = pair_offsets[x.i + 1];
      }
    }
  }
}

constexpr int kTiledSamples = 256;
constexpr int kTileRows = 8;
constexpr int kColSteps = 2;  // column cells per thread

// Thread (f, ct): 16-byte output vector f of columns c0 + ct + CT u,
// u < kColSteps, for every row of the tile (CT = 256 / G cells side by side).
template <typename TI, typename T>
__global__ __launch_bounds__(kThreads) void k_broadcast_tiled(
    const TI* __restrict__ a, const TI* __restrict__ b, T* __restrict__ z,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ lengths,
    const int32_t* __restrict__ col_lengths, int B, int c_z, int G) {
  constexpr int VEC = Vec16<T>::N;
  __shared__ int64_t tile_end[kTiledSamples];  // inclusive prefix of tiles per sample
  __shared__ int64_t wave_sum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int CT = kThreads / G, C = CT * kColSteps;
  int64_t v = 0;
  if (tid < B) {
    const int64_t n = lengths[tid], m = col_lengths[tid];
    v = ((n + kTileRows - 1) / kTileRows) * ((m + C - 1) / C);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wave_sum[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += wave_sum[w];
  tile_end[tid] = v;
  __syncthreads();
  const int64_t g = blockIdx.x;
  if (B == 0 || g >= tile_end[B - 1]) return;  // the grid is an upper bound
  int lo = 0, hi = B - 1;  // first sample with tile_end > g
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tile_end[mid] > g) hi = mid; else lo = mid + 1;
  }
  const int i = lo;
  const int64_t local = g - (i > 0 ? tile_end[i - 1] : 0);
  const int64_t n = lengths[i], m = col_lengths[i];
  const int64_t nct = (m + C - 1) / C;
  const int64_t r0 = (local / nct) * kTileRows, c0 = (local % nct) * C;
  const int f = tid % G, ct = tid / G;
  const int64_t fo = (int64_t)f * VEC;
  const int64_t eta = single_offsets[i], mu = col_offsets[i], o = pair_offsets[i];
  float vb[kColSteps][VEC];
  bool ok[kColSteps];
#pragma unroll
  for (int u = 0; u < kColSteps; ++u) {
    const int64_t c = c0 + ct + CT * u;
    ok[u] = c < m;
    load_vec<TI, VEC>(b + (mu + (ok[u] ? c : 0)) * c_z + fo, vb[u]);
  }
  const int64_t rows = n - r0 < kTileRows ? n - r0 : kTileRows;
#pragma unroll
  for (int k = 0; k < kTileRows; ++k) {
    const int64_t r = r0 + (k < rows ? k : rows - 1);  // past the end: the last row, not stored
    float va[VEC];
    load_vec<TI, VEC>(a + (eta + r) * c_z + fo, va);
#pragma unroll
    for (int u = 0; u < kColSteps; ++u) {
      if (k < rows && ok[u]) {
        Vec16<T> out;
#pragma unroll
        for (int e = 0; e < VEC; ++e) out.set(e, va[e] + vb[u][e]);
        store16(z + (o + r * m + c0 + ct + CT * u) * c_z + fo, out);
      }
    }
  }
}

template <typename TI, typename T>
hipError_t launch_t(const nt_partition& p, const void* a, const void* b, void* z, int c_z,
                    hipStream_t stream) {
  const int G = c_z / Vec16<T>::N;  // <= 256 for c_z <= kMaxCz
  if (p.B <= kTiledSamples && G <= kThreads / 2) {
    // an upper bound of the tiles, sum ceil(N_i / R) ceil(M_i / C) <=
    // sum (N_i / R + 1)(M_i / C + 1), rounded up term by term; workgroups
    // past the last tile return at once
    const int64_t C = (kThreads / G) * kColSteps, RC = kTileRows * C;
    const int64_t tiles = (p.cells + RC - 1) / RC + (p.T + kTileRows - 1) / kTileRows +
                          (p.T_cols + C - 1) / C + p.B;
    hipLaunchKernelGGL((k_broadcast_tiled<TI, T>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, static_cast<const TI*>(a), static_cast<const TI*>(b),
                       static_cast<T*>(z), p.pair_offsets, p.single_offsets, p.col_offsets,
                       p.lengths, p.col_lengths, p.B, c_z, G);
    return hipGetLastError();
  }
  const int CL = kThreads / G;
  const int64_t per_block = (int64_t)CL * kSteps;
  const int64_t blocks = (p.cells + per_block - 1) / per_block;
  hipLaunchKernelGGL((k_broadcast<TI, T>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const TI*>(a), static_cast<const TI*>(b), static_cast<T*>(z),
                     p.pair_offsets, p.single_offsets, p.col_offsets, p.col_lengths, p.B, p.cells,
                     c_z, G, CL);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_broadcast(const nt_partition& p, const void* a, const void* b, void* z, int c_z,
                            nt_dtype dtype, hipStream_t stream, bool f32_inputs) {
  if (p.cells == 0) return hipSuccess;
  if (dtype == NT_BF16)
    return f32_inputs ? launch_t<float, bf16>(p, a, b, z, c_z, stream)
                      : launch_t<bf16, bf16>(p, a, b, z, c_z, stream);
  return launch_t<float, float>(p, a, b, z, c_z, stream);
}

}  // namespace nt
