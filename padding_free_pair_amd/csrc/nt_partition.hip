// Partition construction for square and rectangular pairs (DanLing
// NestedTensor, Section 3.1
// "Numerical storage" / Equation 2, Figure 2, Appendix A "Structural
// invariants") and the materialised cell decode used as a test hook.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kScanThreads = 256;

// One workgroup scans all B length pairs in chunks of 256, carrying the
// running totals: eta_i = sum_{k<i} N_k, mu_i = sum_{k<i} M_k,
// o_i = sum_{k<i} N_k M_k and the column-mean item offsets. Each chunk is an
// inclusive Hillis-Steele scan in LDS. mu is written when it is its own array.
__global__ __launch_bounds__(kScanThreads) void k_offsets_scan(
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ col_lengths, int B,
    int64_t* __restrict__ eta, int64_t* __restrict__ mu, int64_t* __restrict__ o,
    int64_t* __restrict__ items) {
  constexpr int Q = 4;
  __shared__ int64_t buf[2][Q][kScanThreads];
  __shared__ int64_t carry[Q];
  const int tid = threadIdx.x;
  const bool write_mu = mu != eta;
  if (tid < Q) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < B; base += kScanThreads) {
    const int idx = base + tid;
    const int64_t n = idx < B ? (int64_t)lengths[idx] : 0;
    const int64_t m = idx < B ? (int64_t)col_lengths[idx] : 0;
    const int64_t v[Q] = {n, m, n * m, items_of(n, m)};
    int cur = 0;
    for (int q = 0; q < Q; ++q) buf[cur][q][tid] = v[q];
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
      for (int q = 0; q < Q; ++q) {
        int64_t x = buf[cur][q][tid];
        if (tid >= off) x += buf[cur][q][tid - off];
        buf[cur ^ 1][q][tid] = x;
      }
      cur ^= 1;
      __syncthreads();
    }
    if (idx < B) {
      eta[idx] = carry[0] + buf[cur][0][tid] - v[0];
      if (write_mu) mu[idx] = carry[1] + buf[cur][1][tid] - v[1];
      o[idx] = carry[2] + buf[cur][2][tid] - v[2];
      items[idx] = carry[3] + buf[cur][3][tid] - v[3];
    }
    __syncthreads();
    if (tid == 0) {
      for (int q = 0; q < Q; ++q) carry[q] += buf[cur][q][kScanThreads - 1];
    }
    __syncthreads();
  }
  if (tid == 0) {
    eta[B] = carry[0];
    if (write_mu) mu[B] = carry[1];
    o[B] = carry[2];
    items[B] = carry[3];
  }
}

// Second-level row splits: pair row g = eta_i + r starts at o_i + r * M_i
// (Equation 3 at column 0); row_splits[T] closes with the cell total. The
// same threads fill the tile index: entry k holds the sample of cell 256 k.
__global__ __launch_bounds__(256) void k_row_splits(
    const int32_t* __restrict__ col_lengths, const int64_t* __restrict__ eta,
    const int64_t* __restrict__ o, int B, int64_t T, int64_t K,
    int64_t* __restrict__ row_splits, int32_t* __restrict__ row_sample,
    int32_t* __restrict__ tile_sample) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g == 0) row_splits[T] = o[B];
  if (g < K) tile_sample[g] = find_segment(o, 0, B, g * kSampleIndexSpan);
  if (g >= T) return;
  const int i = find_segment(eta, 0, B, g);
  const int64_t r = g - eta[i];
  row_splits[g] = o[i] + r * (int64_t)col_lengths[i];
  row_sample[g] = i;
}

// Small batches in one launch: the lengths travel by value in the kernel
// arguments (no host-to-device copy), every workgroup rescans them in LDS
// (at most kArgSamples entries), workgroup 0 writes the per-sample arrays and
// each workgroup fills 256 entries of the row splits.
struct LengthsArg {
  int32_t n[kArgSamples];
  int32_t m[kArgSamples];
};

__global__ __launch_bounds__(kArgSamples) void k_partition_small(
    LengthsArg len, int B, int64_t T, int64_t K, bool rect, int32_t* __restrict__ lengths,
    int32_t* __restrict__ col_lengths, int64_t* __restrict__ eta, int64_t* __restrict__ mu,
    int64_t* __restrict__ o, int64_t* __restrict__ items, int64_t* __restrict__ row_splits,
    int32_t* __restrict__ row_sample, int32_t* __restrict__ tile_sample) {
  constexpr int Q = 4;
  __shared__ int64_t buf[2][Q][kArgSamples];
  __shared__ int64_t s_eta[kArgSamples + 1], s_o[kArgSamples + 1];
  const int tid = threadIdx.x;
  const int64_t n = tid < B ? (int64_t)len.n[tid] : 0;
  const int64_t m = tid < B ? (int64_t)len.m[tid] : 0;
  const int64_t v[Q] = {n, m, n * m, items_of(n, m)};
  int cur = 0;
  for (int q = 0; q < Q; ++q) buf[cur][q][tid] = v[q];
  __syncthreads();
  for (int off = 1; off < kArgSamples; off <<= 1) {
    for (int q = 0; q < Q; ++q) {
      int64_t x = buf[cur][q][tid];
      if (tid >= off) x += buf[cur][q][tid - off];
      buf[cur ^ 1][q][tid] = x;
    }
    cur ^= 1;
    __syncthreads();
  }
  // exclusive offsets; entry B closes each array
  s_eta[tid + 1] = buf[cur][0][tid];
  s_o[tid + 1] = buf[cur][2][tid];
  if (tid == 0) s_eta[0] = s_o[0] = 0;
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < B) {
      lengths[tid] = (int32_t)n;
      eta[tid] = s_eta[tid];
      o[tid] = s_o[tid];
      items[tid] = tid == 0 ? 0 : buf[cur][3][tid - 1];
      if (rect) {
        col_lengths[tid] = (int32_t)m;
        mu[tid] = tid == 0 ? 0 : buf[cur][1][tid - 1];
      }
    }
    if (tid == 0) {  // entry B closes each array (B may equal kArgSamples)
      eta[B] = s_eta[B];
      o[B] = s_o[B];
      items[B] = B == 0 ? 0 : buf[cur][3][B - 1];
      if (rect) mu[B] = B == 0 ? 0 : buf[cur][1][B - 1];
    }
  }
  const int64_t g = (int64_t)blockIdx.x * kArgSamples + tid;
  if (g == 0) row_splits[T] = s_o[B];
  if (g < K) tile_sample[g] = find_segment(s_o, 0, B, g * kSampleIndexSpan);
  if (g < T) {
    const int i = find_segment(s_eta, 0, B, g);
    row_splits[g] = s_o[i] + (g - s_eta[i]) * (int64_t)len.m[i];
    row_sample[g] = i;
  }
}

__global__ __launch_bounds__(256) void k_decode(
    const int64_t* __restrict__ o, const int64_t* __restrict__ eta,
    const int64_t* __restrict__ mu, const int32_t* __restrict__ col_lengths, int B,
    int64_t cells, int32_t* __restrict__ sample, int32_t* __restrict__ row,
    int32_t* __restrict__ col) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= cells) return;
  const Cell x = decode_cell(o, eta, mu, col_lengths, B, t);
  sample[t] = x.i;
  row[t] = (int32_t)x.r;
  col[t] = (int32_t)x.c;
}

}  // namespace

hipError_t launch_partition(const nt_partition& p, int64_t* single_offsets, int64_t* col_offsets,
                            int64_t* pair_offsets, int64_t* item_offsets, int64_t* row_splits,
                            int32_t* row_sample, int32_t* tile_sample, hipStream_t stream) {
  hipLaunchKernelGGL(k_offsets_scan, dim3(1), dim3(kScanThreads), 0, stream, p.lengths,
                     p.col_lengths, p.B, single_offsets, col_offsets, pair_offsets, item_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t K = sample_index_entries(p.cells);
  const int64_t n = p.T > K ? p.T : K;
  const int64_t blocks = n > 0 ? (n + 255) / 256 : 1;
  hipLaunchKernelGGL(k_row_splits, dim3((unsigned)blocks), dim3(256), 0, stream, p.col_lengths,
                     single_offsets, pair_offsets, p.B, p.T, K, row_splits, row_sample,
                     tile_sample);
  return hipGetLastError();
}

hipError_t launch_partition_small(const int32_t* lengths_host, const int32_t* cols_host,
                                  const nt_partition& p, int32_t* lengths, int32_t* col_lengths,
                                  int64_t* single_offsets, int64_t* col_offsets,
                                  int64_t* pair_offsets, int64_t* item_offsets,
                                  int64_t* row_splits, int32_t* row_sample, int32_t* tile_sample,
                                  hipStream_t stream) {
  LengthsArg arg;
  for (int i = 0; i < kArgSamples; ++i) {
    arg.n[i] = i < p.B ? lengths_host[i] : 0;
    arg.m[i] = i < p.B ? cols_host[i] : 0;
  }
  const bool rect = col_lengths != lengths;
  const int64_t K = sample_index_entries(p.cells);
  const int64_t n = p.T > K ? p.T : K;
  const int64_t blocks = n > 0 ? (n + kArgSamples - 1) / kArgSamples : 1;
  hipLaunchKernelGGL(k_partition_small, dim3((unsigned)blocks), dim3(kArgSamples), 0, stream, arg,
                     p.B, p.T, K, rect, lengths, col_lengths, single_offsets, col_offsets,
                     pair_offsets, item_offsets, row_splits, row_sample, tile_sample);
  return hipGetLastError();
}

hipError_t launch_decode(const nt_partition& p, int32_t* sample, int32_t* row, int32_t* col,
                         hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  const int64_t blocks = (p.cells + 255) / 256;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)blocks), dim3(256), 0, stream, p.pair_offsets,
                     p.single_offsets, p.col_offsets, p.col_lengths, p.B, p.cells, sample, row,
                     col);
  return hipGetLastError();
}

}  // namespace nt
