// Partition construction for square pairs (DanLing NestedTensor, Section 3.1
// "Numerical storage" / Equation 2, Figure 2, Appendix A "Structural
// invariants") and the materialised cell decode used as a test hook.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kScanThreads = 256;

// One workgroup scans all B lengths in chunks of 256, carrying the running
// totals: eta_i = sum_{k<i} N_k, o_i = sum_{k<i} N_k^2 and the column-mean
// item offsets. Each chunk is an inclusive Hillis-Steele scan in LDS.
__global__ __launch_bounds__(kScanThreads) void k_offsets_scan(
    const int32_t* __restrict__ lengths, int B, int64_t* __restrict__ eta,
    int64_t* __restrict__ o, int64_t* __restrict__ items) {
  __shared__ int64_t buf[2][3][kScanThreads];
  __shared__ int64_t carry[3];
  const int tid = threadIdx.x;
  if (tid == 0) carry[0] = carry[1] = carry[2] = 0;
  __syncthreads();
  for (int base = 0; base < B; base += kScanThreads) {
    const int idx = base + tid;
    const int64_t n = idx < B ? (int64_t)lengths[idx] : 0;
    int64_t v[3] = {n, n * n, items_of(n)};
    int cur = 0;
    for (int q = 0; q < 3; ++q) buf[cur][q][tid] = v[q];
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
      for (int q = 0; q < 3; ++q) {
        int64_t x = buf[cur][q][tid];
        if (tid >= off) x += buf[cur][q][tid - off];
        buf[cur ^ 1][q][tid] = x;
      }
      cur ^= 1;
      __syncthreads();
    }
    if (idx < B) {
      eta[idx] = carry[0] + buf[cur][0][tid] - v[0];
      o[idx] = carry[1] + buf[cur][1][tid] - v[1];
      items[idx] = carry[2] + buf[cur][2][tid] - v[2];
    }
    __syncthreads();
    if (tid == 0) {
      for (int q = 0; q < 3; ++q) carry[q] += buf[cur][q][kScanThreads - 1];
    }
    __syncthreads();
  }
  if (tid == 0) {
    eta[B] = carry[0];
    o[B] = carry[1];
    items[B] = carry[2];
  }
}

// Second-level row splits: pair row g = eta_i + r starts at o_i + r * N_i
// (Equation 3 at column 0); row_splits[T] closes with the cell total.
__global__ __launch_bounds__(256) void k_row_splits(
    const int32_t* __restrict__ lengths, const int64_t* __restrict__ eta,
    const int64_t* __restrict__ o, int B, int64_t T, int64_t* __restrict__ row_splits,
    int32_t* __restrict__ row_sample) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g == 0) row_splits[T] = o[B];
  if (g >= T) return;
  const int i = find_segment(eta, 0, B, g);
  const int64_t r = g - eta[i];
  row_splits[g] = o[i] + r * (int64_t)lengths[i];
  row_sample[g] = i;
}

__global__ __launch_bounds__(256) void k_decode(
    const int64_t* __restrict__ o, const int64_t* __restrict__ eta,
    const int32_t* __restrict__ lengths, int B, int64_t cells, int32_t* __restrict__ sample,
    int32_t* __restrict__ row, int32_t* __restrict__ col) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= cells) return;
  const Cell x = decode_cell(o, eta, lengths, B, t);
  sample[t] = x.i;
  row[t] = (int32_t)x.r;
  col[t] = (int32_t)x.c;
}

}  // namespace

hipError_t launch_partition(const nt_partition& p, int64_t* single_offsets, int64_t* pair_offsets,
                            int64_t* item_offsets, int64_t* row_splits, int32_t* row_sample,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_offsets_scan, dim3(1), dim3(kScanThreads), 0, stream, p.lengths, p.B,
                     single_offsets, pair_offsets, item_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = p.T > 0 ? (p.T + 255) / 256 : 1;
  hipLaunchKernelGGL(k_row_splits, dim3((unsigned)blocks), dim3(256), 0, stream, p.lengths,
                     single_offsets, pair_offsets, p.B, p.T, row_splits, row_sample);
  return hipGetLastError();
}

hipError_t launch_decode(const nt_partition& p, int32_t* sample, int32_t* row, int32_t* col,
                         hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  const int64_t blocks = (p.cells + 255) / 256;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)blocks), dim3(256), 0, stream, p.pair_offsets,
                     p.single_offsets, p.lengths, p.B, p.cells, sample, row, col);
  return hipGetLastError();
}

}  // namespace nt
