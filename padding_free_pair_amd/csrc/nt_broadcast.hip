// Pair broadcast (DanLing NestedTensor, Equation 1 first line; Section 3.2
// "Creating axes through broadcasting"):
//   z[o_i + r M_i + c, :] = a[eta_i + r, :] + b[mu_i + c, :]
// (M_i = N_i and mu = eta for square pairs).
// HBM-write bound: each cell writes c_z elements, a and b are L2 resident.
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

template <typename TI, typename T>
hipError_t launch_t(const nt_partition& p, const void* a, const void* b, void* z, int c_z,
                    hipStream_t stream) {
  const int G = c_z / Vec16<T>::N;  // <= 256 for c_z <= kMaxCz
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
