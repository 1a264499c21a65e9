// Element-wise and per-cell kernels of the SwiGLU transition's gradient
// (DanLing NestedTensor, Equation 1 second line with the paper's own update,
// P~ = P + h(LN_{C_p}(P)), h a SwiGLU; Appendix A.1). The products between
// them run on the library's matrix-core GEMMs; these kernels carry the parts
// that are not contractions:
//  * k_ln_rows: x = LN(z) in fp32, re-formed from the fp32 pair state (the
//    gradient's products read it unrounded: rounding x to bf16 here moves
//    the weight gradients by up to 2.5e-2 of their scale);
//  * k_swiglu_gate_bwd: from the gate and value pre-activations g, u and
//    the gated activation's adjoint g_A, the activation A = silu(g) u and the
//    adjoints g_u = g_A silu(g), g_g = g_A u silu'(g), silu' = s (1 + g (1 - s)),
//    s = sigmoid(g), all rounded to bf16 (operands of the next products);
//  * k_ln_backward: LN's adjoint added to G (in place), and per-workgroup
//    partial sums of dgamma = sum g_x xhat and dbeta = sum g_x, summed in a
//    fixed order afterwards (deterministic);
// A cell's c_z features are spread over c_z / 4 lanes (16-byte loads), so
// one wave holds 256 / c_z cells at a time.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kLnThreads = 256;
constexpr int kLnMaxBlocks = 1024;

// Sum over the L lanes of one cell (aligned groups of L within the wave).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <int CZ>
__global__ __launch_bounds__(kLnThreads) void k_ln_rows(const float* __restrict__ z,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta,
                                                        float* __restrict__ x, int64_t rows,
                                                        float eps) {
  constexpr int L = CZ / 4, PER = kLnThreads / L;
  const int lane = threadIdx.x % L, slot = threadIdx.x / L;
  const f32x4 gm = *reinterpret_cast<const f32x4*>(gamma + 4 * lane);
  const f32x4 bt = *reinterpret_cast<const f32x4*>(beta + 4 * lane);
  for (int64_t r = (int64_t)blockIdx.x * PER + slot; r < rows; r += (int64_t)gridDim.x * PER) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(z + r * CZ + 4 * lane);
    const float mu = group_sum<L>(v[0] + v[1] + v[2] + v[3]) * (1.f / CZ);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) q += (v[e] - mu) * (v[e] - mu);
    const float rstd = 1.f / sqrtf(group_sum<L>(q) * (1.f / CZ) + eps);
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (v[e] - mu) * rstd * gm[e] + bt[e];
    *reinterpret_cast<f32x4*>(x + r * CZ + 4 * lane) = o;
  }
}

__global__ __launch_bounds__(kLnThreads) void k_swiglu_gate_bwd(
    const f32x4* __restrict__ g, const f32x4* __restrict__ u, const f32x4* __restrict__ gA,
    bf16* __restrict__ A, bf16* __restrict__ gu, bf16* __restrict__ gg, int64_t n4) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  for (int64_t i = (int64_t)blockIdx.x * kLnThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kLnThreads) {
    const f32x4 vg = g[i], vu = u[i], va = gA[i];
    bf16x4 oA, ou, og;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = 1.f / (1.f + __expf(-vg[e]));
      const float silu = vg[e] * s;
      oA[e] = (bf16)(silu * vu[e]);
      ou[e] = (bf16)(va[e] * silu);
      og[e] = (bf16)(va[e] * vu[e] * s * (1.f + vg[e] * (1.f - s)));
    }
    reinterpret_cast<bf16x4*>(A)[i] = oA;
    reinterpret_cast<bf16x4*>(gu)[i] = ou;
    reinterpret_cast<bf16x4*>(gg)[i] = og;
  }
}

// G += LN's adjoint of g_x, row by row; part_gamma / part_beta [gridDim.x,
// CZ] receive this workgroup's sums of g_x xhat and g_x over its rows.
template <int CZ>
__global__ __launch_bounds__(kLnThreads) void k_ln_backward(
    const float* __restrict__ z, const float* __restrict__ gamma, const float* __restrict__ gx,
    float* G, float* __restrict__ part_gamma, float* __restrict__ part_beta, int64_t rows,
    float eps) {
  constexpr int L = CZ / 4, PER = kLnThreads / L;
  __shared__ f32x4 acc_g[kLnThreads], acc_b[kLnThreads];
  const int lane = threadIdx.x % L, slot = threadIdx.x / L;
  const f32x4 gm = *reinterpret_cast<const f32x4*>(gamma + 4 * lane);
  f32x4 dg = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
  for (int64_t r = (int64_t)blockIdx.x * PER + slot; r < rows; r += (int64_t)gridDim.x * PER) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(z + r * CZ + 4 * lane);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(gx + r * CZ + 4 * lane);
    const float mu = group_sum<L>(v[0] + v[1] + v[2] + v[3]) * (1.f / CZ);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) q += (v[e] - mu) * (v[e] - mu);
    const float rstd = 1.f / sqrtf(group_sum<L>(q) * (1.f / CZ) + eps);
    f32x4 xh, gh;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xh[e] = (v[e] - mu) * rstd;
      gh[e] = gv[e] * gm[e];
      s1 += gh[e];
      s2 += gh[e] * xh[e];
      dg[e] += gv[e] * xh[e];
      db[e] += gv[e];
    }
    const float m1 = group_sum<L>(s1) * (1.f / CZ), m2 = group_sum<L>(s2) * (1.f / CZ);
    f32x4* gp = reinterpret_cast<f32x4*>(G + r * CZ + 4 * lane);
    f32x4 o = *gp;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += rstd * (gh[e] - m1 - xh[e] * m2);
    *gp = o;
  }
  acc_g[threadIdx.x] = dg;
  acc_b[threadIdx.x] = db;
  __syncthreads();
  if (threadIdx.x < L) {  // the PER slots of feature group `lane`, in slot order
    f32x4 sg = acc_g[threadIdx.x], sb = acc_b[threadIdx.x];
    for (int k = 1; k < PER; ++k) {
      const f32x4 a = acc_g[threadIdx.x + k * L], b = acc_b[threadIdx.x + k * L];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sg[e] += a[e];
        sb[e] += b[e];
      }
    }
    *reinterpret_cast<f32x4*>(part_gamma + (int64_t)blockIdx.x * CZ + 4 * threadIdx.x) = sg;
    *reinterpret_cast<f32x4*>(part_beta + (int64_t)blockIdx.x * CZ + 4 * threadIdx.x) = sb;
  }
}

int64_t grid_for(int64_t items, int64_t per_block) {
  const int64_t g = (items + per_block - 1) / per_block;
  return g < 1 ? 1 : (g > 65536 ? 65536 : g);
}

}  // namespace

int ln_backward_blocks(int64_t rows, int c_z) {
  const int64_t per = kLnThreads / (c_z / 4);
  const int64_t g = (rows + per - 1) / per;
  return (int)(g < 1 ? 1 : (g > kLnMaxBlocks ? kLnMaxBlocks : g));
}

hipError_t launch_ln_rows(const float* z, const float* gamma, const float* beta, float* x,
                          int64_t rows, int c_z, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t per = kLnThreads / (c_z / 4);
  const dim3 grid((unsigned)grid_for(rows, per));
  if (c_z == 128)
    hipLaunchKernelGGL(k_ln_rows<128>, grid, dim3(kLnThreads), 0, s, z, gamma, beta, x, rows,
                       eps);
  else
    hipLaunchKernelGGL(k_ln_rows<64>, grid, dim3(kLnThreads), 0, s, z, gamma, beta, x, rows,
                       eps);
  return hipGetLastError();
}

hipError_t launch_swiglu_gate_bwd(const float* g, const float* u, const float* gA, void* A,
                                  void* gu, void* gg, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t n4 = n / 4;  // n = rows * hidden, hidden a multiple of 32
  hipLaunchKernelGGL(k_swiglu_gate_bwd, dim3((unsigned)grid_for(n4, kLnThreads)),
                     dim3(kLnThreads), 0, s, reinterpret_cast<const f32x4*>(g),
                     reinterpret_cast<const f32x4*>(u), reinterpret_cast<const f32x4*>(gA),
                     static_cast<bf16*>(A), static_cast<bf16*>(gu), static_cast<bf16*>(gg), n4);
  return hipGetLastError();
}

hipError_t launch_ln_backward(const float* z, const float* gamma, const float* gx, float* G,
                              float* part_gamma, float* part_beta, float* dgamma, float* dbeta,
                              int64_t rows, int c_z, float eps, hipStream_t s) {
  const int blocks = ln_backward_blocks(rows, c_z);
  if (rows > 0) {
    if (c_z == 128)
      hipLaunchKernelGGL(k_ln_backward<128>, dim3(blocks), dim3(kLnThreads), 0, s, z, gamma, gx,
                         G, part_gamma, part_beta, rows, eps);
    else
      hipLaunchKernelGGL(k_ln_backward<64>, dim3(blocks), dim3(kLnThreads), 0, s, z, gamma, gx,
                         G, part_gamma, part_beta, rows, eps);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int S = rows > 0 ? blocks : 0;
  const hipError_t e = launch_sum_splits(part_gamma, dgamma, S, c_z, s);
  return e != hipSuccess ? e : launch_sum_splits(part_beta, dbeta, S, c_z, s);
}

}  // namespace nt
