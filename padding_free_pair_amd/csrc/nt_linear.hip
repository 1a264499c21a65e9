// Projections on packed single rows (DanLing NestedTensor, Section 3.3 "Dense
// work across valid positions": V' = V W^T, here without bias):
//   C[M, N] = R[M, N] + A[M, K] W[N, K]^T      (R optional).
// These are the block's small GEMMs (a, b and the output projection), a few
// hundred MFLOP each; one wave computes a 32 x 32 tile straight from L2.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

// A, W: storage types; C, R: output type. BF16MMA: A and W are bf16 and K is a
// multiple of 32 (v_mfma_f32_16x16x32_bf16); otherwise v_mfma_f32_16x16x4_f32
// on fp32 values (bf16 inputs are widened exactly).
template <typename TA, typename TW, typename TO, bool BF16MMA>
__global__ __launch_bounds__(64) void k_linear(const TA* __restrict__ A, const TW* __restrict__ W,
                                               const TO* R, TO* C, int64_t M, int N, int K) {
  const int lane = threadIdx.x;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int n0 = blockIdx.y * 32;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const TA* arow[2];
  const TW* wrow[2];
  bool aok[2], wok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t row = m0 + 16 * i + l16;
    aok[i] = row < M;
    arow[i] = A + (aok[i] ? row : 0) * K;
    const int col = n0 + 16 * i + l16;
    wok[i] = col < N;
    wrow[i] = W + (int64_t)(wok[i] ? col : 0) * K;
  }

  if constexpr (BF16MMA) {
    for (int k0 = 0; k0 < K; k0 += 32) {
      bf16x8 af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = aok[i] ? *reinterpret_cast<const bf16x8*>(arow[i] + k0 + 8 * g) : bf16x8{};
        wf[i] = wok[i] ? *reinterpret_cast<const bf16x8*>(wrow[i] + k0 + 8 * g) : bf16x8{};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
    }
  } else {
    // 16 k per step: lane group g holds k0 + 4g .. 4g+3 of its row, and the
    // four sub-steps s pair A[., k0 + 4g + s] with W[., k0 + 4g + s].
    for (int k0 = 0; k0 < K; k0 += 16) {
      const int kk = k0 + 4 * g;
      const bool kin = kk < K;  // K is a multiple of 8, so groups are whole
      float av[2][4], wv[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          av[i][s] = (aok[i] && kin) ? to_f32(arow[i][kk + s]) : 0.f;
          wv[i][s] = (wok[i] && kin) ? to_f32(wrow[i][kk + s]) : 0.f;
        }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][s], wv[j][s], acc[i][j], 0, 0, 0);
    }
  }

  // result lane layout: rows 4g + e, column l16 of each 16x16 block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + 16 * j + l16;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + 16 * i + 4 * g + e;
        if (row >= M) continue;
        float v = acc[i][j][e];
        if (R) v += to_f32(R[row * N + col]);
        C[row * N + col] = from_f32<TO>(v);
      }
    }
}

// bf16-weight GEMM for the block's projections. A workgroup of four waves
// owns a 32 x 32 output tile and splits K between its waves (wave w takes
// k-steps w, w + 4, ...), so each wave's fragment loads are all in flight at
// once; the four partial tiles are summed through LDS. An fp32 left operand is
// split into bf16 hi + lo parts (two MFMAs), which keeps ~16 significant bits.
// blockIdx.z selects one of two (W, C) pairs, so the a and b projections of a
// block share one launch.
template <typename TA, typename TO>
__global__ __launch_bounds__(256) void k_gemm_bf16w(const TA* __restrict__ A,
                                                    const bf16* __restrict__ W0,
                                                    const bf16* __restrict__ W1, const TO* R,
                                                    TO* C0, TO* C1, int64_t M, int N, int K) {
  constexpr bool SPLIT = sizeof(TA) == 4;
  constexpr int UNROLL = 4;  // k-steps of one wave issued together
  __shared__ float part[4][32 * 33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int n0 = blockIdx.y * 32;
  const bf16* W = blockIdx.z ? W1 : W0;
  TO* C = blockIdx.z ? C1 : C0;

  const TA* arow[2];
  const bf16* wrow[2];
  bool aok[2], wok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t row = m0 + 16 * i + l16;
    aok[i] = row < M;
    arow[i] = A + (aok[i] ? row : 0) * K + 8 * g;
    const int col = n0 + 16 * i + l16;
    wok[i] = col < N;
    wrow[i] = W + (int64_t)(wok[i] ? col : 0) * K + 8 * g;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = K / 32;
  for (int ks0 = wave; ks0 < ksteps; ks0 += 4 * UNROLL) {
    bf16x8 af[UNROLL][2], al[UNROLL][2], wf[UNROLL][2];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int ks = ks0 + 4 * u;
      const bool kin = ks < ksteps;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        wf[u][i] = (kin && wok[i]) ? *reinterpret_cast<const bf16x8*>(wrow[i] + 32 * ks)
                                   : bf16x8{};
        if constexpr (SPLIT) {
          f32x4 x0 = f32x4{0.f, 0.f, 0.f, 0.f}, x1 = x0;
          if (kin && aok[i]) {
            x0 = *reinterpret_cast<const f32x4*>(arow[i] + 32 * ks);
            x1 = *reinterpret_cast<const f32x4*>(arow[i] + 32 * ks + 4);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16 h0 = (bf16)x0[e], h1 = (bf16)x1[e];
            af[u][i][e] = h0;
            af[u][i][4 + e] = h1;
            al[u][i][e] = (bf16)(x0[e] - (float)h0);
            al[u][i][4 + e] = (bf16)(x1[e] - (float)h1);
          }
        } else {
          af[u][i] = (kin && aok[i]) ? *reinterpret_cast<const bf16x8*>(arow[i] + 32 * ks)
                                     : bf16x8{};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][i], wf[u][j], acc[i][j], 0, 0, 0);
          if constexpr (SPLIT)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u][i], wf[u][j], acc[i][j], 0, 0, 0);
        }
  }
  // partial tiles -> LDS (row 16 i + 4 g + e, column 16 j + l16), then sum
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) part[wave][(16 * i + 4 * g + e) * 33 + 16 * j + l16] = acc[i][j][e];
  __syncthreads();
  const int r = tid >> 3, c0 = (tid & 7) * 4;
  const int64_t row = m0 + r;
  if (row < M) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = n0 + c0 + q;
      if (col >= N) continue;
      float v = part[0][r * 33 + c0 + q] + part[1][r * 33 + c0 + q] +
                part[2][r * 33 + c0 + q] + part[3][r * 33 + c0 + q];
      if (R) v += to_f32(R[row * N + col]);
      C[row * N + col] = from_f32<TO>(v);
    }
  }
}

template <typename TA, typename TW, typename TO, bool BF16MMA>
hipError_t launch_t(const void* A, const void* W, const void* R, void* C, int64_t M, int N, int K,
                    hipStream_t stream) {
  const dim3 grid((unsigned)((M + 31) / 32), (unsigned)((N + 31) / 32));
  hipLaunchKernelGGL((k_linear<TA, TW, TO, BF16MMA>), grid, dim3(64), 0, stream,
                     static_cast<const TA*>(A), static_cast<const TW*>(W),
                     static_cast<const TO*>(R), static_cast<TO*>(C), M, N, K);
  return hipGetLastError();
}

template <typename TA, typename TO>
hipError_t launch_gemm(const void* A, const void* W0, const void* W1, const void* R, void* C0,
                       void* C1, int64_t M, int N, int K, hipStream_t stream) {
  const dim3 grid((unsigned)((M + 31) / 32), (unsigned)((N + 31) / 32), W1 ? 2u : 1u);
  hipLaunchKernelGGL((k_gemm_bf16w<TA, TO>), grid, dim3(256), 0, stream,
                     static_cast<const TA*>(A), static_cast<const bf16*>(W0),
                     static_cast<const bf16*>(W1), static_cast<const TO*>(R),
                     static_cast<TO*>(C0), static_cast<TO*>(C1), M, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear2(const void* A, nt_dtype a_dtype, const void* W0, const void* W1,
                          void* C0, void* C1, int64_t M, int N, int K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (a_dtype == NT_BF16 && K % 32 == 0)
    return launch_gemm<bf16, float>(A, W0, W1, nullptr, C0, C1, M, N, K, stream);
  hipError_t e = launch_linear(A, a_dtype, W0, a_dtype, nullptr, C0, NT_F32, M, N, K, stream);
  if (e != hipSuccess) return e;
  return launch_linear(A, a_dtype, W1, a_dtype, nullptr, C1, NT_F32, M, N, K, stream);
}

hipError_t launch_linear(const void* A, nt_dtype a_dtype, const void* W, nt_dtype w_dtype,
                         const void* R, void* C, nt_dtype c_dtype, int64_t M, int N, int K,
                         hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (w_dtype == NT_BF16 && K % 32 == 0) {
    if (a_dtype == NT_BF16 && c_dtype == NT_F32)
      return launch_gemm<bf16, float>(A, W, nullptr, R, C, nullptr, M, N, K, stream);
    if (a_dtype == NT_F32 && c_dtype == NT_BF16)
      return launch_gemm<float, bf16>(A, W, nullptr, R, C, nullptr, M, N, K, stream);
    if (a_dtype == NT_F32 && c_dtype == NT_F32)
      return launch_gemm<float, float>(A, W, nullptr, R, C, nullptr, M, N, K, stream);
  }
  if (a_dtype == NT_BF16 && w_dtype == NT_BF16 && c_dtype == NT_F32) {
    if (K % 32 == 0) return launch_t<bf16, bf16, float, true>(A, W, R, C, M, N, K, stream);
    return launch_t<bf16, bf16, float, false>(A, W, R, C, M, N, K, stream);
  }
  if (a_dtype == NT_F32 && w_dtype == NT_BF16 && c_dtype == NT_BF16)
    return launch_t<float, bf16, bf16, false>(A, W, R, C, M, N, K, stream);
  if (a_dtype == NT_F32 && w_dtype == NT_BF16 && c_dtype == NT_F32)
    return launch_t<float, bf16, float, false>(A, W, R, C, M, N, K, stream);
  if (a_dtype == NT_F32 && w_dtype == NT_F32 && c_dtype == NT_F32)
    return launch_t<float, float, float, false>(A, W, R, C, M, N, K, stream);
  return hipErrorInvalidValue;  // combination not used by the block
}

}  // namespace nt
