// Boundary between two blocks of a chain (DanLing NestedTensor, Section 4.3
// "A larger pair application": blocks applied in sequence, the singles of one
// feeding the next). For one tile of 16 single rows it finishes block k and
// starts block k + 1:
//   s~ = s + m Wo^T                         (Equation 1, third line; rounded
//                                            to bf16 once and stored)
//   a  = s~ Wa'^T,  b = s~ Wb'^T            (Equation 1, first line's
//                                            projections of the next block)
// Every row is computed from that row alone, so results do not depend on the
// other samples of the batch. One launch replaces the output projection and
// the next block's a/b projection; s~ goes from registers to LDS and feeds
// the second product without a round trip through HBM. One workgroup of
// sixteen waves per row tile: the waves split the first product's column
// tiles, then each takes one 16-column tile of [a | b].
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kRows = 16;  // single rows per workgroup (one 16x16x32 MFMA row block)

__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sixteen waves. Lane (l16, g): l16 is a row of the A operand / a column of the
// B operand, g picks 8 of the 32 k of a step; accumulator element e is row
// 4 g + e, column l16 of the 16 x 16 result.
constexpr int kWaves = 16;

template <int CS, int CZ>
__global__ __launch_bounds__(64 * kWaves) void k_out_then_ab(
    const float* __restrict__ m, const bf16* __restrict__ Wo, const bf16* s_res, bf16* s_new,
    const bf16* __restrict__ Wa, const bf16* __restrict__ Wb, float* __restrict__ a,
    float* __restrict__ b, int64_t M) {
  constexpr int KS1 = CZ / 32;         // k-steps of s~ = s + m Wo^T
  constexpr int NT1 = CS / 16;         // 16-column tiles of s~
  constexpr int NJ1 = (NT1 + kWaves - 1) / kWaves;  // per wave, the last ones partly idle
  constexpr int KS2 = CS / 32;         // k-steps of a, b
  constexpr int LD = CS + 8;           // LDS row stride of s~ (bf16): 16 B of padding
  static_assert(CS % 32 == 0 && CZ % 32 == 0 && 2 * CZ / 16 <= kWaves, "tile counts");
  __shared__ __align__(16) bf16 st[kRows * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const bool row_ok = r0 + l16 < M;

  // ---- s~ = s + m Wo^T for columns 16 j .. 16 j + 15, j = wave + 16 i
  bf16x8 mh[KS1], ml[KS1];
  {
    const float* mrow = m + (row_ok ? r0 + l16 : 0) * CZ + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) {
      f32x4 x0 = f32x4{0.f, 0.f, 0.f, 0.f}, x1 = x0;
      if (row_ok) {
        x0 = *reinterpret_cast<const f32x4*>(mrow + 32 * ks);
        x1 = *reinterpret_cast<const f32x4*>(mrow + 32 * ks + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16 h0 = (bf16)x0[e], h1 = (bf16)x1[e];
        mh[ks][e] = h0;
        mh[ks][4 + e] = h1;
        ml[ks][e] = (bf16)(x0[e] - (float)h0);
        ml[ks][4 + e] = (bf16)(x1[e] - (float)h1);
      }
    }
  }
  bf16x8 wo[NJ1][KS1];
  float res[NJ1][4];
#pragma unroll
  for (int i = 0; i < NJ1; ++i) {
    const int j = wave + kWaves * i;
    const int col = 16 * (j < NT1 ? j : 0) + l16;
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks)
      wo[i][ks] = *reinterpret_cast<const bf16x8*>(Wo + (int64_t)col * CZ + 32 * ks + 8 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = r0 + 4 * g + e;
      res[i][e] = row < M ? (float)s_res[row * CS + col] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < NJ1; ++i) {
    const int j = wave + kWaves * i;
    if (j < NT1) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks) {
        acc = mma16(mh[ks], wo[i][ks], acc);
        acc = mma16(ml[ks], wo[i][ks], acc);
      }
      const int col = 16 * j + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) st[(4 * g + e) * LD + col] = (bf16)(acc[e] + res[i][e]);
    }
  }
  __syncthreads();

  // ---- s~ rows out (16-byte stores), by the first column group only
  constexpr int VPR = CS / 8;  // 16-byte vectors per row
  for (int v = tid; v < kRows * VPR; v += 64 * kWaves) {
    const int r = v / VPR, c = 8 * (v % VPR);
    if (r0 + r < M)
      *reinterpret_cast<bf16x8*>(s_new + (r0 + r) * CS + c) =
          *reinterpret_cast<const bf16x8*>(&st[r * LD + c]);
  }

  // ---- [a | b] = s~ [Wa | Wb]^T, wave t takes 16-column tile t of 2 CZ / 16
  bf16x8 sf[KS2];
#pragma unroll
  for (int ks = 0; ks < KS2; ++ks)
    sf[ks] = *reinterpret_cast<const bf16x8*>(&st[l16 * LD + 32 * ks + 8 * g]);
  if (wave < 2 * CZ / 16) {
    const int t = wave;
    const bool is_b = t >= CZ / 16;
    const int col = 16 * (is_b ? t - CZ / 16 : t) + l16;
    const bf16* wrow = (is_b ? Wb : Wa) + (int64_t)col * CS + 8 * g;
    bf16x8 wf[KS2];
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) wf[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) acc = mma16(sf[ks], wf[ks], acc);
    float* out = is_b ? b : a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = r0 + 4 * g + e;
      if (row < M) out[row * CZ + col] = acc[e];
    }
  }
}

template <int CS, int CZ>
hipError_t launch_t(const float* m, const void* Wo, const void* s_res, void* s_new,
                    const void* Wa, const void* Wb, float* a, float* b, int64_t M,
                    hipStream_t stream) {
  const int64_t tiles = (M + kRows - 1) / kRows;
  hipLaunchKernelGGL((k_out_then_ab<CS, CZ>), dim3((unsigned)tiles), dim3(64 * kWaves), 0, stream, m,
                     static_cast<const bf16*>(Wo), static_cast<const bf16*>(s_res),
                     static_cast<bf16*>(s_new), static_cast<const bf16*>(Wa),
                     static_cast<const bf16*>(Wb), a, b, M);
  return hipGetLastError();
}

}  // namespace

bool out_then_ab_supported(int c_s, int c_z, nt_dtype dtype) {
  if (dtype != NT_BF16) return false;
  return (c_s == 384 && c_z == 128) || (c_s == 64 && c_z == 64);
}

hipError_t launch_out_then_ab(const float* m, const void* Wo, const void* s_res, void* s_new,
                              const void* Wa, const void* Wb, float* a, float* b, int64_t M,
                              int c_s, int c_z, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (c_s == 384 && c_z == 128)
    return launch_t<384, 128>(m, Wo, s_res, s_new, Wa, Wb, a, b, M, stream);
  if (c_s == 64 && c_z == 64) return launch_t<64, 64>(m, Wo, s_res, s_new, Wa, Wb, a, b, M, stream);
  return hipErrorInvalidValue;
}

}  // namespace nt
