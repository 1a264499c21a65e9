// Weight gradients of the pair transition: contractions over the packed
// cells (DanLing NestedTensor, Equation 1's second line differentiated; the
// cells are Section 3.3's valid positions, so the sum runs over sum N_i M_i
// rows and no padding):
//   C[m, n] = sum_k A[k, m] B[k, n],   A [K, M], B [K, N] bf16, row-major,
// used for dW1 = g_H^T z and dW2 = G^T H with K = cells.
//
// Split-K on the matrix cores: workgroup (tile, slice) multiplies a 128 x 128
// tile of C over one slice of K and writes an fp32 partial tile; the slices
// are then added in order (k_sum_splits in nt_backward.hip), so the result is
// deterministic. Both operands arrive cell-major (K outermost), while a
// 32x32x16 MFMA operand wants 8 consecutive k per lane, so each thread loads
// an 8 (k) x 8 (m) block with eight 16-byte row loads, transposes it in
// registers and writes eight 16-byte k-runs into LDS ([m][k] layout); the
// fragment reads are then plain 16-byte LDS reads.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kWgThreads = 256;
constexpr int kWgTile = 128;   // C tile edge
constexpr int kWgK = 64;       // k per step
constexpr int kWgPitch = kWgK + 8;  // LDS row pitch in elements (144 bytes)

__device__ __forceinline__ f32x16 wg_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// blockIdx.x: tile of C (tm, tn) = (x % tiles_m, x / tiles_m); blockIdx.y:
// the K slice [y * kchunk, min(K, (y + 1) * kchunk)), kchunk a multiple of
// kWgK. Threads 0..127 stage A, 128..255 stage B: thread (bk, bm) of its half
// moves the 8 x 8 block at rows 8 bk.., columns 8 bm.. of the step's 64 x 128
// operand tile. Waves own 64 x 64 quadrants of the C tile.
__global__ __launch_bounds__(kWgThreads) void k_wgrad(const bf16* __restrict__ A,
                                                      const bf16* __restrict__ B,
                                                      float* __restrict__ part, int64_t K,
                                                      int M, int N, int64_t kchunk) {
  __shared__ bf16x8 lds[2][kWgTile * kWgPitch / 8];  // [operand][m * pitch + k] in 8s
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_m = M / kWgTile;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t kb = (int64_t)blockIdx.y * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;

  // staging role
  const int op = tid >> 7;              // 0: A, 1: B
  const int st = tid & 127;
  const int bm = st & 15, bk = st >> 4;  // 16 column blocks x 8 row blocks
  const bf16* src = op == 0 ? A + (int64_t)tm * kWgTile + 8 * bm
                            : B + (int64_t)tn * kWgTile + 8 * bm;
  const int ld = op == 0 ? M : N;
  bf16* dst = reinterpret_cast<bf16*>(lds[op]);

  const int wm = wave & 1, wn = wave >> 1;  // quadrant of the C tile
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  for (int64_t k0 = kb; k0 < ke; k0 += kWgK) {
    bf16x8 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t k = k0 + 8 * bk + i;
      rows[i] = k < ke ? *reinterpret_cast<const bf16x8*>(src + k * ld) : bf16x8{};
    }
    __syncthreads();  // the previous step's fragment reads are done
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x8 col;
#pragma unroll
      for (int i = 0; i < 8; ++i) col[i] = rows[i][e];
      *reinterpret_cast<bf16x8*>(dst + (8 * bm + e) * kWgPitch + 8 * bk) = col;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kWgK / 16; ++s) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = 64 * wm + 32 * i + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(lds[0]) +
                                                 m * kWgPitch + 16 * s + 8 * h);
        const int n = 64 * wn + 32 * i + l32;
        bfr[i] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(lds[1]) +
                                                  n * kWgPitch + 16 * s + 8 * h);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = wg_mfma(af[i], bfr[j], acc[i][j]);
    }
  }
  // partial tile: element r of block (i, j) is row 8 (r / 4) + 4 h + r % 4,
  // column l32 of that 32 x 32 block
  float* out = part + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tm * kWgTile + 64 * wm + 32 * i + 8 * (r / 4) + 4 * h + r % 4;
        const int n = tn * kWgTile + 64 * wn + 32 * j + l32;
        out[(int64_t)m * N + n] = acc[i][j][r];
      }
}

}  // namespace

int wgrad_splits(int64_t K, int M, int N) {
  const int64_t tiles = (int64_t)(M / kWgTile) * (N / kWgTile);
  int64_t S = (512 + tiles - 1) / tiles;  // about 512 workgroups (two per CU of a 256-CU part)
  const int64_t kmax = (K + 4 * kWgK - 1) / (4 * kWgK);  // at least four steps a slice
  if (S > kmax) S = kmax;
  return (int)(S < 1 ? 1 : (S > 512 ? 512 : S));
}

bool wgrad_supported(int M, int N) { return M % kWgTile == 0 && N % kWgTile == 0; }

hipError_t launch_wgrad(const void* A, const void* B, float* C, float* part, int64_t K, int M,
                        int N, int splits, hipStream_t stream) {
  if (K == 0) return launch_sum_splits(part, C, 0, (int64_t)M * N, stream);
  int64_t kchunk = (K + splits - 1) / splits;
  kchunk = (kchunk + kWgK - 1) / kWgK * kWgK;
  const int64_t S = (K + kchunk - 1) / kchunk;
  const dim3 grid((unsigned)((M / kWgTile) * (N / kWgTile)), (unsigned)S);
  hipLaunchKernelGGL(k_wgrad, grid, dim3(kWgThreads), 0, stream, static_cast<const bf16*>(A),
                     static_cast<const bf16*>(B), part, K, M, N, kchunk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_splits(part, C, (int)S, (int64_t)M * N, stream);
}

}  // namespace nt
