// Gradient of the residual pair transition on the matrix cores (DanLing
// NestedTensor, Equation 1's second line differentiated; Section 4 measures
// forward, loss and backward). For an incoming G = dL/dz' per cell:
//   pre = z W1^T,  H = relu(pre),  g_H = (G W2) * [pre > 0],
//   g_z = G + g_H W1,
// and bf16(G) (plus, on request, H and g_H) is written for the weight
// gradients dW1 = g_H^T z and dW2 = G^T H, contractions over all cells in
// nt_wgrad.hip (k_wgrad_rc recomputes H and g_H from z and bf16(G)).
//
// Persistent kernel, bf16, c_z = 128, hidden a multiple of 32. A workgroup
// of eight waves (two per SIMD) takes 256 cells at a time, 32 per wave (one
// 32-cell column block, kBwCB).
// Per 32-unit hidden chunk j, three products run on v_mfma_f32_32x32x16_bf16
// with the cells as the N dimension:
//   pre^T (32 x cells) = W1[j]   . z^T        (k = features)
//   gh^T  (32 x cells) = W2T[j]  . bf16(G)^T  (k = features)
//   g_z^T (c_z x cells) += W1T[:, j] . g_H^T  (k = the chunk's units)
// The chunk's 24 KiB of weight fragments are double-buffered through LDS:
// the loads of chunk j + 2 are issued at the start of chunk j, and chunk
// j + 1 is written after chunk j's products. Result rows of the first two products are permuted
// (bits 2 and 3 of the row swapped) so that lane group h holds units
// 16 s + 8 h + 0..7 in elements 8 s .. 8 s + 7: the mask, the bf16 pack of
// g_H and the third product's operand are lane-local, and the third
// product's rows (features) use the same permutation, so its accumulator
// matches the lane's slice of G and g_z (features 16 t + 8 h + 0..7).
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kBwCB = 1;                          // 32-cell blocks per wave
constexpr int kBwWaves = 8;
constexpr int kBwThreads = kBwWaves * 64;
constexpr int kBwTileCells = kBwWaves * 32 * kBwCB;
// s_waitcnt immediate (gfx9 encoding): every vector-memory load has completed
constexpr int kBwWaitVm0 = 0x0F70;

__device__ __forceinline__ f32x16 bw_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Result row rho of a 32x32 product <-> unit (or feature) within its block of
// 32: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int bw_p32(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Where G comes from: read from memory, or formed from the column mean's
// adjoint, G[cell] = g_m[row] / M_i (+ g_in[cell]), with the cell decoded on
// the fly (Eq. 3 inverted from the tile's first sample). The division is
// done once per row beforehand (k_mean_rows), so `g_m` here holds the
// quotients.
struct MeanAdjoint {
  const float* g_m;             // [T, c_z], g_m[row] / M_i
  const float* g_in;            // [cells, c_z] or null
  const int64_t* pair_offsets;
  const int64_t* single_offsets;
  const int32_t* col_lengths;   // M_i, the divisor
  const int32_t* tile_sample;   // sample of cell 256 k
};

// WRITE_H: also store H and g_H per cell (for contractions that read them);
// without it the weight gradients are recomputed from z and bf16(G).
// FROM_MEAN: G is formed from `ma` instead of read.
template <int CZ, int HID, bool WRITE_H, bool FROM_MEAN>
__global__ __launch_bounds__(kBwThreads, 2) void k_transition_bwd(
    const bf16* __restrict__ z, const float* G, MeanAdjoint ma, const bf16* __restrict__ W1,
    const bf16* __restrict__ W2T, const bf16* __restrict__ W1T, float* g_z,
    bf16* __restrict__ H, bf16* __restrict__ GH, bf16* __restrict__ Gb, int64_t cells,
    int64_t ntiles) {
  constexpr int KT = CZ / 16;    // k-steps of the first two products
  constexpr int FB = CZ / 32;    // feature blocks of the third
  constexpr int NCH = HID / 32;  // hidden chunks
  constexpr int CB = kBwCB;
  // one chunk's fragments: W1 (KT x 64 lanes), W2T (KT x 64), W1T (FB x 2 x 64)
  constexpr int F1 = KT * 64, F2 = KT * 64, F3 = FB * 2 * 64;
  constexpr int FRAGS = F1 + F2 + F3;                 // 16-byte pieces
  constexpr int PER = FRAGS / kBwThreads;             // pieces per thread
  static_assert(FRAGS % kBwThreads == 0, "chunk staging splits evenly");
  static_assert(FB * 2 == KT, "shape");

  __shared__ bf16x8 wbuf[2][FRAGS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  // Slot p of a chunk's fragment area and the 16 bytes of the weights it
  // holds; thread tid fills slots tid, tid + threads, ... (consecutive lanes
  // write consecutive LDS slots). W1 / W2T fragment t, lane L: row
  // 32 j + p32(L % 32), features 16 t + 8 (L / 32) ..; W1T fragment
  // 2 fb + s, lane L: row 32 fb + p32(L % 32), units 32 j + 16 s + 8 (L / 32) ..
  auto piece_src = [&](int j, int p) -> const bf16* {
    const int L = p & 63, r = bw_p32(L & 31), hh = L >> 5;
    if (p < F1 + F2) {
      const bf16* M = p < F1 ? W1 : W2T;
      const int t = (p < F1 ? p : p - F1) >> 6;
      return M + (int64_t)(32 * j + r) * CZ + 16 * t + 8 * hh;
    }
    const int i = (p - F1 - F2) >> 6, fb = i >> 1, sh = i & 1;
    return W1T + (int64_t)(32 * fb + r) * HID + 32 * j + 16 * sh + 8 * hh;
  };
  auto piece_slot = [&](int p) -> int { return p; };

  // Two register sets of staged pieces: the loads of chunk j + 2 are issued
  // at the start of chunk j, and chunk j + 1 (loaded a chunk earlier) is
  // written to LDS at its end, so each write waits only for loads that had a
  // whole chunk of products to land. The chunk loop is unrolled by two so
  // that the sets are fixed registers.
  bf16x8 stA[PER], stB[PER];
  auto load_chunk = [&](int j, bf16x8 (&st)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      st[k] = *reinterpret_cast<const bf16x8*>(piece_src(j % NCH, tid + k * kBwThreads));
  };
  auto store_chunk = [&](int buf, const bf16x8 (&st)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k) wbuf[buf][piece_slot(tid + k * kBwThreads)] = st[k];
  };
  static_assert(NCH % 2 == 0, "the chunk loop is unrolled by two");

  load_chunk(0, stA);
  store_chunk(0, stA);
  load_chunk(1, stB);
  __syncthreads();

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t cell0 = tile * kBwTileCells + wave * 32 * CB;
    // z and G of this wave's cells: lane (l32, h) of block cb holds features
    // 16 t + 8 h + 0..7 of cell cell0 + 32 cb + l32
    bf16x8 zb[CB][KT], gb[CB][KT];
    f32x16 y[CB][FB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      int64_t c = cell0 + 32 * cb + l32;
      c = c < cells ? c : cells - 1;
      const float* grow = nullptr;  // g_m[row] / M_i for the cell's row (FROM_MEAN)
      if constexpr (FROM_MEAN) {
        int i = ma.tile_sample[tile];  // tiles are 256 cells, the index's span
        while (ma.pair_offsets[i + 1] <= c) ++i;
        const int64_t m = ma.col_lengths[i];
        grow = ma.g_m + (ma.single_offsets[i] + (c - ma.pair_offsets[i]) / m) * CZ;
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        zb[cb][t] = *reinterpret_cast<const bf16x8*>(z + c * CZ + 16 * t + 8 * h);
        f32x4 g0, g1;
        if constexpr (FROM_MEAN) {
          // as the mean's adjoint kernel: g_m / M_i, then + g_in
          g0 = *reinterpret_cast<const f32x4*>(grow + 16 * t + 8 * h);
          g1 = *reinterpret_cast<const f32x4*>(grow + 16 * t + 8 * h + 4);
          if (ma.g_in) {
            const f32x4 i0 = *reinterpret_cast<const f32x4*>(ma.g_in + c * CZ + 16 * t + 8 * h);
            const f32x4 i1 =
                *reinterpret_cast<const f32x4*>(ma.g_in + c * CZ + 16 * t + 8 * h + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              g0[e] = g0[e] + i0[e];
              g1[e] = g1[e] + i1[e];
            }
          }
        } else {
          g0 = *reinterpret_cast<const f32x4*>(G + c * CZ + 16 * t + 8 * h);
          g1 = *reinterpret_cast<const f32x4*>(G + c * CZ + 16 * t + 8 * h + 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[cb][t >> 1][8 * (t & 1) + e] = g0[e];
          y[cb][t >> 1][8 * (t & 1) + 4 + e] = g1[e];
          gb[cb][t][e] = (bf16)g0[e];
          gb[cb][t][4 + e] = (bf16)g1[e];
        }
      }
    }

    // The tile's z and G have landed before the chunk loop. Without this wait
    // the compiler's count at the loop header merges the prologue's pending
    // loads with the loop's own, and it waits on vmcnt before the products
    // of every chunk, which then also waits for the weight loads issued at
    // the chunk's start for two chunks ahead.
    __builtin_amdgcn_s_waitcnt(kBwWaitVm0);

    // chunk j reads buffer j % 2; `nxt` holds chunk j + 1, `fill` receives
    // chunk j + 2 (chunks wrap into the next tile's: the weights repeat)
    auto chunk = [&](int j, bf16x8 (&nxt)[PER], bf16x8 (&fill)[PER]) {
      const int buf = j & 1;
      load_chunk(j + 2, fill);
      const bf16x8* wb = wbuf[buf];
      f32x16 pre[CB], gh[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        pre[cb] = f32x16{};
        gh[cb] = f32x16{};
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const bf16x8 a1 = wb[64 * t + lane];
        const bf16x8 a2 = wb[F1 + 64 * t + lane];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          pre[cb] = bw_mfma(a1, zb[cb][t], pre[cb]);
          gh[cb] = bw_mfma(a2, gb[cb][t], gh[cb]);
        }
      }
      // mask, pack, and the per-cell rows of H and g_H for the weight gradients
      bf16x8 hf[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t c = cell0 + 32 * cb + l32;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 hv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = pre[cb][8 * s + e];
            hv[e] = (bf16)(pv > 0.f ? pv : 0.f);
            hf[cb][s][e] = (bf16)(pv > 0.f ? gh[cb][8 * s + e] : 0.f);
          }
          if (WRITE_H && c < cells) {
            const int64_t o = c * HID + 32 * j + 16 * s + 8 * h;
            *reinterpret_cast<bf16x8*>(H + o) = hv;
            *reinterpret_cast<bf16x8*>(GH + o) = hf[cb][s];
          }
        }
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 a3 = wb[F1 + F2 + 64 * (2 * fb + s) + lane];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) y[cb][fb] = bw_mfma(a3, hf[cb][s], y[cb][fb]);
        }
      // the other buffer was last read in chunk j - 1, before the previous barrier
      store_chunk(buf ^ 1, nxt);
      __syncthreads();
    };
    for (int j = 0; j < NCH; j += 2) {
      chunk(j, stB, stA);
      chunk(j + 1, stA, stB);
    }

    // g_z (fp32) and bf16(G) of this wave's cells
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int64_t c = cell0 + 32 * cb + l32;
      if (c >= cells) continue;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        f32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o0[e] = y[cb][t >> 1][8 * (t & 1) + e];
          o1[e] = y[cb][t >> 1][8 * (t & 1) + 4 + e];
        }
        *reinterpret_cast<f32x4*>(g_z + c * CZ + 16 * t + 8 * h) = o0;
        *reinterpret_cast<f32x4*>(g_z + c * CZ + 16 * t + 8 * h + 4) = o1;
        *reinterpret_cast<bf16x8*>(Gb + c * CZ + 16 * t + 8 * h) = gb[cb][t];
      }
    }
  }
}

// g_m[row] / M_i for every pair row, each a float4 per thread (the same
// division, in the same precision, as the mean's adjoint kernel).
__global__ __launch_bounds__(256) void k_mean_rows(const float* __restrict__ g_m,
                                                   float* __restrict__ out,
                                                   const int64_t* __restrict__ row_splits,
                                                   int64_t T, int c_z) {
  const int q4 = c_z / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 of the rows
  if (idx >= T * q4) return;
  const int64_t r = idx / q4;
  const float nf = (float)(row_splits[r + 1] - row_splits[r]);
  f32x4 v = *reinterpret_cast<const f32x4*>(g_m + 4 * idx);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = v[e] / nf;
  *reinterpret_cast<f32x4*>(out + 4 * idx) = v;
}

}  // namespace

bool transition_backward_has_mfma(int c_z, int hidden, nt_dtype dtype) {
  return dtype == NT_BF16 && c_z == 128 && hidden == 512;
}

hipError_t launch_transition_backward_mfma(const nt_partition& p, const void* z, const float* G,
                                           const float* g_m, const float* g_in, const void* W1,
                                           const void* W2T, const void* W1T, float* g_z,
                                           void* H, void* GH, void* Gb, float* gm_rows,
                                           int cus, hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  if (g_m) {
    const int64_t n4 = p.T * (128 / 4);
    hipLaunchKernelGGL(k_mean_rows, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       g_m, gm_rows, p.row_splits, p.T, 128);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_m = gm_rows;
  }
  static_assert(kBwTileCells == kSampleIndexSpan, "tiles use the partition's sample index");
  const int64_t ntiles = (p.cells + kBwTileCells - 1) / kBwTileCells;
  const int64_t grid = ntiles < cus ? ntiles : cus;
  const MeanAdjoint ma{g_m, g_in, p.pair_offsets, p.single_offsets, p.col_lengths,
                       p.tile_sample};
  const bf16* zz = static_cast<const bf16*>(z);
  const bf16* w1 = static_cast<const bf16*>(W1);
  const bf16* w2t = static_cast<const bf16*>(W2T);
  const bf16* w1t = static_cast<const bf16*>(W1T);
  bf16* hh = static_cast<bf16*>(H);
  bf16* gh = static_cast<bf16*>(GH);
  bf16* gb = static_cast<bf16*>(Gb);
  const dim3 gd((unsigned)grid), bd(kBwThreads);
  if (H && g_m)
    hipLaunchKernelGGL((k_transition_bwd<128, 512, true, true>), gd, bd, 0, stream, zz, G, ma,
                       w1, w2t, w1t, g_z, hh, gh, gb, p.cells, ntiles);
  else if (H)
    hipLaunchKernelGGL((k_transition_bwd<128, 512, true, false>), gd, bd, 0, stream, zz, G, ma,
                       w1, w2t, w1t, g_z, hh, gh, gb, p.cells, ntiles);
  else if (g_m)
    hipLaunchKernelGGL((k_transition_bwd<128, 512, false, true>), gd, bd, 0, stream, zz, G, ma,
                       w1, w2t, w1t, g_z, hh, gh, gb, p.cells, ntiles);
  else
    hipLaunchKernelGGL((k_transition_bwd<128, 512, false, false>), gd, bd, 0, stream, zz, G, ma,
                       w1, w2t, w1t, g_z, hh, gh, gb, p.cells, ntiles);
  return hipGetLastError();
}

}  // namespace nt
