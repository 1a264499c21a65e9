// Pre-normalised SwiGLU pair transition (DanLing NestedTensor, Equation 1
// second line, P~ = P + h(LN(P)); Appendix A.1: the measured update is a
// residual, pre-normalised SwiGLU of expansion four):
//   x = LN(z) = (z - mean) / sqrt(var + eps) * gamma + beta   over the c_z features
//   z_out = z + (silu(x Wg^T) * (x Wu^T)) Wd^T,               silu(g) = g / (1 + e^-g)
// over the packed cells (Section 3.3: dense work on the sum N_i^2 valid cells).
//
// bf16 storage, fp32 statistics and accumulation, c_z in {64, 128}, hidden a
// multiple of 32. A workgroup of four waves owns 256 consecutive cells, 64 per
// wave as four 16-cell MFMA column blocks (v_mfma_f32_16x16x32_bf16). Lane
// (l16, g) holds cell 16 cb + l16, features 32 kb + 8 g .. + 7:
//  * LN: each lane sums its 8 KB features; a butterfly over the four lanes of
//    the cell (lane xor 16, xor 32) gives the mean, then the variance of the
//    centred values the same way (two passes, fp32);
//  * per 32-unit hidden chunk the gate and value products G^T = Wg . x^T and
//    U^T = Wu . x^T land with lane group g holding hidden units 8 g .. 8 g + 7
//    (rows permuted as in the ReLU kernels), so silu(G) * U packs lane-locally
//    into the second product's operand, Y^T += Wd . A^T;
//  * the residual adds the bf16 input in fp32 and rounds once.
// The three weight chunks stream through two LDS buffers.
//
// Fused form (the block's, Equation 1's first two lines in one kernel): z is
// not read but formed, z = a[row] + b[col] from the fp32 projections, each
// lane decoding its cell (Equation 3 inverted, from the first sample of the
// 256-cell tile); LN takes its statistics on that fp32 z, and the epilogue
// forms z again in fp32 for the residual, so the pair state is rounded once,
// on output.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kSgWaves = 8;            // two waves per SIMD
constexpr int kSgCellsPerWave = 32;
constexpr int kSgBlocks = kSgCellsPerWave / 16;
constexpr int kSgTileCells = kSgWaves * kSgCellsPerWave;
constexpr int kSgChunk = 32;

__device__ __forceinline__ f32x4 sg_mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// GEMM1 hid-block hb, result row q -> hidden unit 8 (q / 4) + 4 hb + q % 4 of
// the chunk: lane group g then holds hidden units 8 g .. 8 g + 7 (both blocks).
__device__ __forceinline__ int sg_hid_row(int hb, int q) {
  return 8 * (q >> 2) + 4 * hb + (q & 3);
}
// GEMM2 feature block fb, result row q -> feature 32 (fb / 2) + 8 (q / 4) +
// 4 (fb % 2) + q % 4: lane group g holds the features of its z slice.
__device__ __forceinline__ int sg_feat_row(int fb, int q) {
  return 32 * (fb >> 1) + 8 * (q >> 2) + 4 * (fb & 1) + (q & 3);
}

static_assert(kSgTileCells == kSampleIndexSpan, "a tile is one entry of the sample index");

template <int CZ, bool FUSED>
__global__ __launch_bounds__(kSgWaves * 64, 2) void k_transition_swiglu(
    const bf16* __restrict__ z_in, const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths,
    const int32_t* __restrict__ tile_sample, const float* __restrict__ gamma,
    const float* __restrict__ beta, const bf16* __restrict__ Wg, const bf16* __restrict__ Wu,
    const bf16* __restrict__ Wd, bf16* z_out, int64_t cells, int hidden, float eps) {
  constexpr int KB = CZ / 32;          // k-blocks of GEMM1 (K = c_z)
  constexpr int FB = CZ / 16;          // feature blocks of GEMM2's result
  constexpr int GF = 2 * KB;           // fragments per chunk of each of Wg, Wu
  constexpr int NFRAG = 2 * GF + FB;   // fragments per chunk, 1 KiB each
  constexpr int PIECES = NFRAG * 64;
  constexpr int THREADS = kSgWaves * 64;
  constexpr int PER_THREAD = (PIECES + THREADS - 1) / THREADS;  // the last may be partial

  __shared__ bf16x8 lds[2][PIECES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t cell0 = (int64_t)blockIdx.x * kSgTileCells + wave * kSgCellsPerWave;

  // ---- prologue: z slices and their LN. Fused: the single rows of each
  // lane's cell (a cell past the end decodes as the last one; it is not
  // stored).
  int64_t arow[kSgBlocks], bcol[kSgBlocks];
  if constexpr (FUSED) {
    const int i0 = tile_sample[blockIdx.x];
#pragma unroll
    for (int cb = 0; cb < kSgBlocks; ++cb) {
      const int64_t c0 = cell0 + cb * 16 + l16;
      const int64_t cell = c0 < cells ? c0 : cells - 1;
      int i = i0;
      while (pair_offsets[i + 1] <= cell) ++i;
      const int64_t m = col_lengths[i], local = cell - pair_offsets[i];
      const int64_t r = local / m;
      arow[cb] = (single_offsets[i] + r) * CZ + 8 * g;
      bcol[cb] = (col_offsets[i] + (local - r * m)) * CZ + 8 * g;
    }
  }
  // z of one lane's cell: 8 features of each k-block, fp32
  auto fused_z = [&](int cb, int kb, float* z8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 va = *reinterpret_cast<const f32x4*>(a + arow[cb] + 32 * kb + 4 * h);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(b + bcol[cb] + 32 * kb + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) z8[4 * h + e] = va[e] + vb[e];
    }
  };
  bf16x8 zb[kSgBlocks][KB], xb[kSgBlocks][KB];
  if constexpr (!FUSED) {
#pragma unroll
    for (int cb = 0; cb < kSgBlocks; ++cb) {
      const int64_t cell = cell0 + cb * 16 + l16;
      if (cell < cells) {
        const bf16* zr = z_in + cell * CZ + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          zb[cb][kb] = *reinterpret_cast<const bf16x8*>(zr + 32 * kb);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) zb[cb][kb][e] = (bf16)0.f;
      }
    }
  }
  float gam[KB][8], bet[KB][8];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 vg = *reinterpret_cast<const f32x4*>(gamma + 32 * kb + 8 * g + 4 * h);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(beta + 32 * kb + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gam[kb][4 * h + e] = vg[e];
        bet[kb][4 * h + e] = vb[e];
      }
    }
#pragma unroll
  for (int cb = 0; cb < kSgBlocks; ++cb) {
    float zf[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (FUSED) {
        fused_z(cb, kb, zf[kb]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) zf[kb][e] = (float)zb[cb][kb][e];
      }
    }
    float s = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += zf[kb][e];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    const float mu = s * (1.f / CZ);
    float q = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = zf[kb][e] - mu;
        q += d * d;
      }
    q += __shfl_xor(q, 16);
    q += __shfl_xor(q, 32);
    const float rstd = 1.f / sqrtf(q * (1.f / CZ) + eps);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        xb[cb][kb][e] = (bf16)((zf[kb][e] - mu) * rstd * gam[kb][e] + bet[kb][e]);
  }

  // ---- weight staging: piece p of a chunk -> fragment p / 64, lane p % 64
  auto stage_src = [&](int ch, int p) -> const bf16* {
    const int F = p >> 6, L = p & 63, q = L & 15, gg = L >> 4;
    if (F < 2 * GF) {
      const bf16* W = F < GF ? Wg : Wu;
      const int f = F % GF, hb = f / KB, kb = f % KB;
      const int hid = ch * kSgChunk + sg_hid_row(hb, q);
      return W + (int64_t)hid * CZ + 32 * kb + 8 * gg;
    }
    const int fb = F - 2 * GF;
    return Wd + (int64_t)sg_feat_row(fb, q) * hidden + ch * kSgChunk + 8 * gg;
  };
  const int nchunks = hidden / kSgChunk;
  bf16x8 stage[PER_THREAD];
#pragma unroll
  for (int k = 0; k < PER_THREAD; ++k)
    if (tid + k * THREADS < PIECES)
      stage[k] = *reinterpret_cast<const bf16x8*>(stage_src(0, tid + k * THREADS));
#pragma unroll
  for (int k = 0; k < PER_THREAD; ++k)
    if (tid + k * THREADS < PIECES) lds[0][tid + k * THREADS] = stage[k];
  __syncthreads();

  f32x4 y[kSgBlocks][FB];
#pragma unroll
  for (int cb = 0; cb < kSgBlocks; ++cb)
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) y[cb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < nchunks; ++ch) {
    const int cur = ch & 1;
    const bool more = ch + 1 < nchunks;
    if (more) {
#pragma unroll
      for (int k = 0; k < PER_THREAD; ++k)
        if (tid + k * THREADS < PIECES)
          stage[k] = *reinterpret_cast<const bf16x8*>(stage_src(ch + 1, tid + k * THREADS));
    }
    // gate and value products, one 16-cell block at a time
    bf16x8 af[kSgBlocks];
#pragma unroll
    for (int cb = 0; cb < kSgBlocks; ++cb) {
      f32x4 hg[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 hu[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          hg[hb] = sg_mfma(lds[cur][(hb * KB + kb) * 64 + lane], xb[cb][kb], hg[hb]);
          hu[hb] = sg_mfma(lds[cur][(GF + hb * KB + kb) * 64 + lane], xb[cb][kb], hu[hb]);
        }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gt = hg[hb][j];
          af[cb][4 * hb + j] = (bf16)(gt / (1.f + __expf(-gt)) * hu[hb][j]);
        }
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      const bf16x8 wd = lds[cur][(2 * GF + fb) * 64 + lane];
#pragma unroll
      for (int cb = 0; cb < kSgBlocks; ++cb) y[cb][fb] = sg_mfma(wd, af[cb], y[cb][fb]);
    }
    if (more) {
#pragma unroll
      for (int k = 0; k < PER_THREAD; ++k)
        if (tid + k * THREADS < PIECES) lds[cur ^ 1][tid + k * THREADS] = stage[k];
    }
    __syncthreads();
  }

  // ---- epilogue: residual in fp32, one rounding, 16-byte stores
#pragma unroll
  for (int cb = 0; cb < kSgBlocks; ++cb) {
    const int64_t cell = cell0 + cb * 16 + l16;
    if (cell >= cells) continue;
    bf16* dst = z_out + cell * CZ + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float zf[8];
      if constexpr (FUSED) {
        fused_z(cb, kb, zf);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) zf[e] = (float)zb[cb][kb][e];
      }
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)(zf[e] + y[cb][2 * kb + (e >> 2)][e & 3]);
      *reinterpret_cast<bf16x8*>(dst + 32 * kb) = o;
    }
  }
}

}  // namespace

bool transition_swiglu_supported(int c_z, int hidden, nt_dtype dtype) {
  return dtype == NT_BF16 && (c_z == 64 || c_z == 128) && hidden > 0 && hidden % kSgChunk == 0;
}

hipError_t launch_transition_swiglu(const nt_partition& p, const void* z_in, const void* a,
                                    const void* b, void* z_out, const float* gamma,
                                    const float* beta, const void* Wg, const void* Wu,
                                    const void* Wd, int c_z, int hidden, float eps,
                                    hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  const int64_t blocks = (p.cells + kSgTileCells - 1) / kSgTileCells;
  const bf16 *zi = static_cast<const bf16*>(z_in), *wg = static_cast<const bf16*>(Wg),
             *wu = static_cast<const bf16*>(Wu), *wd = static_cast<const bf16*>(Wd);
  const float *af = static_cast<const float*>(a), *bf = static_cast<const float*>(b);
  bf16* zo = static_cast<bf16*>(z_out);
  auto kern = z_in ? (c_z == 128 ? k_transition_swiglu<128, false> : k_transition_swiglu<64, false>)
                   : (c_z == 128 ? k_transition_swiglu<128, true> : k_transition_swiglu<64, true>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kSgWaves * 64), 0, stream, zi, af, bf,
                     p.pair_offsets, p.single_offsets, p.col_offsets, p.col_lengths,
                     p.tile_sample, gamma, beta, wg, wu, wd, zo, p.cells, hidden, eps);
  return hipGetLastError();
}

}  // namespace nt
