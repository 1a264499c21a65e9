// Residual pair transition z_out = z + relu(z W1^T) W2^T over the packed
// cells (DanLing NestedTensor, Equation 1 second line with a ReLU MLP update;
// Section 3.3 "Dense work across valid positions": the transition runs over
// sum N_i^2 cells, never over the B x N_max^2 envelope).
//
// bf16 fast path (c_z in {64, 128}, hidden a multiple of 32): a workgroup of
// four waves owns 256 consecutive cells, 64 per wave, and streams the weights
// through LDS in chunks of 32 hidden units. Per chunk each wave computes
//   H^T (32 x 64)  = W1_chunk (32 x c_z) . z^T (c_z x 64)   (v_mfma 16x16x32 bf16)
//   Y^T (c_z x 64) += W2_chunk (c_z x 32) . relu(H)^T       (v_mfma 16x16x32 bf16)
// Computing the transposed products makes the accumulator layout of H^T
// (lane = cell, 4 consecutive rows per lane group) the operand layout of the
// second product after a lane-local relu + bf16 pack, so H never leaves the
// registers. z stays in registers from prologue to epilogue; the residual is
// added in fp32 and rounded once. With fp32 a and b given instead of z, the
// broadcast a[row] + b[col] is formed in the prologue (fused form): the MLP
// reads it rounded to bf16 and the epilogue re-forms it in fp32 for the
// residual, so the pair state is rounded once, on output.
//
// Generic path (any width, fp32 or bf16): plain fp32 arithmetic through LDS.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

// ---------------------------------------------------------------- MFMA path
constexpr int kWaves = 4;
constexpr int kCellsPerWave = 64;
constexpr int kCellBlocks = kCellsPerWave / 16;       // 16-cell MFMA column blocks
constexpr int kTileCells = kWaves * kCellsPerWave;    // 256
constexpr int kChunk = 32;                            // hidden units per LDS chunk

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row permutations that make accumulator layouts line up with operand layouts.
// In a 16x16 MFMA result, lane group g = lane / 16 holds rows 4g..4g+3.
//  - GEMM1 hid-block hb, result row q -> hidden unit 8 (q / 4) + 4 hb + (q % 4),
//    so lane group g ends up holding hidden units 8g..8g+7 (both blocks).
//  - GEMM2 feature-block fb, result row q -> feature
//    32 (fb / 2) + 8 (q / 4) + 4 (fb % 2) + (q % 4), so lane group g holds
//    features 32 k + 8 g + (0..7) for k = fb / 2: the same features its z
//    operand slice holds, making the residual add lane-local.
__device__ __forceinline__ int w1_row(int hb, int q) { return 8 * (q >> 2) + 4 * hb + (q & 3); }
__device__ __forceinline__ int w2_row(int fb, int q) {
  return 32 * (fb >> 1) + 8 * (q >> 2) + 4 * (fb & 1) + (q & 3);
}

template <int CZ, bool FUSED>
__global__ __launch_bounds__(kWaves * 64, 1) void k_transition_mfma(
    const bf16* __restrict__ z_in, const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths, int B,
    const bf16* __restrict__ W1,
    const bf16* __restrict__ W2, bf16* z_out, int64_t cells, int hidden) {
  constexpr int KB = CZ / 32;             // k-blocks of GEMM1 (K = c_z)
  constexpr int FB = CZ / 16;             // feature blocks of GEMM2's result
  constexpr int W1F = 2 * KB;             // W1 fragments per chunk (2 hid-blocks)
  constexpr int NFRAG = W1F + FB;         // fragments per chunk, 1 KiB each
  constexpr int PIECES = NFRAG * 64;      // 16-byte pieces per chunk
  constexpr int PER_THREAD = PIECES / (kWaves * 64);
  static_assert(PIECES % (kWaves * 64) == 0, "chunk staging must divide evenly");

  __shared__ bf16x8 lds[2][PIECES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t cell0 = (int64_t)blockIdx.x * kTileCells + wave * kCellsPerWave;

  // ---- prologue: this lane's z slices, cell 16 cb + l16, features 32 kb + 8 g ..
  bf16x8 zb[kCellBlocks][KB];
  int32_t arow[kCellBlocks], brow[kCellBlocks];  // fused form: single rows of the cell
#pragma unroll
  for (int cb = 0; cb < kCellBlocks; ++cb) {
    const int64_t cell = cell0 + cb * 16 + l16;
    arow[cb] = brow[cb] = 0;
    if (cell < cells) {
      if constexpr (FUSED) {
        const Cell x = decode_cell(pair_offsets, single_offsets, col_offsets, col_lengths, B, cell);
        arow[cb] = (int32_t)(x.eta + x.r);
        brow[cb] = (int32_t)(x.mu + x.c);
        const float* ar = a + (int64_t)arow[cb] * CZ + 8 * g;
        const float* br = b + (int64_t)brow[cb] * CZ + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 va = *reinterpret_cast<const f32x4*>(ar + 32 * kb + 4 * h);
            const f32x4 vb = *reinterpret_cast<const f32x4*>(br + 32 * kb + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) zb[cb][kb][4 * h + e] = (bf16)(va[e] + vb[e]);
          }
        }
      } else {
        const bf16* zr = z_in + cell * CZ + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) zb[cb][kb] = *reinterpret_cast<const bf16x8*>(zr + 32 * kb);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) zb[cb][kb][e] = (bf16)0.f;
    }
  }

  // ---- weight staging: piece p of a chunk -> fragment p / 64, lane p % 64
  auto stage_src = [&](int ch, int p) -> const bf16* {
    const int F = p >> 6, L = p & 63, q = L & 15, gg = L >> 4;
    if (F < W1F) {
      const int hb = F / KB, kb = F % KB;
      const int hid = ch * kChunk + w1_row(hb, q);
      return W1 + (int64_t)hid * CZ + 32 * kb + 8 * gg;
    }
    const int fb = F - W1F;
    return W2 + (int64_t)w2_row(fb, q) * hidden + ch * kChunk + 8 * gg;
  };

  const int nchunks = hidden / kChunk;
  bf16x8 stage[PER_THREAD];
#pragma unroll
  for (int k = 0; k < PER_THREAD; ++k)
    stage[k] = *reinterpret_cast<const bf16x8*>(stage_src(0, tid + k * kWaves * 64));
#pragma unroll
  for (int k = 0; k < PER_THREAD; ++k) lds[0][tid + k * kWaves * 64] = stage[k];
  __syncthreads();

  f32x4 y[kCellBlocks][FB];
#pragma unroll
  for (int cb = 0; cb < kCellBlocks; ++cb)
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) y[cb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < nchunks; ++ch) {
    const int cur = ch & 1;
    const bool more = ch + 1 < nchunks;
    if (more) {
#pragma unroll
      for (int k = 0; k < PER_THREAD; ++k)
        stage[k] = *reinterpret_cast<const bf16x8*>(stage_src(ch + 1, tid + k * kWaves * 64));
    }
    bf16x8 w1f[2][KB], w2f[FB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) w1f[hb][kb] = lds[cur][(hb * KB + kb) * 64 + lane];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) w2f[fb] = lds[cur][(W1F + fb) * 64 + lane];

    f32x4 h[kCellBlocks][2];
#pragma unroll
    for (int cb = 0; cb < kCellBlocks; ++cb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) h[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cb = 0; cb < kCellBlocks; ++cb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) h[cb][hb] = mfma16(w1f[hb][kb], zb[cb][kb], h[cb][hb]);

    bf16x8 hf[kCellBlocks];
#pragma unroll
    for (int cb = 0; cb < kCellBlocks; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hf[cb][j] = (bf16)fmaxf(h[cb][0][j], 0.f);
        hf[cb][4 + j] = (bf16)fmaxf(h[cb][1][j], 0.f);
      }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int cb = 0; cb < kCellBlocks; ++cb) y[cb][fb] = mfma16(w2f[fb], hf[cb], y[cb][fb]);

    if (more) {
#pragma unroll
      for (int k = 0; k < PER_THREAD; ++k) lds[cur ^ 1][tid + k * kWaves * 64] = stage[k];
    }
    __syncthreads();
  }

  // ---- epilogue: residual in fp32, one rounding, 16-byte stores
#pragma unroll
  for (int cb = 0; cb < kCellBlocks; ++cb) {
    const int64_t cell = cell0 + cb * 16 + l16;
    if (cell >= cells) continue;
    bf16* dst = z_out + cell * CZ + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bf16x8 o;
      if constexpr (FUSED) {
        const float* ar = a + (int64_t)arow[cb] * CZ + 8 * g + 32 * kb;
        const float* br = b + (int64_t)brow[cb] * CZ + 8 * g + 32 * kb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 va = *reinterpret_cast<const f32x4*>(ar + 4 * h);
          const f32x4 vb = *reinterpret_cast<const f32x4*>(br + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[4 * h + e] = (bf16)((va[e] + vb[e]) + y[cb][2 * kb + h][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = (bf16)((float)zb[cb][kb][e] + y[cb][2 * kb + (e >> 2)][e & 3]);
      }
      *reinterpret_cast<bf16x8*>(dst + 32 * kb) = o;
    }
  }
}

// ------------------------------------------------- persistent MFMA path
// Throughput path for c_z in {64, 128} when W1 fits in LDS
// (hidden * c_z * 2 bytes <= 128 KiB). v_mfma_f32_32x32x16_bf16 keeps the
// matrix cores busy from a single wave per SIMD, which the 16x16 shape does
// not. Organisation:
//  * one workgroup (four waves) per CU, looping over 256-cell tiles; each
//    wave owns 64 cells as two 32-cell MFMA column blocks;
//  * W1 is loaded into LDS once per workgroup and stays resident;
//  * W2 streams through a three-slot LDS ring, one 32-hidden chunk per step;
//    its global loads are issued two steps before the ring slot is written;
//  * each wave prefetches the next step's W2 fragments into registers, and
//    the two GEMMs are skewed by one chunk: step j issues GEMM2 of chunk j - 1
//    and GEMM1 of chunk j, one MFMA of each in turn.
// Lane layouts of a 32x32x16 MFMA: operand lane l holds row / column l % 32
// and k-group l / 32 (8 consecutive k); result element j of lane group
// h = l / 32 is row 8 (j / 4) + 4 h + (j % 4) of column l % 32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Result row rho of GEMM1 -> hidden unit within its 32-unit chunk, chosen so
// that lane group h holds units 16 s + 8 h + (0..7) in elements 8 s .. 8 s + 7:
// exactly the k-group of the second product's operand for its k-step s.
__device__ __forceinline__ int p32_row(int rho) {
  return 16 * (rho >> 4) + 8 * ((rho >> 2) & 1) + 4 * ((rho >> 3) & 1) + (rho & 3);
}
// GEMM2 feature block fb uses the same pattern over features 32 fb .. 32 fb + 31,
// so result element j of lane group h is feature 16 (2 fb + j / 8) + 8 h + j % 8:
// the feature the lane's z operand slice (k-step 2 fb + j / 8, slot j % 8) holds.

// relu by the sign bit: a non-negative float has a non-negative integer image,
// a negative one a negative image, so an integer max with 0 is max(x, +0).
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Samples whose partition arrays the fused persistent kernel keeps in LDS.
constexpr int kLdsSamples = 384;

// Sample, row and column of packed cell `cell` (Equation 3 inverted), with the
// sample searched from `i0` upwards; po/eta/mu/m are the pair offsets, the
// row and column single offsets and the cells per pair row (M_i), in LDS or
// in global memory.
template <typename OFF, typename IDX, typename CIDX>
__device__ __forceinline__ void decode_from(const OFF* po, const IDX* eta, const CIDX* mu,
                                            const int32_t* m, int i0, int64_t cell, int64_t& row,
                                            int64_t& col) {
  int i = i0;
  while (po[i + 1] <= cell) ++i;  // ends: po[B] = cells > cell
  const int64_t len = m[i], local = cell - (int64_t)po[i];
  int64_t r, c;
  if (len <= 65535 && local <= 0xffffffffLL) {
    const uint32_t q32 = (uint32_t)local / (uint32_t)len;
    r = q32;
    c = (uint32_t)local - q32 * (uint32_t)len;
  } else {
    r = local / len;
    c = local - r * len;
  }
  row = (int64_t)eta[i] + r;
  col = (int64_t)mu[i] + c;
}

template <int CZ, int HID, bool FUSED>
__global__ __launch_bounds__(kWaves * 64, 1) void k_transition_p32(
    const bf16* __restrict__ z_in, const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths, int B,
    bool lds_part, const bf16* __restrict__ W1,
    const bf16* __restrict__ W2, bf16* z_out, int64_t cells, int64_t ntiles, int64_t T) {
  constexpr int KT = CZ / 16;        // GEMM1 k-steps
  constexpr int FB = CZ / 32;        // GEMM2 feature blocks
  constexpr int NCH = HID / kChunk;  // hidden chunks
  constexpr int CB = kCellsPerWave / 32;
  constexpr int THREADS = kWaves * 64;
  constexpr int W1_PIECES = NCH * KT * 64;
  constexpr int W2_PIECES = FB * 2 * 64;
  constexpr int W2_PER_THREAD = W2_PIECES / THREADS;
  constexpr int W1_PER_THREAD = W1_PIECES / THREADS;
  constexpr int W1_BATCH = W1_PER_THREAD < 8 ? W1_PER_THREAD : 8;
  static_assert(W2_PIECES % THREADS == 0 && W1_PIECES % THREADS == 0, "staging split");
  static_assert(W1_PER_THREAD % W1_BATCH == 0, "W1 load batches");
  static_assert(NCH >= 2 && CZ % 32 == 0, "shape");
  // GEMM1 and GEMM2 each issue CB * KT MFMAs per step (CB * FB * 2 == CB * KT)
  static_assert(FB * 2 == KT, "the two products interleave one to one");
  // Between tiles the W2 ring is empty and each wave stages rows through its
  // quarter of it: RB bytes of 32 rows per round, rows SR bytes apart (the
  // 16-byte pad spreads a column of 16-byte reads over all banks). A 16-byte
  // per-lane access covers LPR lanes per row and CPI rows, 1 KiB per wave.
  constexpr int STAGE = 3 * W2_PIECES * 16 / kWaves;
  constexpr int RB = CZ == 128 ? 128 : 64;
  constexpr int SR = RB + 16;
  constexpr int LPR = RB / 16;
  constexpr int CPI = 64 / LPR;
  constexpr int IPR = 32 / CPI;
  constexpr int AROW = CZ * 4;       // bytes of one fp32 row of a or b
  constexpr int NBR = AROW / RB;     // rounds per fp32 row
  constexpr int NZR = 2 * CZ / RB;   // rounds per bf16 row
  static_assert(32 * SR + (FUSED ? 2 * AROW : 0) <= STAGE, "staging fits in the ring");
  static_assert(RB % 64 == 0 && IPR * CPI == 32, "staging geometry");

  __shared__ bf16x8 w1s[W1_PIECES];
  __shared__ bf16x8 ring[3 * W2_PIECES];
  __shared__ int64_t po_s[FUSED ? kLdsSamples + 1 : 1];
  __shared__ int32_t eta_s[FUSED ? kLdsSamples : 1];
  __shared__ int32_t n_s[FUSED ? kLdsSamples : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int prow = lane / LPR, pseg = 16 * (lane % LPR);  // coalesced-access coordinates
  unsigned char* const stage = reinterpret_cast<unsigned char*>(ring) + wave * STAGE;

  auto w1_src = [&](int p) -> const bf16* {
    const int c = p / (KT * 64), t = (p >> 6) % KT, L = p & 63;
    const int hid = c * kChunk + p32_row(L & 31);
    return W1 + (int64_t)hid * CZ + 16 * t + 8 * (L >> 5);
  };
  auto w2_src = [&](int c, int p) -> const bf16* {
    const int fb = p >> 7, s = (p >> 6) & 1, L = p & 63;
    return W2 + (int64_t)(32 * fb + p32_row(L & 31)) * HID + c * kChunk + 16 * s + 8 * (L >> 5);
  };
  auto slot = [&](int s) -> bf16x8* { return ring + s * W2_PIECES; };

  if constexpr (FUSED) {
    if (lds_part) {  // B <= kLdsSamples and every single offset fits in 32 bits
      for (int i = tid; i <= B; i += THREADS) {
        po_s[i] = pair_offsets[i];
        if (i < B) {
          eta_s[i] = (int32_t)single_offsets[i];
          n_s[i] = col_lengths[i];
        }
      }
    }
  }
  // resident W1 in fragment order (chunk, k-step, lane), batches of loads in flight
  for (int k0 = 0; k0 < W1_PER_THREAD; k0 += W1_BATCH) {
    bf16x8 tmp[W1_BATCH];
#pragma unroll
    for (int k = 0; k < W1_BATCH; ++k)
      tmp[k] = *reinterpret_cast<const bf16x8*>(w1_src(tid + (k0 + k) * THREADS));
#pragma unroll
    for (int k = 0; k < W1_BATCH; ++k) w1s[tid + (k0 + k) * THREADS] = tmp[k];
  }
  __syncthreads();

  // Fragments are read from LDS one step before the MFMAs that use them:
  // w1f holds W1 of the chunk the next GEMM1 multiplies, w2f the W2 of the
  // chunk the next GEMM2 multiplies.
  bf16x8 w1f[KT], w2f[FB][2];
#pragma unroll
  for (int t = 0; t < KT; ++t) w1f[t] = w1s[t * 64 + lane];
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t tile0 = tile * kTileCells;
    const int64_t cell0 = tile0 + wave * kCellsPerWave;

    // W2 chunks 0..2 of this tile, in flight while the prologue runs. The
    // stream restarts every tile (position j carries chunk j) so the ring is
    // free for staging between tiles.
    bf16x8 s0[W2_PER_THREAD], s1[W2_PER_THREAD], s_cur[W2_PER_THREAD];
#pragma unroll
    for (int k = 0; k < W2_PER_THREAD; ++k) {
      s0[k] = *reinterpret_cast<const bf16x8*>(w2_src(0, tid + k * THREADS));
      s1[k] = *reinterpret_cast<const bf16x8*>(w2_src(1, tid + k * THREADS));
      s_cur[k] = *reinterpret_cast<const bf16x8*>(w2_src(2 % NCH, tid + k * THREADS));
    }

    // ---- prologue. The accumulator starts at z (fp32), so the epilogue only
    // rounds and stores: y[cb][fb] element j is feature 16 (2 fb + j / 8) +
    // 8 h + j % 8, the feature of operand slice zb[cb][2 fb + j / 8] slot j % 8.
    bf16x8 zb[CB][KT];
    f32x16 y[CB][FB];
    if constexpr (FUSED) {
      int row32[CB], col32[CB];
      {
        int64_t row[CB], col[CB];
        if (lds_part) {
          const int i0 = find_segment(po_s, 0, B, tile0);  // tile-uniform
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int64_t cell = cell0 + 32 * cb + l32;
            decode_from(po_s, eta_s, eta_s, n_s, i0, cell < cells ? cell : cells - 1, row[cb],
                        col[cb]);
          }
        } else {
          const int i0 = find_segment(pair_offsets, 0, B, tile0);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int64_t cell = cell0 + 32 * cb + l32;
            decode_from(pair_offsets, single_offsets, col_offsets, col_lengths, i0,
                        cell < cells ? cell : cells - 1, row[cb], col[cb]);
          }
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {  // T < 2^31 on this path
          row32[cb] = (int)row[cb];
          col32[cb] = (int)col[cb];
        }
      }
      // The gathers of both cell blocks are issued together: the 32 b rows of
      // each in coalesced 16-byte accesses, and the two a rows its cells
      // start in (a cell past the end repeats the last cell's inputs; it is
      // not stored).
      constexpr int ALANES = 2 * AROW / 16;
      f32x4 braw[CB][NBR][IPR], araw[CB];
      int row_first[CB];
      bool two_rows[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        row_first[cb] =
            __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(row32[cb], 0));
        const int row_last =
            __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(row32[cb], 31));
        two_rows[cb] = row_last - row_first[cb] <= 1;  // every block does when N >= 32
        int src[IPR];
#pragma unroll
        for (int k = 0; k < IPR; ++k) src[k] = __shfl(col32[cb], k * CPI + prow);
#pragma unroll
        for (int q = 0; q < NBR; ++q)
#pragma unroll
          for (int k = 0; k < IPR; ++k)
            braw[cb][q][k] = *reinterpret_cast<const f32x4*>(
                b + (int64_t)src[k] * CZ + (q * RB + pseg) / 4);
        const int al = lane % ALANES;  // lanes past ALANES repeat lower ones
        int64_t ar = row_first[cb] + al / (AROW / 16);
        ar = ar < T ? ar : T - 1;
        araw[cb] = *reinterpret_cast<const f32x4*>(a + ar * CZ + 4 * (al % (AROW / 16)));
      }
      __builtin_amdgcn_sched_barrier(0);
      // Per block: its b rows go through LDS round by round and are read back
      // in the operand layout; the a terms come from the two staged a rows,
      // or, for a block of many short rows, from a second pass of per-cell a
      // rows through the same registers and LDS (fp32 addition commutes, so
      // the order of the two terms does not change z).
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        unsigned char* const sb = stage;
        unsigned char* const sa = stage + 32 * SR;
        if (lane < ALANES) *reinterpret_cast<f32x4*>(sa + 16 * lane) = araw[cb];
        const int dr = row32[cb] - row_first[cb];
        const unsigned char* const my_a = sa + (dr == 1 ? AROW : 0) + 32 * h;
#pragma unroll
        for (int q = 0; q < NBR; ++q) {
#pragma unroll
          for (int k = 0; k < IPR; ++k)
            *reinterpret_cast<f32x4*>(sb + (k * CPI + prow) * SR + pseg) = braw[cb][q][k];
#pragma unroll
          for (int mm = 0; mm < RB / 64; ++mm) {
            const int m = q * (RB / 64) + mm;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const f32x4 vb =
                  *reinterpret_cast<const f32x4*>(sb + l32 * SR + 64 * mm + 32 * h + 16 * u);
              // read unconditionally (inside the staging area) and select
              const f32x4 vs = *reinterpret_cast<const f32x4*>(my_a + 64 * m + 16 * u);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float zf = (two_rows[cb] ? vs[e] : 0.f) + vb[e];
                zb[cb][m][4 * u + e] = (bf16)zf;
                y[cb][m >> 1][8 * (m & 1) + 4 * u + e] = zf;
              }
            }
          }
        }
        if (!two_rows[cb]) {
          int src[IPR];
#pragma unroll
          for (int k = 0; k < IPR; ++k) src[k] = __shfl(row32[cb], k * CPI + prow);
#pragma unroll
          for (int q = 0; q < NBR; ++q)
#pragma unroll
            for (int k = 0; k < IPR; ++k)
              braw[cb][q][k] = *reinterpret_cast<const f32x4*>(
                  a + (int64_t)src[k] * CZ + (q * RB + pseg) / 4);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < NBR; ++q) {
#pragma unroll
            for (int k = 0; k < IPR; ++k)
              *reinterpret_cast<f32x4*>(sb + (k * CPI + prow) * SR + pseg) = braw[cb][q][k];
#pragma unroll
            for (int mm = 0; mm < RB / 64; ++mm) {
              const int m = q * (RB / 64) + mm;
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const f32x4 va =
                    *reinterpret_cast<const f32x4*>(sb + l32 * SR + 64 * mm + 32 * h + 16 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int j = 8 * (m & 1) + 4 * u + e;
                  const float zf = y[cb][m >> 1][j] + va[e];
                  zb[cb][m][4 * u + e] = (bf16)zf;
                  y[cb][m >> 1][j] = zf;
                }
              }
            }
          }
        }
      }
    } else {
      // z rows of a cell block are contiguous: coalesced loads through LDS
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        bf16x8 zraw[NZR][IPR];
#pragma unroll
        for (int r = 0; r < NZR; ++r)
#pragma unroll
          for (int k = 0; k < IPR; ++k) {
            int64_t c = cell0 + 32 * cb + k * CPI + prow;
            c = c < cells ? c : cells - 1;
            zraw[r][k] = *reinterpret_cast<const bf16x8*>(z_in + c * CZ + (r * RB + pseg) / 2);
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NZR; ++r) {
#pragma unroll
          for (int k = 0; k < IPR; ++k)
            *reinterpret_cast<bf16x8*>(stage + (k * CPI + prow) * SR + pseg) = zraw[r][k];
#pragma unroll
          for (int tt = 0; tt < RB / 32; ++tt) {
            const int t = r * (RB / 32) + tt;
            zb[cb][t] = *reinterpret_cast<const bf16x8*>(stage + l32 * SR + 32 * tt + 16 * h);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[cb][t >> 1][8 * (t & 1) + e] = (float)zb[cb][t][e];
          }
        }
      }
    }

    // Chunks 0 and 1 into their ring slots once every wave is done staging.
    __syncthreads();
#pragma unroll
    for (int k = 0; k < W2_PER_THREAD; ++k) {
      slot(0)[tid + k * THREADS] = s0[k];
      slot(1)[tid + k * THREADS] = s1[k];
    }
    __syncthreads();

    // Step j runs GEMM1 of chunk j into hacc[j & 1] while the relu of chunk
    // j - 1 (hacc[(j - 1) & 1]) is packed into hf a few values at a time, then
    // GEMM2 of chunk j - 1. Each fragment register is refilled from LDS for
    // the next step right after the two MFMAs that read it, so the reads have
    // the rest of the step to arrive. sched_barrier keeps this order. Ring
    // slot j % 3 holds chunk j; step j stores chunk j + 2 (loaded one step
    // earlier) and issues the loads of chunk j + 3.
    f32x16 hacc[2][CB];
    bf16x8 hf[CB][2];
#pragma unroll
    for (int j = 0; j <= NCH; ++j) {
      const int jn = j + 1 < NCH ? j + 1 : 0;  // W1 chunk of the next step
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        if (j < NCH) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            hacc[j & 1][cb] = mfma32(w1f[t], zb[cb][t], t == 0 ? f32x16{} : hacc[j & 1][cb]);
          w1f[t] = w1s[(jn * KT + t) * 64 + lane];
        }
        if (j > 0) {  // relu of chunk j - 1: piece t of CB * 2 * 8 values
          constexpr int PER = CB * 2 * 8 / KT;
#pragma unroll
          for (int q = 0; q < PER; ++q) {
            const int v = t * PER + q, cb = v / 16, s = (v / 8) % 2, e = v % 8;
            hf[cb][s][e] = (bf16)relu_bits(hacc[(j - 1) & 1][cb][8 * s + e]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j > 0) {
#pragma unroll
        for (int k = 0; k < 2 * FB; ++k) {
          const int s = k / FB, fb = k % FB;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) y[cb][fb] = mfma32(w2f[fb][s], hf[cb][s], y[cb][fb]);
          if (j < NCH) w2f[fb][s] = slot(j % 3)[(fb * 2 + s) * 64 + lane];
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int s = 0; s < 2; ++s) w2f[fb][s] = slot(0)[(fb * 2 + s) * 64 + lane];
      }
      if (j < NCH) {
        bf16x8 s_next[W2_PER_THREAD];
        if (j + 3 < NCH) {
#pragma unroll
          for (int k = 0; k < W2_PER_THREAD; ++k)
            s_next[k] = *reinterpret_cast<const bf16x8*>(w2_src(j + 3, tid + k * THREADS));
        }
        if (j + 2 < NCH) {
#pragma unroll
          for (int k = 0; k < W2_PER_THREAD; ++k) slot((j + 2) % 3)[tid + k * THREADS] = s_cur[k];
        }
        // The reads of slot j % 3 must stay above the barrier: the next step
        // overwrites that slot (or, after the last step, the staging does).
        // Plain loads may otherwise sink past the fence.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if (j + 3 < NCH) {
#pragma unroll
          for (int k = 0; k < W2_PER_THREAD; ++k) s_cur[k] = s_next[k];
        }
      }
    }

    // ---- epilogue: one rounding of z + Y, staged through LDS so that each
    // store writes whole 16-byte-aligned runs of consecutive cells' rows.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int r = 0; r < NZR; ++r) {
#pragma unroll
        for (int tt = 0; tt < RB / 32; ++tt) {
          const int t = r * (RB / 32) + tt;
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)y[cb][t >> 1][8 * (t & 1) + e];
          *reinterpret_cast<bf16x8*>(stage + l32 * SR + 32 * tt + 16 * h) = o;
        }
        bf16x8 v[IPR];
#pragma unroll
        for (int k = 0; k < IPR; ++k)
          v[k] = *reinterpret_cast<const bf16x8*>(stage + (k * CPI + prow) * SR + pseg);
        const int64_t blk0 = cell0 + 32 * cb;
        if (blk0 + 32 <= cells) {  // every cell of the block is valid: no per-lane guards
#pragma unroll
          for (int k = 0; k < IPR; ++k)
            *reinterpret_cast<bf16x8*>(z_out + (blk0 + k * CPI + prow) * CZ + (r * RB + pseg) / 2) =
                v[k];
        } else {
#pragma unroll
          for (int k = 0; k < IPR; ++k) {
            const int64_t cell = blk0 + k * CPI + prow;
            if (cell < cells)
              *reinterpret_cast<bf16x8*>(z_out + cell * CZ + (r * RB + pseg) / 2) = v[k];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- generic path
constexpr int kGenCells = 16;
constexpr int kGenThreads = 256;
constexpr int kGenChunk = 32;
constexpr int kGenMaxAcc = kMaxCz / 16;  // features per thread at most

// Thread (cell = tid / 16, lane16 = tid % 16) accumulates features
// lane16 + 16 k of its cell. Per hidden chunk, the 16 x 32 activations are
// formed in LDS (rounded to the storage type, as the bf16 fast path does),
// then folded into the accumulators. In the fused form z = a + b is kept in
// fp32 for the residual and rounded to T where the MLP reads it.
template <typename T, bool FUSED>
__global__ __launch_bounds__(kGenThreads) void k_transition_generic(
    const T* __restrict__ z_in, const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths, int B,
    const T* __restrict__ W1,
    const T* __restrict__ W2, T* z_out, int64_t cells, int c_z, int hidden) {
  extern __shared__ float smem[];
  float* zs = smem;                       // [kGenCells][c_z]
  float* hs = smem + kGenCells * c_z;     // [kGenCells][kGenChunk]
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kGenCells;

  for (int idx = tid; idx < kGenCells * c_z; idx += kGenThreads) {
    const int cl = idx / c_z, f = idx - cl * c_z;
    const int64_t t = t0 + cl;
    float v = 0.f;
    if (t < cells) {
      if constexpr (FUSED) {
        const Cell x = decode_cell(pair_offsets, single_offsets, col_offsets, col_lengths, B, t);
        v = a[(x.eta + x.r) * c_z + f] + b[(x.mu + x.c) * c_z + f];
      } else {
        v = to_f32(z_in[t * c_z + f]);
      }
    }
    zs[idx] = v;
  }
  __syncthreads();

  const int my_cell = tid >> 4, l16 = tid & 15;
  const int nacc = c_z / 16 + ((c_z & 15) > l16 ? 1 : 0);
  float acc[kGenMaxAcc];
#pragma unroll
  for (int k = 0; k < kGenMaxAcc; ++k) acc[k] = 0.f;

  for (int h0 = 0; h0 < hidden; h0 += kGenChunk) {
    for (int p = tid; p < kGenCells * kGenChunk; p += kGenThreads) {
      const int cl = p / kGenChunk, hh = p - cl * kGenChunk;
      const int hid = h0 + hh;
      float v = 0.f;
      if (hid < hidden) {
        const float* zr = zs + cl * c_z;
        const T* wr = W1 + (int64_t)hid * c_z;
        for (int k = 0; k < c_z; ++k) v = fmaf(to_f32(from_f32<T>(zr[k])), to_f32(wr[k]), v);
        v = to_f32(from_f32<T>(fmaxf(v, 0.f)));
      }
      hs[p] = v;
    }
    __syncthreads();
    const float* hr = hs + my_cell * kGenChunk;
    const int hn = hidden - h0 < kGenChunk ? hidden - h0 : kGenChunk;
#pragma unroll
    for (int k = 0; k < kGenMaxAcc; ++k) {
      if (k < nacc) {
        const T* wr = W2 + (int64_t)(l16 + 16 * k) * hidden + h0;
        float s = acc[k];
        for (int hh = 0; hh < hn; ++hh) s = fmaf(hr[hh], to_f32(wr[hh]), s);
        acc[k] = s;
      }
    }
    __syncthreads();
  }

  const int64_t t = t0 + my_cell;
  if (t < cells) {
#pragma unroll
    for (int k = 0; k < kGenMaxAcc; ++k) {
      if (k < nacc) {
        const int f = l16 + 16 * k;
        z_out[t * c_z + f] = from_f32<T>(zs[my_cell * c_z + f] + acc[k]);
      }
    }
  }
}

template <int CZ>
hipError_t launch_mfma(const nt_partition& p, const void* z_in, const void* a, const void* b,
                       void* z_out, const void* W1, const void* W2, int hidden,
                       hipStream_t stream) {
  const int64_t blocks = (p.cells + kTileCells - 1) / kTileCells;
  if (z_in) {
    hipLaunchKernelGGL((k_transition_mfma<CZ, false>), dim3((unsigned)blocks), dim3(kWaves * 64),
                       0, stream, static_cast<const bf16*>(z_in), nullptr, nullptr,
                       p.pair_offsets, p.single_offsets, p.col_offsets, p.col_lengths, p.B,
                       static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                       static_cast<bf16*>(z_out), p.cells, hidden);
  } else {
    hipLaunchKernelGGL((k_transition_mfma<CZ, true>), dim3((unsigned)blocks), dim3(kWaves * 64),
                       0, stream, nullptr, static_cast<const float*>(a),
                       static_cast<const float*>(b), p.pair_offsets, p.single_offsets,
                       p.col_offsets, p.col_lengths,
                       p.B, static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                       static_cast<bf16*>(z_out), p.cells, hidden);
  }
  return hipGetLastError();
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int CZ, int HID>
hipError_t launch_persistent(const nt_partition& p, const void* z_in, const void* a,
                             const void* b, void* z_out, const void* W1, const void* W2,
                             hipStream_t stream) {
  const int64_t ntiles = (p.cells + kTileCells - 1) / kTileCells;
  const int64_t grid = ntiles < device_cus() ? ntiles : device_cus();
  // the LDS copy of the partition holds square partitions (mu = eta, M = N)
  const bool lds_part = p.B <= kLdsSamples && p.T <= INT32_MAX &&
                        p.col_offsets == p.single_offsets;
  if (z_in) {
    hipLaunchKernelGGL((k_transition_p32<CZ, HID, false>), dim3((unsigned)grid),
                       dim3(kWaves * 64), 0, stream, static_cast<const bf16*>(z_in), nullptr,
                       nullptr, p.pair_offsets, p.single_offsets, p.col_offsets, p.col_lengths,
                       p.B, false,
                       static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                       static_cast<bf16*>(z_out), p.cells, ntiles, p.T);
  } else {
    hipLaunchKernelGGL((k_transition_p32<CZ, HID, true>), dim3((unsigned)grid),
                       dim3(kWaves * 64), 0, stream, nullptr, static_cast<const float*>(a),
                       static_cast<const float*>(b), p.pair_offsets, p.single_offsets,
                       p.col_offsets, p.col_lengths, p.B, lds_part, static_cast<const bf16*>(W1),
                       static_cast<const bf16*>(W2), static_cast<bf16*>(z_out), p.cells, ntiles,
                       p.T);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_generic(const nt_partition& p, const void* z_in, const void* a, const void* b,
                          void* z_out, const void* W1, const void* W2, int c_z, int hidden,
                          hipStream_t stream) {
  const int64_t blocks = (p.cells + kGenCells - 1) / kGenCells;
  const size_t shmem = sizeof(float) * (size_t)kGenCells * (c_z + kGenChunk);
  if (z_in) {
    hipLaunchKernelGGL((k_transition_generic<T, false>), dim3((unsigned)blocks),
                       dim3(kGenThreads), shmem, stream, static_cast<const T*>(z_in), nullptr,
                       nullptr, p.pair_offsets, p.single_offsets, p.col_offsets, p.col_lengths, p.B,
                       static_cast<const T*>(W1), static_cast<const T*>(W2),
                       static_cast<T*>(z_out), p.cells, c_z, hidden);
  } else {
    hipLaunchKernelGGL((k_transition_generic<T, true>), dim3((unsigned)blocks), dim3(kGenThreads),
                       shmem, stream, nullptr, static_cast<const float*>(a),
                       static_cast<const float*>(b), p.pair_offsets, p.single_offsets,
                       p.col_offsets, p.col_lengths,
                       p.B, static_cast<const T*>(W1), static_cast<const T*>(W2),
                       static_cast<T*>(z_out), p.cells, c_z, hidden);
  }
  return hipGetLastError();
}

}  // namespace

int device_cu_count() { return device_cus(); }

bool transition_ws_slices_supported(const nt_partition& p, int c_z, int hidden, nt_dtype dtype,
                                    int S) {
  const int64_t t = (p.T > p.T_cols ? p.T : p.T_cols) * S;
  return dtype == NT_BF16 && c_z == 128 && hidden == 512 && p.tile_sample &&
         t <= (int64_t)(INT32_MAX / (128 * 4));
}

bool transition_has_mfma(int c_z, int hidden, nt_dtype dtype) {
  return dtype == NT_BF16 && (c_z == 64 || c_z == 128) && hidden % kChunk == 0;
}

hipError_t launch_transition(const nt_partition& p, const void* z_in, const void* a, const void* b,
                             void* z_out, const void* W1, const void* W2, int c_z, int hidden,
                             nt_dtype dtype, hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  if (transition_has_mfma(c_z, hidden, dtype)) {
    // the persistent kernel keeps single indices in 32 bits
    const bool small_t = p.T <= INT32_MAX && p.T_cols <= INT32_MAX;
    // the weight-stationary kernel addresses a and b through 32-bit buffer
    // ranges: T * 512 bytes must fit; larger batches take the persistent kernel
    const bool fits = (p.T > p.T_cols ? p.T : p.T_cols) <= (int64_t)(INT32_MAX / (128 * 4));
    if (fits && !z_in && c_z == 128 && hidden == 512 && p.tile_sample)
      return launch_transition_ws(p, a, b, z_out, W1, W2, device_cus(), stream);
    if (small_t && c_z == 128 && hidden == 512)
      return launch_persistent<128, 512>(p, z_in, a, b, z_out, W1, W2, stream);
    if (small_t && c_z == 64 && hidden == 128)
      return launch_persistent<64, 128>(p, z_in, a, b, z_out, W1, W2, stream);
    if (c_z == 128) return launch_mfma<128>(p, z_in, a, b, z_out, W1, W2, hidden, stream);
    return launch_mfma<64>(p, z_in, a, b, z_out, W1, W2, hidden, stream);
  }
  if (dtype == NT_BF16)
    return launch_generic<bf16>(p, z_in, a, b, z_out, W1, W2, c_z, hidden, stream);
  return launch_generic<float>(p, z_in, a, b, z_out, W1, W2, c_z, hidden, stream);
}

}  // namespace nt
