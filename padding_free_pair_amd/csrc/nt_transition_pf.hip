// Fused broadcast + residual pair transition with the next tile's inputs
// prefetched during the current tile (DanLing NestedTensor, Equation 1 second
// line with a ReLU MLP update over the packed cells of Section 3.3; the
// broadcast z = a[row] + b[col] follows Equation 3's cell addressing).
//
// Same arithmetic as the persistent MFMA kernel (32x32x16 bf16 products
// H^T = W1 . z^T and Y^T += W2 . relu(H)^T over 32-unit hidden chunks, fp32
// accumulators seeded with the fp32 broadcast, one bf16 rounding on output),
// reorganised so that the work between two tiles no longer waits on memory:
//  * W1 and W2 both stream through a three-entry LDS ring (8 KiB per entry).
//    The stream of a tile is W1(0), W1(1), W2(0), W1(2), W2(1), ..., W2(last):
//    entry m is read during half-step m (GEMM1 half, then GEMM2 half of each
//    step) and written during half-step m - 1, one barrier per half-step.
//    Ring entries are filled from coalesced global reads (a quad of lanes
//    reads 64 contiguous bytes) and scattered into fragment order with an
//    XOR swizzle that keeps both the scattered writes and the fragment reads
//    free of bank conflicts.
//  * The 128 KiB that the resident W1 used to occupy now receives, by
//    global-to-LDS DMA during the first half of the tile, the fp32 b rows of
//    the workgroup's next tile (one 512-byte row per cell). Each DMA writes
//    two cells' rows; consecutive DMAs are placed 16 bytes further round the
//    banks so that 16 lanes reading 16 different cells hit 16 bank groups.
//    The two a rows a 32-cell block starts in ride along in registers.
//  * Between tiles a wave only rounds and stores its outputs, then forms the
//    next tile's z from LDS; the index decode of the tile after that happens
//    there too (from the tile_sample index and the partition in LDS).
#include "nt_device.hpp"
#include "nt_internal.hpp"

// The DMA below sets M0 in inline assembly; nothing else in this file uses it.
#pragma clang diagnostic ignored "-Winline-asm"

namespace nt {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTileCells = 256;
constexpr int kPfSamples = 256;       // partitions up to this many samples decode from LDS
constexpr int kPfRegion = 33280;      // bytes of DMA'd b rows per wave (64 cells + rotation)
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ f32x16 pf_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Result row rho of a 32x32 product -> row of the 32-row block it computes:
// bits 2 and 3 swapped, so that lane group h of the accumulator holds rows
// 16 s + 8 h + (0..7) in elements 8 s .. 8 s + 7, the k-group layout of the
// following product's operand. The map is its own inverse.
__device__ __forceinline__ int pf_p32(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

__device__ __forceinline__ float pf_relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Workgroup barrier for the LDS traffic of the kernel below: this wave's LDS
// operations except the N most recent have completed, then s_barrier. The
// DMA'd b rows are excluded on purpose: each wave reads only its own, after
// its own vmcnt wait, so a fence (which would wait for every DMA and weight
// load in flight) is not needed. The asm statements keep the compiler from
// moving memory accesses across.
template <int N>
__device__ __forceinline__ void pf_barrier() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Byte offset of the DMA block that holds cells x and x + 32 of a wave.
__device__ __forceinline__ int pf_block(int x) {
  return 1024 * x + 16 * (x & 15) + 256 * (x >> 4);
}

// Sample, row and column of packed cell `cell` (Equation 3 inverted),
// searching upwards from sample i0 <= the cell's sample; eta and mu are the
// row and column single offsets, m the cells per pair row (M_i).
template <typename OFF, typename IDX, typename CIDX>
__device__ __forceinline__ void pf_decode(const OFF* po, const IDX* eta, const CIDX* mu,
                                          const int32_t* m, int i0, int64_t cell, int& row,
                                          int& col) {
  int i = i0;
  while (po[i + 1] <= cell) ++i;
  const int64_t len = m[i], local = cell - (int64_t)po[i];
  int64_t r, c;
  if (len <= 65535 && local <= 0xffffffffLL) {
    const uint32_t q = (uint32_t)local / (uint32_t)len;
    r = q;
    c = (uint32_t)local - q * (uint32_t)len;
  } else {
    r = local / len;
    c = local - r * len;
  }
  row = (int)((int64_t)eta[i] + r);
  col = (int)((int64_t)mu[i] + c);
}

template <int HID>
__global__ __launch_bounds__(kPfWaves * 64, 1) void k_transition_pf(
    const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths,
    const int32_t* __restrict__ tile_sample, int B,
    bool lds_part, const bf16* __restrict__ W1, const bf16* __restrict__ W2,
    bf16* __restrict__ z_out, int64_t cells, int64_t ntiles, int64_t T) {
  constexpr int CZ = 128;
  constexpr int KT = CZ / 16;          // GEMM1 k-steps
  constexpr int FB = CZ / 32;          // GEMM2 feature blocks
  constexpr int NCH = HID / 32;        // hidden chunks
  constexpr int CB = 2;                // 32-cell blocks per wave
  constexpr int THREADS = kPfWaves * 64;
  constexpr int QP = 512;              // 16-byte pieces of one stream entry
  constexpr int QPT = QP / THREADS;
  constexpr int LASTQ = 2 * NCH;       // stream entries 0 .. LASTQ; entry LASTQ - 1 is empty
  constexpr int LA = 4;                // ring entries in flight from global memory
  // ring entry layout (see the weight stream below)
  constexpr int W1F = 1056, W1H = 528, W2F = 1088, W2H = 544;
  constexpr int QB = 8 * W2F;          // bytes of one ring entry (the larger of the two)
  static_assert(8 * W1F <= QB && W1H + 512 <= W1F && W2H + 512 <= W2F, "entry layout");
  constexpr int STAGE = 3 * QB / kPfWaves;
  // staging geometry for coalesced row access (as in the persistent kernel)
  constexpr int RB = 128, SR = RB + 16, LPR = RB / 16, CPI = 64 / LPR, IPR = 32 / CPI;
  constexpr int AROW = CZ * 4, NBR = AROW / RB, NZR = 2 * CZ / RB;
  static_assert(QP % THREADS == 0 && QPT == 2 && FB * 2 == KT && NCH >= 4, "shape");
  static_assert(32 * SR + 2 * AROW <= STAGE, "staging fits in a wave's quarter of the ring");
  static_assert(2 * NCH >= 16, "the b prefetch is spread over the first sixteen half-steps");

  __shared__ __attribute__((aligned(16))) unsigned char ring[3 * QB];
  __shared__ __attribute__((aligned(16))) unsigned char bbuf[kPfWaves * kPfRegion];
  __shared__ int64_t po_s[kPfSamples + 1];
  __shared__ int32_t eta_s[kPfSamples];
  __shared__ int32_t n_s[kPfSamples];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int prow = lane / LPR, pseg = 16 * (lane % LPR);
  unsigned char* const ringb = ring;
  unsigned char* const stage = ringb + wave * STAGE;
  unsigned char* const bwave = bbuf + wave * kPfRegion;

  // ---- weight stream: natural-order global pieces -> padded fragment order.
  // A W1 entry holds fragment t (k-step t, 64 lanes x 16 bytes) at 1056 t, its
  // lanes 32..63 528 bytes after lanes 0..31; a W2 entry holds fragment
  // i = 2 fb + s at 1088 i, lanes 32..63 544 bytes further. The pads place the
  // 16-byte pieces that one store instruction scatters (four 64-byte runs of
  // a row in the weight's natural layout) and the pieces that 16 lanes of a
  // fragment read in distinct bank groups, and make every fragment read a
  // fixed per-lane base plus an immediate offset.
  int w1_pos, w2_pos;                  // this thread's first piece; the second is a fixed step on
  {
    const int r = tid >> 4, s = tid & 15;  // W1: hidden row r of the chunk, 16-byte column s
    w1_pos = W1F * (s >> 1) + 16 * pf_p32(r) + W1H * (s & 1);
    const int f = tid >> 2, g = tid & 3;   // W2: feature row f, 16-byte column g of the chunk
    w2_pos = W2F * (2 * (f >> 5) + (g >> 1)) + 16 * pf_p32(f & 31) + W2H * (g & 1);
  }
  // second piece: W1 row r + 16 (fragment row + 16), W2 row f + 64 (fb + 2)
  constexpr int W1_STEP = 16 * 16, W2_STEP = 4 * W2F;
  const int w1_rd = 16 * l32 + W1H * h;
  const int w2_rd = 16 * l32 + W2H * h;

  // Weights and a are read through buffer descriptors: a per-thread 32-bit
  // offset plus a constant per chunk, instead of a 64-bit address per load.
  const __amdgpu_buffer_rsrc_t w1_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)W1, 0, HID * CZ * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t w2_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)W2, 0, HID * CZ * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a, 0, (int)(T * AROW), kBufferFlags);
  int w1_src = 16 * tid;                                  // W1 chunk: 8 KiB contiguous
  int w2_src = (tid >> 2) * (HID * 2) + 16 * (tid & 3);   // W2 chunk: 64 B of each row
  auto q_load = [&](int m, bf16x8 (&q)[QPT]) {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      f32x4 v;
      if (m == 0 || (m & 1)) {
        const int c = (m + 1) / 2;
        v = __builtin_amdgcn_raw_buffer_load_b128(w1_rsrc, w1_src, 8192 * c + 4096 * k, 0);
      } else {
        const int c = m / 2 - 1;
        v = __builtin_amdgcn_raw_buffer_load_b128(w2_rsrc, w2_src, 64 * c + 64 * HID * 2 * k, 0);
      }
      q[k] = __builtin_bit_cast(bf16x8, v);
    }
  };
  auto q_store = [&](int m, const bf16x8 (&q)[QPT]) {
    const bool w1 = m == 0 || (m & 1);
    unsigned char* const base = ringb + (m % 3) * QB + (w1 ? w1_pos : w2_pos);
#pragma unroll
    for (int k = 0; k < QPT; ++k)
      *reinterpret_cast<bf16x8*>(base + k * (w1 ? W1_STEP : W2_STEP)) = q[k];
  };
  auto read_w1 = [&](int m, int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(ringb + w1_rd + (m % 3) * QB + W1F * t);
  };
  auto read_w2 = [&](int m, int fb, int s) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(ringb + w2_rd + (m % 3) * QB + W2F * (2 * fb + s));
  };
  // ---- partition in LDS, decode and prefetch helpers
  if (lds_part) {
    for (int i = tid; i <= B; i += THREADS) {
      po_s[i] = pair_offsets[i];
      if (i < B) {
        eta_s[i] = (int32_t)single_offsets[i];
        n_s[i] = col_lengths[i];
      }
    }
  }
  __syncthreads();

  // lane L of a wave decodes cell L of the wave's 64 cells of `tile`
  auto decode = [&](int64_t tile, int& row, int& col) {
    int64_t cell = tile * kPfTileCells + wave * 64 + lane;
    cell = cell < cells ? cell : cells - 1;  // a cell past the end repeats the last one
    const int i0 = tile_sample[tile];
    if (lds_part)
      pf_decode(po_s, eta_s, eta_s, n_s, i0, cell, row, col);
    else
      pf_decode(pair_offsets, single_offsets, col_offsets, col_lengths, i0, cell, row, col);
  };
  // DMA block x: lanes 0..31 fetch the b row of cell x, lanes 32..63 that of
  // cell x + 32. Issued from inline assembly so that the compiler does not
  // treat every later LDS access as a possible conflict with the DMA (it
  // would wait for all memory traffic in flight before each one); the
  // kernel waits for the DMAs itself before it reads the rows. M0 carries
  // the LDS destination; one wait state separates its write from the DMA.
  const unsigned lds_b = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_ptr)bbuf) +
                         __builtin_amdgcn_readfirstlane(wave) * kPfRegion;
  auto dma_b = [&](int x, int col) {
    const int c0 = __builtin_amdgcn_readlane(col, x), c1 = __builtin_amdgcn_readlane(col, x + 32);
    const unsigned off = (unsigned)(h ? c1 : c0) * (unsigned)AROW + 16u * l32;  // < 2^31 here
    const unsigned dst = lds_b + pf_block(x);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                 :: "v"(off), "s"(dst), "s"(b) : "m0");
  };
  // the two a rows cell block cb starts in, 16 bytes per lane
  auto load_a = [&](int row, f32x4 (&araw)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      int ar = __builtin_amdgcn_readlane(row, 32 * cb) + h;
      ar = ar < T ? ar : (int)T - 1;
      araw[cb] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, ar * AROW + 16 * l32, 0, 0);
    }
  };

  int64_t tile = blockIdx.x;
  int row_n, col_n;
  f32x4 araw[CB];
  bf16x8 init[2][QPT], pend[LA][QPT];
  decode(tile, row_n, col_n);
#pragma unroll
  for (int x = 0; x < 32; ++x) dma_b(x, col_n);
  load_a(row_n, araw);
  q_load(0, init[0]);
  q_load(1, init[1]);
#pragma unroll
  for (int m = 2; m < 2 + LA; ++m) q_load(m, pend[m % LA]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first tile's b rows are in LDS

  for (;;) {
    const int64_t cell0 = tile * kPfTileCells + wave * 64;
    // ---- form z = a[row] + b[col] of this tile: y[cb][fb] element j is
    // feature 16 (2 fb + j / 8) + 8 h + j % 8, zb[cb][t] features 16 t + 8 h + 0..7.
    bf16x8 zb[CB][KT];
    f32x16 y[CB][FB];
    {
      const unsigned char* const bl = bwave + pf_block(l32) + 32 * h;
      unsigned char* const sb = stage;
      unsigned char* const sa = stage + 32 * SR;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int row_first =
            __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(row_n, 32 * cb));
        const int row_last =
            __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(row_n, 32 * cb + 31));
        const bool two_rows = row_last - row_first <= 1;
        const int xrow = __shfl_xor(row_n, 32);
        const int my_row = h == cb ? row_n : xrow;
        *reinterpret_cast<f32x4*>(sa + 16 * lane) = araw[cb];
        const unsigned char* const my_a = sa + (my_row - row_first == 1 ? AROW : 0) + 32 * h;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const f32x4 vb = *reinterpret_cast<const f32x4*>(bl + 512 * cb + 64 * t + 16 * u);
            const f32x4 vs = *reinterpret_cast<const f32x4*>(my_a + 64 * t + 16 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float zf = (two_rows ? vs[e] : 0.f) + vb[e];
              zb[cb][t][4 * u + e] = (bf16)zf;
              y[cb][t >> 1][8 * (t & 1) + 4 * u + e] = zf;
            }
          }
        }
        if (!two_rows) {  // a block of short rows: per-cell a rows, coalesced through LDS
          int src[IPR];
#pragma unroll
          for (int k = 0; k < IPR; ++k) src[k] = __shfl(row_n, 32 * cb + k * CPI + prow);
          f32x4 raw[NBR][IPR];
#pragma unroll
          for (int q = 0; q < NBR; ++q)
#pragma unroll
            for (int k = 0; k < IPR; ++k)
              raw[q][k] = *reinterpret_cast<const f32x4*>(a + (int64_t)src[k] * CZ +
                                                          (q * RB + pseg) / 4);
#pragma unroll
          for (int q = 0; q < NBR; ++q) {
#pragma unroll
            for (int k = 0; k < IPR; ++k)
              *reinterpret_cast<f32x4*>(sb + (k * CPI + prow) * SR + pseg) = raw[q][k];
#pragma unroll
            for (int mm = 0; mm < RB / 64; ++mm) {
              const int t = q * (RB / 64) + mm;
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const f32x4 va =
                    *reinterpret_cast<const f32x4*>(sb + l32 * SR + 64 * mm + 32 * h + 16 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int j = 8 * (t & 1) + 4 * u + e;
                  const float zf = y[cb][t >> 1][j] + va[e];
                  zb[cb][t][4 * u + e] = (bf16)zf;
                  y[cb][t >> 1][j] = zf;
                }
              }
            }
          }
        }
      }
    }
    const int64_t next = tile + gridDim.x;
    const bool has_next = next < ntiles;
    if (has_next) decode(next, row_n, col_n);

    // ring entries 0 and 1 once every wave is done with its staging area
    pf_barrier<0>();
    q_store(0, init[0]);
    q_store(1, init[1]);
    pf_barrier<0>();
    bf16x8 w1f[KT], w2f[FB][2];
#pragma unroll
    for (int t = 0; t < KT; ++t) w1f[t] = read_w1(0, t);

    // Half-step H writes ring entry H + 1 (loaded LA half-steps earlier)
    // into the slot that entry H - 2 occupied and issues the loads of entry
    // H + 1 + LA, right after its first MFMAs; its MFMAs then read entry H
    // into the fragment registers for half-step H + 1. The barrier closing it waits
    // only for this wave's ring write (the 8 fragment reads issued after it
    // may still be in flight): the write must be visible at half-step H + 1,
    // and the slot it overwrote was last read at H - 2, reads that every wave
    // consumed before the barrier that closed H - 1. Step j = GEMM1 of chunk
    // j (half-step 2 j + 1) then GEMM2 of chunk j - 1 (half-step 2 j + 2).
    //
    // Half-steps 1..16 also issue two DMAs each of the next tile's b rows
    // (after the last tile: this tile's rows again, into a buffer already
    // consumed, so the code stays straight-line). They go out just before
    // the half-step's weight loads: the compiler does not count them, and
    // in this order its waits for a ring entry still only cover loads at
    // least two half-steps old.
    // The work is spread over the half-step's first MFMA groups (piece 0:
    // ring write, 1 and 2: one DMA each, 3: weight loads) so that each piece
    // runs while MFMAs execute.
    auto head = [&](int H, int piece) {
      if (piece == 0) {
        if (H + 1 <= LASTQ && H + 1 != LASTQ - 1) q_store(H + 1, pend[(H + 1) % LA]);
      } else if (piece <= 2) {
        if (H <= 16) {
          // col_n looks redefined here, so the DMA addresses are formed where
          // they are used instead of all at the top of the tile
          asm volatile("" : "+v"(col_n));
          dma_b(2 * (H - 1) + piece - 1, col_n);
        }
      } else {
        if (H + 1 + LA <= LASTQ && H + 1 + LA != LASTQ - 1)
          q_load(H + 1 + LA, pend[(H + 1 + LA) % LA]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    f32x16 hacc[2][CB];
    bf16x8 hf[CB][2];
#pragma unroll
    for (int j = 0; j <= NCH; ++j) {
      if (j == NCH) {
        // every DMA of the next tile's b rows (issued in steps 0..7) and
        // every weight load of this tile has landed
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // the next tile's first stream entries and a rows (also after the
        // last tile: unconditional loads keep these registers dead across
        // the steps). The weights are the same every tile; redefining the
        // offsets stops the compiler from keeping them live across the loop.
        asm volatile("" : "+v"(w1_src), "+v"(w2_src));
        q_load(0, init[0]);
        q_load(1, init[1]);
#pragma unroll
        for (int m = 2; m < 2 + LA; ++m) q_load(m, pend[m % LA]);
        load_a(row_n, araw);
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        if (j < NCH) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            hacc[j & 1][cb] = pf_mfma(w1f[t], zb[cb][t], t == 0 ? f32x16{} : hacc[j & 1][cb]);
          // the half-step's ring write, DMAs and loads go out while the
          // first MFMAs run
          if (t < 4) head(2 * j + 1, t);
          if (j + 1 < NCH) w1f[t] = read_w1(2 * j + 1, t);
        }
        if (j > 0) {
          constexpr int PER = CB * 2 * 8 / KT;
#pragma unroll
          for (int q = 0; q < PER; ++q) {
            const int v = t * PER + q, cb = v / 16, s = (v / 8) % 2, e = v % 8;
            hf[cb][s][e] = (bf16)pf_relu(hacc[(j - 1) & 1][cb][8 * s + e]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j + 1 < NCH) pf_barrier<KT>();  // KT fragment reads follow the ring write
      else if (j + 1 == NCH) pf_barrier<0>();
      if (j > 0) {
#pragma unroll
        for (int k = 0; k < 2 * FB; ++k) {
          const int s = k / FB, fb = k % FB;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) y[cb][fb] = pf_mfma(w2f[fb][s], hf[cb][s], y[cb][fb]);
          if (k < 4 && j < NCH) head(2 * j + 2, k);
          if (j < NCH) w2f[fb][s] = read_w2(2 * j + 2, fb, s);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int piece = 0; piece < 4; ++piece) head(2, piece);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int s = 0; s < 2; ++s) w2f[fb][s] = read_w2(2, fb, s);
      }
      // after the last ring read every wave's reads must be done: the
      // epilogue stages through the ring
      if (j + 1 < NCH) pf_barrier<2 * FB>();
      else if (j + 1 == NCH) pf_barrier<0>();
    }

    // ---- epilogue: one rounding of z + Y, staged so that stores are whole rows
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
        if (blk0 + 32 <= cells) {
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
    if (!has_next) break;
    tile = next;
  }
}

}  // namespace

hipError_t launch_transition_prefetch(const nt_partition& p, const void* a, const void* b,
                                      void* z_out, const void* W1, const void* W2, int cus,
                                      hipStream_t stream) {
  const int64_t ntiles = (p.cells + kPfTileCells - 1) / kPfTileCells;
  const int64_t grid = ntiles < cus ? ntiles : cus;
  // the LDS copy of the partition holds square partitions (mu = eta, M = N)
  const bool lds_part = p.B <= kPfSamples && p.col_offsets == p.single_offsets;
  hipLaunchKernelGGL((k_transition_pf<512>), dim3((unsigned)grid), dim3(kPfWaves * 64), 0, stream,
                     static_cast<const float*>(a), static_cast<const float*>(b), p.pair_offsets,
                     p.single_offsets, p.col_offsets, p.col_lengths, p.tile_sample, p.B, lds_part,
                     static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                     static_cast<bf16*>(z_out), p.cells, ntiles, p.T);
  return hipGetLastError();
}

}  // namespace nt
