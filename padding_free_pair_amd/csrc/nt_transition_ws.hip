// Weight-stationary fused broadcast + residual pair transition (DanLing
// NestedTensor, Equation 1 second line with a ReLU MLP update over the packed
// cells of Section 3.3; z = a[row] + b[col] follows Equation 3's addressing).
//
// Arithmetic: the 32x32x16 bf16 products H^T = W1 . z^T and
// Y^T += W2 . relu(H)^T with fp32 accumulators, one bf16 rounding of z as the
// first product's operand and one of the output; the residual is the fp32
// z = a + b.
//
// Organisation (c_z = 128, hidden = 512, four waves per workgroup, one
// workgroup per CU):
//  * Wave w keeps hidden units 128 w .. 128 w + 127 of both weights in its
//    accumulation registers (AGPRs) for the whole launch: their W1 rows as
//    the first product's A fragments (128 registers) and the matching W2
//    columns as the second's (128 registers). Nothing is streamed per cell.
//  * Cells move in blocks of 32 (one MFMA column block). For each block every
//    wave computes its hidden quarter and a partial Y over all 128 outputs.
//    Out block j (outputs 32 j .. 32 j + 31) belongs to wave j: the owner's
//    partial starts from the fp32 residual, the other three waves' partials
//    reach it through LDS, and the owner adds them, rounds and stores.
//  * A workgroup walks a contiguous range of blocks, one phase per block.
//    During the MFMAs of block k a wave also sums and stores block k - 1,
//    stages block k + 1 and gathers the rows of block k + 2: eight threads
//    per cell load a[row] and b[col] (64 contiguous bytes each), form z in
//    fp32 and write the bf16 operand fragments and the fp32 residual in the
//    owners' accumulator layout.
//  * With S > 1 (the non-leading layout) the rows are S slices per pair
//    cell: row R is slice R mod S of cell R / S, and its operands are
//    a[(eta_i + r) S + s] and b[(mu_i + c) S + s].
//  * LDS, double-buffered: operand fragments 2 x 8 KiB, residuals
//    2 x 16 KiB, partials 2 x 48 KiB. Two barriers per phase (the staging
//    writes at its end, the partial writes in slot 1 of the next).
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kWsWaves = 4;
constexpr int kWsCells = 32;     // cells per block
constexpr int kWsSamples = 256;  // partitions up to this many samples decode from LDS
constexpr int kWsBufFlags = 0x00020000;  // raw buffer, 32-bit data format

template <int V>
struct ws_int {
  static constexpr int value = V;
};

__device__ __forceinline__ f32x16 ws_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Result row rho of a 32x32 product -> row of the 32-row block it computes
// (bits 2 and 3 swapped). With the weight rows loaded in this order, lane
// group h of an accumulator holds rows 16 s + 8 h + (0..7) in elements
// 8 s .. 8 s + 7: the operand layout of the next product's k-step s, and
// eight consecutive outputs of one cell. The map is its own inverse.
__device__ __forceinline__ int ws_perm(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Index of workgroup g among the workgroups of its XCD, counted XCD by XCD:
// XCD x = g mod 8 holds q or q + 1 of the grid's G = 8 q + rem workgroups.
// A bijection of [0, G).
__device__ __forceinline__ int64_t ws_xcd_order(int64_t g, int64_t G) {
  const int64_t q = G / 8, rem = G % 8, x = g % 8, pos = g / 8;
  return x * q + (x < rem ? x : rem) + pos;
}

// Lane-index swizzle of the staging buffers. A staging store is issued by
// eight threads of one cell (k = 0..7) and its two neighbours' cells; with
// this key the eight stores of one cell land in eight different 16-byte bank
// groups and those of a cell pair in sixteen, while a fragment read (lane
// index XOR a constant below 16) stays a permutation of 16-lane groups.
__device__ __forceinline__ int ws_key(int k) { return k + 8 * (k & 1); }

// Eight floats rounded to bf16 (nearest-even) two at a time: one
// v_cvt_pk_bf16_f32 per pair instead of a conversion and a permute per value.
typedef float ws_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 ws_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 ws_pack8(float v0, float v1, float v2, float v3, float v4,
                                          float v5, float v6, float v7) {
  const ws_bf16x2 p0 = __builtin_convertvector((ws_f32x2){v0, v1}, ws_bf16x2);
  const ws_bf16x2 p1 = __builtin_convertvector((ws_f32x2){v2, v3}, ws_bf16x2);
  const ws_bf16x2 p2 = __builtin_convertvector((ws_f32x2){v4, v5}, ws_bf16x2);
  const ws_bf16x2 p3 = __builtin_convertvector((ws_f32x2){v6, v7}, ws_bf16x2);
  return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// This wave's LDS operations except the N most recent have completed, then
// s_barrier. Global stores and loads in flight are not waited for (nothing in
// LDS depends on them); the asm statements keep the compiler from moving
// memory accesses across.
template <int N>
__device__ __forceinline__ void ws_barrier() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Row and column single of packed cell `cell` (Equation 3 inverted),
// searching upwards from sample i0, which is at most the cell's sample.
template <typename OFF, typename IDX, typename CIDX>
__device__ __forceinline__ void ws_decode(const OFF* po, const IDX* eta, const CIDX* mu,
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

// LDS_PART: a square partition of at most kWsSamples samples with N_i <=
// 65535, decoded from an LDS copy with 32-bit arithmetic; otherwise the
// partition is read from global memory. SLICES: S > 1 (the non-leading
// layout); without it S is 1 at compile time and the row arithmetic has no
// divisions by S.
template <bool LDS_PART, bool SLICES>
__global__ __launch_bounds__(kWsWaves * 64, 1) void k_transition_ws(
    const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths,
    const int32_t* __restrict__ tile_sample, int B,
    const bf16* __restrict__ W1, const bf16* __restrict__ W2, bf16* __restrict__ z_out,
    int64_t cells, int64_t nblocks, int64_t per, int64_t T_rows, int64_t T_cols, int S_arg) {
  const int S = SLICES ? S_arg : 1;
  constexpr int CZ = 128, HID = 512;
  constexpr int KT = CZ / 16;  // first-product k-steps
  constexpr int ROW = CZ * 4;  // bytes of one fp32 single row
  // LDS: operand fragments [buf][k-step t][64 lanes] x 16 B, lane index XOR
  // ws_key(t); residuals [buf][out block j][q][64 lanes] x 16 B, lane index
  // XOR ws_key(2 j + q / 2);
  // partials [buf][writer wave][rotation slot][q][64 lanes] x 16 B.
  __shared__ __attribute__((aligned(16))) unsigned char zs[2][KT * 1024];
  __shared__ __attribute__((aligned(16))) unsigned char rs[2][4 * 4096];
  __shared__ __attribute__((aligned(16))) unsigned char ps[2][kWsWaves][3][4096];
  __shared__ int64_t po_s[kWsSamples + 1];
  __shared__ int32_t eta_s[kWsSamples];
  __shared__ int32_t n_s[kWsSamples];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  if (LDS_PART) {
    for (int i = tid; i <= B; i += kWsWaves * 64) {
      po_s[i] = pair_offsets[i];
      if (i < B) {
        eta_s[i] = (int32_t)single_offsets[i];
        n_s[i] = col_lengths[i];
      }
    }
  }

  // ---- stationary weights. Out block j of this wave is (wave + j) mod 4.
  // A wave's W1 rows are one contiguous 32 KiB run and its W2 columns 128
  // rows of 256 contiguous bytes, but a fragment takes 16 bytes from each of
  // 32 rows. So each part is fetched with whole-row loads (a wave load covers
  // four 256-byte rows), written to a wave-private LDS region with the 16-byte
  // piece index XORed by the row's low four bits, and read back in fragment
  // order; both the writes and the fragment reads are then conflict-free.
  // The region lies in the partial and residual buffers, which are not yet
  // in use; the barrier below separates it from the first staging.
  bf16x8 w1f[4][KT];    // [hidden block][k-step]
  bf16x8 w2f[4][4][2];  // [rotation j][hidden block][k-step within the block]
  {
    unsigned char* const wscr = wave < 3 ? &ps[0][0][0][0] + 32768 * wave : &rs[0][0];
    const int prow = lane >> 4, piece = lane & 15;
    auto scr = [&](int row, int pc) -> bf16x8* {
      return reinterpret_cast<bf16x8*>(wscr + 256 * row + 16 * (pc ^ (row & 15)));
    };
    const bf16* w1src = W1 + (int64_t)128 * wave * CZ;
#pragma unroll
    for (int i0 = 0; i0 < 32; i0 += 16) {
      bf16x8 tmp[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        tmp[k] = load16(w1src + (int64_t)(4 * (i0 + k) + prow) * CZ + 8 * piece).v;
#pragma unroll
      for (int k = 0; k < 16; ++k) *scr(4 * (i0 + k) + prow, piece) = tmp[k];
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int t = 0; t < KT; ++t) w1f[hb][t] = *scr(32 * hb + ws_perm(n), 2 * t + h);
    const bf16* w2src = W2 + 128 * wave;
#pragma unroll
    for (int i0 = 0; i0 < 32; i0 += 16) {
      bf16x8 tmp[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        tmp[k] = load16(w2src + (int64_t)(4 * (i0 + k) + prow) * HID + 8 * piece).v;
#pragma unroll
      for (int k = 0; k < 16; ++k) *scr(4 * (i0 + k) + prow, piece) = tmp[k];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ob = (wave + j) & 3;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          w2f[j][hb][s] = *scr(32 * ob + ws_perm(n), 4 * hb + 2 * s + h);
    }
  }
  // The products read the weights straight from accumulation registers
  // (AGPRs), which leaves the VGPRs to accumulators, operands and staging.
  // An empty asm with a tied AGPR operand places each fragment there once.
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int t = 0; t < KT; ++t) asm volatile("" : "=a"(w1f[hb][t]) : "0"(w1f[hb][t]));
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int s = 0; s < 2; ++s) asm volatile("" : "=a"(w2f[j][hb][s]) : "0"(w2f[j][hb][s]));
  __syncthreads();

  // ---- staging: thread (cell sc of the block, features 16 k8 .. 16 k8 + 15)
  const int sc = tid >> 3, k8 = tid & 7;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a, 0, (int)(T_rows * ROW), kWsBufFlags);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)b, 0, (int)(T_cols * ROW), kWsBufFlags);
  f32x4 va[2][4], vb[2][4];  // two gather sets: a block is gathered two phases ahead
  // Decode of cell `cell` of the next block, in steps spread over a phase so
  // that every memory read has several products' time to land. Step 1: the
  // first sample of the cell's 256-cell tile (a vector load, so that it does
  // not share a counter with the LDS traffic).
  const __amdgpu_buffer_rsrc_t ts_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)tile_sample, 0, (int)(4 * ((cells / S + kSampleIndexSpan - 1) / kSampleIndexSpan)),
      kWsBufFlags);
  // It is issued a phase ahead, for the block after next.
  int64_t d_cell = 0, d_p1 = 0, d_p2 = 0, d_base = 0;
  int d_i0 = 0, d_i = 0, d_len = 1, d_eta = 0, d_mu = 0, d_row = 0, d_col = 0, d_slice = 0;
  auto dec1 = [&](int64_t blk) {
    d_i0 = __builtin_amdgcn_raw_buffer_load_b32(
        ts_rsrc, (int)((blk * kWsCells / S / kSampleIndexSpan) * 4), 0, 0);
  };
  // step 2: offsets of the next two samples
  auto dec2 = [&](int64_t blk) {
    const int64_t c = blk * kWsCells + sc;
    d_cell = c < cells ? c : cells - 1;  // a row past the end repeats the last one
    if constexpr (SLICES) {  // row d_cell = slice d_slice of pair cell d_cell / S
      const int64_t pc = d_cell / S;
      d_slice = (int)(d_cell - pc * S);
      d_cell = pc;
    }
    d_i = d_i0;
    const int i2 = d_i + 2 < B ? d_i + 2 : B;
    if constexpr (LDS_PART) {
      d_p1 = po_s[d_i + 1];
      d_p2 = po_s[i2];
    } else {
      d_p1 = pair_offsets[d_i + 1];
      d_p2 = pair_offsets[i2];
    }
  };
  // step 3: the sample (at most two steps here, a walk beyond that), then its
  // length, single offsets and first cell
  auto dec3 = [&]() {
    d_i += (d_p1 <= d_cell) + (d_p2 <= d_cell);
    if (d_p2 <= d_cell) {
      if constexpr (LDS_PART) {
        while (po_s[d_i + 1] <= d_cell) ++d_i;
      } else {
        while (pair_offsets[d_i + 1] <= d_cell) ++d_i;
      }
    }
    if constexpr (LDS_PART) {
      d_len = n_s[d_i];
      d_eta = eta_s[d_i];
      d_mu = d_eta;
      d_base = po_s[d_i];
    } else {
      d_len = col_lengths[d_i];
      d_eta = (int)single_offsets[d_i];
      d_mu = (int)col_offsets[d_i];
      d_base = pair_offsets[d_i];
    }
  };
  // step 4: row and column (Equation 3 inverted)
  auto dec4 = [&]() {
    const int64_t local = d_cell - d_base;
    int64_t r, c;
    if (LDS_PART || (d_len <= 65535 && local <= 0xffffffffLL)) {
      const uint32_t q = (uint32_t)local / (uint32_t)d_len;
      r = q;
      c = (uint32_t)local - q * (uint32_t)d_len;
    } else {
      r = local / d_len;
      c = local - r * d_len;
    }
    d_row = (int)((d_eta + r) * S + d_slice);
    d_col = (int)((d_mu + c) * S + d_slice);
  };
  // step 5: the gathers (eight threads per cell, 64 contiguous bytes each)
  auto gather_a = [&](int set) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      va[set][q] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, d_row * ROW + 64 * k8 + 16 * q, 0, 0);
  };
  auto gather_b = [&](int set) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vb[set][q] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, d_col * ROW + 64 * k8 + 16 * q, 0, 0);
  };
  // z = a + b in fp32: bf16 operand fragment k8 (lanes sc and sc + 32) and
  // the fp32 residual of out block k8 / 2, rows 16 (k8 % 2) .. + 15.
  // half hh of the staging store: features 16 k8 + 8 hh .. + 7
  auto stage_half = [&](int buf, int hh, int set) {
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      z[e] = va[set][2 * hh + e / 4][e % 4] + vb[set][2 * hh + e / 4][e % 4];
    const bf16x8 o = ws_pack8(z[0], z[1], z[2], z[3], z[4], z[5], z[6], z[7]);
    *reinterpret_cast<bf16x8*>(zs[buf] + 1024 * k8 + 16 * ((sc + 32 * hh) ^ ws_key(k8))) = o;
    const int ob = k8 >> 1, s = k8 & 1;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = z[4 * qq + e];
      *reinterpret_cast<f32x4*>(rs[buf] + 4096 * ob + 1024 * (2 * s + qq) +
                                16 * ((sc + 32 * hh) ^ ws_key(k8))) = v;
    }
  };

  // ---- per-block state
  f32x16 y[4];     // partial outputs, rotation order; y[0] is this wave's own block
  f32x16 own;      // own block of the previous block (residual + this wave's partial)
  f32x16 hacc[4];  // first-product accumulators, one per hidden block
  bf16x8 hf[4][2];  // relu(H) of the four hidden blocks, two k-steps each
  bf16x8 zf[KT];
  f32x4 pr[3];
  int64_t prev = -1;

  // relu of k-step s of a first-product accumulator, packed to bf16. The
  // rounding comes first: bf16 preserves signs, so relu(bf16(x)) is
  // bf16(relu(x)) bit for bit, and the max is one packed integer op.
  auto relu_pack = [&](const f32x16& acc, int s) -> bf16x8 {
    const int b = 8 * s;
    const bf16x8 o = ws_pack8(acc[b], acc[b + 1], acc[b + 2], acc[b + 3], acc[b + 4], acc[b + 5],
                              acc[b + 6], acc[b + 7]);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = __builtin_elementwise_max(__builtin_bit_cast(s16x8, o), (s16x8){});
    return __builtin_bit_cast(bf16x8, v);
  };
  // part q (elements 4 q .. 4 q + 3) of the sum of the four partials of out
  // block `wave`: own first, then waves wave + 1, + 2, + 3 in turn
  auto read_part = [&](int pbuf, int q, int j) {
    pr[j - 1] =
        *reinterpret_cast<const f32x4*>(&ps[pbuf][(wave + j) & 3][3 - j][1024 * q + 16 * lane]);
  };
  auto add_part = [&](int q, int j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) own[4 * q + e] += pr[j - 1][e];
  };
  auto store_out = [&](int64_t blk, int s) {
    const int64_t cell = blk * kWsCells + n;
    const int b = 8 * s;
    const bf16x8 o = ws_pack8(own[b], own[b + 1], own[b + 2], own[b + 3], own[b + 4], own[b + 5],
                              own[b + 6], own[b + 7]);
    if (blk >= 0 && cell < cells)
      *reinterpret_cast<bf16x8*>(z_out + cell * CZ + 32 * wave + 16 * s + 8 * h) = o;
  };
  auto write_part = [&](int pbuf, int j, int q) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = y[j][4 * q + e];
    *reinterpret_cast<f32x4*>(&ps[pbuf][wave][j - 1][1024 * q + 16 * lane]) = v;
  };

  // blocks past the end are replaced by the last block: staged into a buffer
  // nobody reads, so that the phase body has no branches
  // Workgroup g takes the contiguous blocks [first, last): consecutive phases
  // then gather neighbouring single rows, which the caches still hold.
  // Workgroups are dispatched to the eight XCDs in turn (g mod 8); ranges are
  // numbered so that each XCD's workgroups take neighbouring ranges, and its
  // L2 serves a contiguous eighth of the pair state.
  const int64_t range = ws_xcd_order(blockIdx.x, gridDim.x);
  const int64_t first = range * per;
  const int64_t last = first + per < nblocks ? first + per : nblocks;
  auto clampb = [&](int64_t x) -> int64_t { return x < last ? x : last - 1; };
  int64_t blk = first;
  dec1(blk);
  dec2(blk);
  dec3();
  dec4();
  gather_a(0);
  gather_b(0);
  stage_half(0, 0, 0);
  stage_half(0, 1, 0);
  dec1(clampb(blk + 1));
  dec2(clampb(blk + 1));
  dec3();
  dec4();
  gather_a(1);
  gather_b(1);
  dec1(clampb(blk + 2));
  ws_barrier<0>();

  // One phase per block: 64 product slots. Slots 0..31 run the first
  // product (k-step i / 4 of hidden block i % 4, four independent chains),
  // slots 32..63 the second, two out-block chains at a time (1 and 2, then 3
  // and 0), so that the partials the other waves need are ready early. Each
  // slot carries a small share of the other work:
  //   0..22    this block's operand fragments, read four slots ahead of use
  //   1        barrier: every wave's partials of the previous block are in LDS
  //   3..25    previous block: the other waves' partials, each read four
  //            slots before it is added (and six before its buffer is reused)
  //   5..16    next block: offsets, sample, row and column, gathers
  //   20       the block after next: its tile's first sample
  //   29..32   this block's residual (own out block)
  //   27, 28   previous block: rounding and store
  //   30..42   relu of hidden blocks 0..3, two slots each
  //   44..47   next block: z = a + b into the operand and residual buffers
  //   49..56   this block: partials of out blocks 1 and 2 (block 3 follows
  //            the last product)
  // The barrier closing a phase waits for the staging writes but not for the
  // twelve partial writes; the barrier in slot 1 of the next phase does.
  // Phase P of a pair of phases (P = block parity: LDS buffer P holds this
  // block's operands, gather set P receives the block two ahead, set P ^ 1
  // holds the next block's rows). Returns whether another block follows.
  auto phase = [&](auto par) -> bool {
    constexpr int buf = decltype(par)::value;
    const int64_t next = blk + 1;
    const bool has_next = next < last;
    auto read_zf = [&](int t) {
      zf[t] = *reinterpret_cast<const bf16x8*>(zs[buf] + 1024 * t + 16 * (lane ^ ws_key(t)));
    };
    read_zf(0);
    read_zf(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i < 32) {
        const int t = i >> 2, hb = i & 3;
        hacc[hb] = ws_mfma(w1f[hb][t], zf[t], t == 0 ? f32x16{} : hacc[hb]);
      } else {
        // out blocks two at a time (1 with 2, then 3 with 0), each over
        // hidden block hb and k-step s in turn, so that the blocks the
        // other waves need finish first
        const int m = (i - 32) >> 1, hb = (m & 7) >> 1, s = m & 1;
        const int j = (i < 48 ? 1 : 3) + (i & 1) - (i >= 48 && (i & 1) ? 4 : 0);
        // y[0] starts from the residual read into it in slots 29..32
        const f32x16 c = hb > 0 || s > 0 || j == 0 ? y[j] : f32x16{};
        y[j] = ws_mfma(w2f[j][hb][s], hf[hb][s], c);
      }
      if (i >= 2 && i <= 22 && (i + 2) % 4 == 0) read_zf((i + 6) / 4);
      if (i == 1) ws_barrier<2>();
      if (i >= 29 && i <= 32) {
        const int q = i - 29;
        const f32x4 v = *reinterpret_cast<const f32x4*>(
            rs[buf] + 4096 * wave + 1024 * q + 16 * (lane ^ ws_key(2 * wave + (q >> 1))));
#pragma unroll
        for (int e = 0; e < 4; ++e) y[0][4 * q + e] = v[e];
      }
      if (i == 5) dec2(clampb(blk + 2));
      if (i == 9) dec3();
      if (i == 13) dec4();
      if (i == 15) gather_a(buf);
      if (i == 16) gather_b(buf);
      if (i == 20) dec1(clampb(blk + 3));
      if (i == 44 || i == 46) stage_half(buf ^ 1, (i - 44) / 2, buf ^ 1);
      if (i >= 2 && i <= 22 && (i - 2) % 6 < 3) read_part(buf ^ 1, (i - 2) / 6, (i - 2) % 6 + 1);
      if (i >= 6 && i <= 26 && (i - 6) % 6 < 3) add_part((i - 6) / 6, (i - 6) % 6 + 1);
      if (i == 27 || i == 28) store_out(prev, i - 27);
      if (i == 30 || i == 31) hf[0][i - 30] = relu_pack(hacc[0], i - 30);
      if (i == 33 || i == 34) hf[1][i - 33] = relu_pack(hacc[1], i - 33);
      if (i == 37 || i == 38) hf[2][i - 37] = relu_pack(hacc[2], i - 37);
      if (i == 41 || i == 42) hf[3][i - 41] = relu_pack(hacc[3], i - 41);
      if (i >= 49 && i <= 56) write_part(buf, 1 + (i - 49) / 4, (i - 49) % 4);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) write_part(buf, 3, q);
    own = y[0];
    ws_barrier<12>();
    prev = blk;
    blk = next;
    return has_next;
  };
  int buf;
  for (;;) {
    if (!phase(ws_int<0>{})) {
      buf = 0;
      break;
    }
    if (!phase(ws_int<1>{})) {
      buf = 1;
      break;
    }
  }
  ws_barrier<0>();
  // the last block's sum
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      read_part(buf, q, j);
      add_part(q, j);
    }
  store_out(prev, 0);
  store_out(prev, 1);
}

}  // namespace

hipError_t launch_transition_ws(const nt_partition& p, const void* a, const void* b, void* z_out,
                                const void* W1, const void* W2, int cus, hipStream_t stream,
                                int S) {
  const int64_t rows = p.cells * S;  // rows of c_z: S slices per pair cell
  const int64_t nblocks = (rows + kWsCells - 1) / kWsCells;
  // `per` blocks to a workgroup, and only as many workgroups as that needs,
  // so that (grid - 1) * per < nblocks: every workgroup has a block
  const int64_t per = (nblocks + cus - 1) / cus;
  const int64_t grid = (nblocks + per - 1) / per;
  // the LDS copy of the partition holds square partitions (mu = eta, M = N)
  const bool lds_part =
      p.B <= kWsSamples && p.col_offsets == p.single_offsets && p.n_max <= 65535;
  auto kern = S > 1 ? (lds_part ? k_transition_ws<true, true> : k_transition_ws<false, true>)
                    : (lds_part ? k_transition_ws<true, false> : k_transition_ws<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWsWaves * 64), 0, stream,
                     static_cast<const float*>(a), static_cast<const float*>(b), p.pair_offsets,
                     p.single_offsets, p.col_offsets, p.col_lengths, p.tile_sample, p.B,
                     static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                     static_cast<bf16*>(z_out), rows, nblocks, per, p.T * S, p.T_cols * S, S);
  return hipGetLastError();
}

}  // namespace nt
