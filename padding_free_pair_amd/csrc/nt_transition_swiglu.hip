// Pre-normalised SwiGLU pair transition (DanLing NestedTensor, Equation 1
// second line, P~ = P + h(LN(P)); Appendix A.1: the measured update is a
// residual, pre-normalised SwiGLU of expansion four):
//   x = LN(z) = (z - mean) / sqrt(var + eps) * gamma + beta   over the c_z features
//   z_out = z + (silu(x Wg^T) * (x Wu^T)) Wd^T,               silu(g) = g / (1 + e^-g)
// over the packed cells (Section 3.3: dense work on the sum N_i^2 valid cells).
//
// bf16 storage, fp32 statistics and accumulation. Two kernels:
//  * k_swiglu32 (c_z = 128, hidden a multiple of 64, the measured shapes):
//    persistent, 32x32x16 matrix-core products in a software pipeline; its
//    own comment below gives the layout;
//  * k_transition_swiglu (c_z = 64, or hidden a multiple of 32 only): a
//    workgroup of eight waves owns 256 consecutive cells, 32 per wave as two
//    16-cell MFMA column blocks (v_mfma_f32_16x16x32_bf16); lane (l16, g)
//    holds cell 16 cb + l16, features 32 kb + 8 g .. + 7; LN by butterflies
//    over the four lanes of a cell (two passes, fp32); per 32-unit chunk the
//    gate and value products land with lane group g holding hidden units
//    8 g .. 8 g + 7 (rows permuted as in the ReLU kernels), so silu(G) * U
//    packs lane-locally into the down product's operand; the three weight
//    chunks stream through two LDS buffers.
// The residual is added to the pair state in fp32 and rounded once.
//
// Fused form (the block's, Equation 1's first two lines in one kernel): z is
// not read but formed, z = a[row] + b[col] from the fp32 projections, each
// lane decoding its cell (Equation 3 inverted, from the first sample of its
// 256-cell span of the partition's sample index); LN takes its statistics on
// that fp32 z and the residual uses it too, so the pair state is rounded
// once, on output.
#include "nt_device.hpp"
#include "nt_internal.hpp"


namespace nt {
namespace {

constexpr int kSgWaves = 8;            // two waves per SIMD
constexpr int kSgCellsPerWave = 32;
constexpr int kSgBlocks = kSgCellsPerWave / 16;
constexpr int kSgTileCells = kSgWaves * kSgCellsPerWave;
constexpr int kSgChunk = 32;

__device__ __forceinline__ f32x16 sg32_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
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

// ---------------------------------------------------------------------------
// c_z = 128, hidden a multiple of 64: the same arithmetic on the 32x32x16
// matrix cores (one 1 KiB weight fragment read from LDS per 32x32x16
// product, half the reads per flop of the 16x16x32 form above).
// Lane (l32, h) of a wave holds cell 32 cb + l32 of its cells; its x operand
// of k-step t holds features 16 t + 8 h .. + 7. Per 32-unit chunk j:
//   gate^T, up^T (32 x 32 per block) = Wg[j], Wu[j] . x^T   (k = features)
//   y^T (128 x 32 per block)        += Wd[:, j] . A^T       (k = the units)
// with the weight rows of every fragment loaded in the order of ws32_perm
// (bits 2 and 3 of the row swapped): element 8 s + e of a result is then
// unit (or feature) 16 s + 8 h + e, so silu(gate) * up packs lane-locally
// into the third product's operand and y lands in the layout of x
// (features 16 (2 fb + s) + 8 h + e of block fb). y starts from the fp32
// pair state, so the residual costs nothing at the end.
//
// Persistent: a workgroup per CU walks tiles of TILE cells. The weights
// stream through a ring of LDS buffers, chunk after chunk and across tiles
// (the chunks repeat), in a software pipeline: step j runs the gate and
// value products of chunk j + 1 beside silu of chunk j (independent, so the
// vector work issues under the matrix products), then chunk j's down
// product, in fixed issue groups that read each weight fragment two
// products before its use; it then writes the chunk staged in registers
// into the ring and loads the next one from memory.
template <int NB, int WAVES>
struct Sg32 {
  static constexpr int CZ = 128, KT = 8, FB = 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int TILE = WAVES * 32 * NB;
  static constexpr int FRAGS = 24 * 64;  // 16-byte pieces per chunk
  static constexpr int PER = FRAGS / THREADS;
  static_assert(FRAGS % THREADS == 0, "chunk staging splits evenly");
  static_assert(kSampleIndexSpan % TILE == 0, "tiles nest in the sample index");
};

__device__ __forceinline__ int ws32_perm(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

template <int NB, int WAVES, bool FUSED>
__global__ __launch_bounds__(WAVES * 64, NB == 1 ? 2 : 1) void k_swiglu32(
    const bf16* z_in, const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths,
    const int32_t* __restrict__ tile_sample, const float* __restrict__ gamma,
    const float* __restrict__ beta, const bf16* __restrict__ Wg, const bf16* __restrict__ Wu,
    const bf16* __restrict__ Wd, bf16* z_out, int64_t cells, int64_t ntiles, int hidden,
    float eps) {
  using C = Sg32<NB, WAVES>;
  constexpr int CZ = C::CZ, KT = C::KT, FB = C::FB, PER = C::PER;
  constexpr int WCELLS = 32 * NB;  // cells of one wave
  // LDS ring of weight chunks: five buffers, a chunk written three steps
  // before its first use, a barrier every other step. A buffer is rewritten
  // only after a barrier that follows its last read, and first read only
  // after a barrier that follows its write.
  constexpr int RING = 5, LEAD = 3;
  __shared__ bf16x8 wbuf[RING][C::FRAGS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int nchunks = hidden / 32;  // even, >= 2

  // ---- weight staging: piece p of chunk j is fragment p / 64, lane p % 64
  auto piece_src = [&](int j, int p) -> const bf16* {
    const int F = p >> 6, L = p & 63, r = ws32_perm(L & 31), hh = L >> 5;
    if (F < 2 * KT) {
      const bf16* W = F < KT ? Wg : Wu;
      return W + (int64_t)(32 * j + r) * CZ + 16 * (F % KT) + 8 * hh;
    }
    const int i = F - 2 * KT, fb = i >> 1, s = i & 1;
    return Wd + (int64_t)(32 * fb + r) * hidden + 32 * j + 16 * s + 8 * hh;
  };
  auto load_chunk = [&](int j, bf16x8 (&st)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      st[k] = *reinterpret_cast<const bf16x8*>(piece_src(j, tid + k * C::THREADS));
  };
  auto store_chunk = [&](int buf, const bf16x8 (&st)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k) wbuf[buf][tid + k * C::THREADS] = st[k];
  };
  // the lane's fragments of buffer b; the empty asm makes the byte offset
  // opaque, so fragment offsets stay immediates of the LDS reads instead of
  // a hoisted register per fragment
  auto lane_frags = [&](int b) -> const bf16x8* {
    int off = (b * C::FRAGS + lane) * (int)sizeof(bf16x8);
    asm volatile("" : "+v"(off));
    return reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(&wbuf[0][0]) + off);
  };

  f32x16 y[NB][FB];
  bf16x8 xb[NB][KT];
  // ---- a tile's prologue: y = z (fp32) and x = LN(z) rounded to bf16
  auto prologue = [&](int64_t tile) {
    const int64_t cell0 = tile * C::TILE + wave * WCELLS;
    // an opaque copy of the lane's cell index: the compiler recomputes the
    // z addresses per tile instead of keeping them across the tile loop
    int lz = l32;
    asm volatile("" : "+v"(lz));
    int64_t arow[NB], bcol[NB];
    if constexpr (FUSED) {
      const int i0 = tile_sample[tile * C::TILE / kSampleIndexSpan];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t c0 = cell0 + 32 * cb + l32;
        const int64_t cell = c0 < cells ? c0 : cells - 1;
        int i = i0;
        while (pair_offsets[i + 1] <= cell) ++i;
        const int64_t m = col_lengths[i], local = cell - pair_offsets[i];
        const int64_t r = local / m;
        arow[cb] = (single_offsets[i] + r) * CZ + 8 * h;
        bcol[cb] = (col_offsets[i] + (local - r * m)) * CZ + 8 * h;
      }
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      float zf[KT][8];
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        if constexpr (FUSED) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const f32x4 va = *reinterpret_cast<const f32x4*>(a + arow[cb] + 16 * t + 4 * q);
            const f32x4 vb = *reinterpret_cast<const f32x4*>(b + bcol[cb] + 16 * t + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) zf[t][4 * q + e] = va[e] + vb[e];
          }
        } else {  // a cell past the end reads the last cell; it is never stored
          const int64_t c = cell0 + 32 * cb + lz;
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(
              z_in + (c < cells ? c : cells - 1) * CZ + 16 * t + 8 * h);
#pragma unroll
          for (int e = 0; e < 8; ++e) zf[t][e] = (float)v[e];
        }
      }
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) y[cb][t >> 1][8 * (t & 1) + e] = zf[t][e];
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += zf[t][e];
      s += __shfl_xor(s, 32);
      const float mu = s * (1.f / CZ);
      float q = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = zf[t][e] - mu;
          q += d * d;
        }
      q += __shfl_xor(q, 32);
      const float rstd = 1.f / sqrtf(q * (1.f / CZ) + eps);
      // an opaque copy of the mean: z - mean is formed again below instead
      // of keeping the variance pass's 64 differences beside y
      float mu2 = mu;
      asm volatile("" : "+v"(mu2));
      // the affine pair is read per tile: an opaque offset keeps the compiler
      // from hoisting these loads out of the tile loop into 128 registers
      int ao = 8 * h;
      asm volatile("" : "+v"(ao));
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(beta + ao + 16 * t);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(beta + ao + 16 * t + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xb[cb][t][e] = (bf16)((zf[t][e] - mu2) * rstd * g0[e] + b0[e]);
          xb[cb][t][4 + e] = (bf16)((zf[t][4 + e] - mu2) * rstd * g1[e] + b1[e]);
        }
      }
    }
  };

  // gate and value products of one chunk (wb: the lane's fragments of a buffer)
  auto p12 = [&](const bf16x8* wb, f32x16 (&gt)[NB], f32x16 (&up)[NB]) {
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const bf16x8 a1 = wb[64 * t];
      const bf16x8 a2 = wb[64 * (KT + t)];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        gt[cb] = sg32_mfma(a1, xb[cb][t], t ? gt[cb] : f32x16{});
        up[cb] = sg32_mfma(a2, xb[cb][t], t ? up[cb] : f32x16{});
      }
    }
  };
  // silu(g) u = g u / (1 + e^-g), the reciprocal on v_rcp_f32 (1 ulp; the
  // product is rounded to bf16 next), packed as the down product's operand
  auto silu = [&](const f32x16 (&gt)[NB], const f32x16 (&up)[NB], bf16x8 (&af)[NB][2]) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = gt[cb][8 * s + e];
          af[cb][s][e] =
              (bf16)(g * up[cb][8 * s + e] * __builtin_amdgcn_rcpf(1.f + __expf(-g)));
        }
  };
  auto p3 = [&](const bf16x8* wb, const bf16x8 (&af)[NB][2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        const bf16x8 a3 = wb[64 * (2 * KT + 2 * fb + s)];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) y[cb][fb] = sg32_mfma(a3, af[cb][s], y[cb][fb]);
      }
  };

  // ring state at a tile's start: chunks 0 .. LEAD - 1 in buffers qb, qb + 1,
  // ... (mod RING), chunk LEAD in stg
  bf16x8 stg[PER];
#pragma unroll
  for (int c = 0; c < LEAD; ++c) {
    load_chunk(c % nchunks, stg);
    store_chunk(c, stg);
  }
  load_chunk(LEAD % nchunks, stg);
  int64_t tile = blockIdx.x;
  __syncthreads();
  int qb = 0;
  f32x16 gA[NB], uA[NB], gB[NB], uB[NB];
  // step j of the tile: chunk j + 1's gate and value products, silu and the
  // down product of chunk j, then chunk j + LEAD written and chunk
  // j + LEAD + 1 loaded; sync: this step ends at a barrier
  auto step = [&](int j, const f32x16 (&gc)[NB], const f32x16 (&uc)[NB], f32x16 (&gn)[NB],
                  f32x16 (&un)[NB], bool sync) {
    // 24 issue groups: 0..15 the gate and value products of chunk j + 1
    // (k-step i / 2, gate for even i), 16..23 chunk j's down product (k-step
    // (i - 16) / 4, feature block i % 4). Group i issues its product, the
    // LDS read of group i + 2's fragment and, in groups 0..15, silu of one
    // element of chunk j.
    const bf16x8* wn = lane_frags((qb + j + 1) % RING);
    const bf16x8* wc = lane_frags((qb + j) % RING);
    auto frag = [&](int i) -> bf16x8 {
      return i < 16 ? wn[64 * ((i & 1) * KT + (i >> 1))]
                    : wc[64 * (2 * KT + 2 * ((i - 16) & 3) + ((i - 16) >> 2))];
    };
    bf16x8 f0 = frag(0), f1 = frag(1);
    bf16x8 af[NB][2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      bf16x8 f2{};
      if (i + 2 < 24) f2 = frag(i + 2);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        if (i < 16) {
          const int t = i >> 1;
          if (i & 1)
            un[cb] = sg32_mfma(f0, xb[cb][t], t ? un[cb] : f32x16{});
          else
            gn[cb] = sg32_mfma(f0, xb[cb][t], t ? gn[cb] : f32x16{});
        } else {
          const int k = i - 16;
          y[cb][k & 3] = sg32_mfma(f0, af[cb][k >> 2], y[cb][k & 3]);
        }
      }
      if (i < 16) {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const float g = gc[cb][i];
          af[cb][i >> 3][i & 7] =
              (bf16)(g * uc[cb][i] * __builtin_amdgcn_rcpf(1.f + __expf(-g)));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      f0 = f1;
      f1 = f2;
    }
    store_chunk((qb + j + LEAD) % RING, stg);
    load_chunk((j + LEAD + 1) % nchunks, stg);
    if (sync)
      __syncthreads();
    else
      __builtin_amdgcn_sched_barrier(0);
  };
  for (; tile < ntiles; tile += gridDim.x) {
    prologue(tile);
    p12(lane_frags(qb), gA, uA);
    int j = 0;
    for (; j + 2 < nchunks; j += 2) {
      step(j, gA, uA, gB, uB, false);  // j is even
      step(j + 1, gB, uB, gA, uA, true);
    }
    step(j, gA, uA, gB, uB, false);  // j = nchunks - 2
    {
      // the last chunk's silu and down product (an odd step: a barrier);
      // the ring moves on to the next tile's chunk LEAD - 1 (its earlier
      // chunks were written by the steps above)
      bf16x8 af[NB][2];
      silu(gB, uB, af);
      p3(lane_frags((qb + j + 1) % RING), af);
      store_chunk((qb + j + 1 + LEAD) % RING, stg);
      load_chunk((j + 2 + LEAD) % nchunks, stg);
      __syncthreads();
    }
    qb = (qb + nchunks) % RING;

    // epilogue: y already holds the residual sum; one rounding, 16-byte stores
    const int64_t cell0 = tile * C::TILE + wave * WCELLS;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int64_t cell = cell0 + 32 * cb + l32;
      if (cell >= cells) continue;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)y[cb][fb][8 * s + e];
          *reinterpret_cast<bf16x8*>(z_out + cell * CZ + 16 * (2 * fb + s) + 8 * h) = o;
        }
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
  if (c_z == 128 && hidden % 64 == 0) {
    constexpr int NB = 1, WAVES = 8;  // two waves per SIMD, 32 cells each
    using C = Sg32<NB, WAVES>;
    const int64_t tiles = (p.cells + C::TILE - 1) / C::TILE;
    const int64_t cus = device_cu_count();
    const int64_t grid = tiles < cus ? tiles : cus;  // one workgroup per CU
    auto k32 = z_in ? k_swiglu32<NB, WAVES, false> : k_swiglu32<NB, WAVES, true>;
    hipLaunchKernelGGL(k32, dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                       static_cast<const bf16*>(z_in), static_cast<const float*>(a),
                       static_cast<const float*>(b), p.pair_offsets, p.single_offsets,
                       p.col_offsets, p.col_lengths, p.tile_sample, gamma, beta,
                       static_cast<const bf16*>(Wg), static_cast<const bf16*>(Wu),
                       static_cast<const bf16*>(Wd), static_cast<bf16*>(z_out), p.cells, tiles,
                       hidden, eps);
    return hipGetLastError();
  }
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
