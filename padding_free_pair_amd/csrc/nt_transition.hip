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
    const int32_t* __restrict__ lengths, int B, const bf16* __restrict__ W1,
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
        const Cell x = decode_cell(pair_offsets, single_offsets, lengths, B, cell);
        arow[cb] = (int32_t)(x.eta + x.r);
        brow[cb] = (int32_t)(x.eta + x.c);
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
    const int32_t* __restrict__ lengths, int B, const T* __restrict__ W1,
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
        const Cell x = decode_cell(pair_offsets, single_offsets, lengths, B, t);
        v = a[(x.eta + x.r) * c_z + f] + b[(x.eta + x.c) * c_z + f];
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
                       p.pair_offsets, p.single_offsets, p.lengths, p.B,
                       static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                       static_cast<bf16*>(z_out), p.cells, hidden);
  } else {
    hipLaunchKernelGGL((k_transition_mfma<CZ, true>), dim3((unsigned)blocks), dim3(kWaves * 64),
                       0, stream, nullptr, static_cast<const float*>(a),
                       static_cast<const float*>(b), p.pair_offsets, p.single_offsets, p.lengths,
                       p.B, static_cast<const bf16*>(W1), static_cast<const bf16*>(W2),
                       static_cast<bf16*>(z_out), p.cells, hidden);
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
                       nullptr, p.pair_offsets, p.single_offsets, p.lengths, p.B,
                       static_cast<const T*>(W1), static_cast<const T*>(W2),
                       static_cast<T*>(z_out), p.cells, c_z, hidden);
  } else {
    hipLaunchKernelGGL((k_transition_generic<T, true>), dim3((unsigned)blocks), dim3(kGenThreads),
                       shmem, stream, nullptr, static_cast<const float*>(a),
                       static_cast<const float*>(b), p.pair_offsets, p.single_offsets, p.lengths,
                       p.B, static_cast<const T*>(W1), static_cast<const T*>(W2),
                       static_cast<T*>(z_out), p.cells, c_z, hidden);
  }
  return hipGetLastError();
}

}  // namespace

bool transition_has_mfma(int c_z, int hidden, nt_dtype dtype) {
  return dtype == NT_BF16 && (c_z == 64 || c_z == 128) && hidden % kChunk == 0;
}

hipError_t launch_transition(const nt_partition& p, const void* z_in, const void* a, const void* b,
                             void* z_out, const void* W1, const void* W2, int c_z, int hidden,
                             nt_dtype dtype, hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  if (transition_has_mfma(c_z, hidden, dtype)) {
    if (c_z == 128) return launch_mfma<128>(p, z_in, a, b, z_out, W1, W2, hidden, stream);
    return launch_mfma<64>(p, z_in, a, b, z_out, W1, W2, hidden, stream);
  }
  if (dtype == NT_BF16)
    return launch_generic<bf16>(p, z_in, a, b, z_out, W1, W2, c_z, hidden, stream);
  return launch_generic<float>(p, z_in, a, b, z_out, W1, W2, c_z, hidden, stream);
}

}  // namespace nt
