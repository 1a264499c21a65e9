// Fused gradient of the pre-normalised SwiGLU pair transition at the
// measured shape (DanLing NestedTensor, Equation 1 second line with the
// paper's update P~ = P + h(LN_{C_p}(P)), h a SwiGLU of expansion four;
// Appendix A.1), c_z = 128, hidden a multiple of 128, bf16 weights. With
//   x = LN(z) = xhat gamma + beta,  g = x Wg^T,  u = x Wu^T,  A = silu(g) u,
//   z~ = z + A Wd^T,  G = dL/dz~  (fp32),  s = sigmoid(g),
// the adjoints are
//   g_A = G Wd,  g_u = g_A silu(g),  g_g = g_A u s (1 + g (1 - s)),
//   g_x = g_u Wu + g_g Wg,  g_xhat = g_x gamma,
//   g_z = G + rstd (g_xhat - mean(g_xhat) - xhat mean(g_xhat xhat)),
//   dgamma = sum over cells of g_x xhat,  dbeta = sum of g_x,
//   dWd = G^T A,  dWu = g_u^T x,  dWg = g_g^T x  (sums over the cells).
//
// k_swiglu_bwd32 does everything per cell in one pass and leaves the three
// weight contractions to the matrix-core GEMM (launch_wgrad), on operands it
// writes: A, g_u, g_g in bf16 (the rounding the products take anyway), and x
// and G each as a bf16 pair hi + lo (hi = bf16(v), lo = bf16(v - hi)), so the
// contractions over the cells see them unrounded to about 2^-17. (Rounded to
// one bf16, x and G carry rounding errors that repeat over many cells, such
// as G's mean adjoint along a pair row, and their sums reach the percent
// level of the weight gradients.)
//
// Layout: persistent workgroups of four waves, one per SIMD (so a wave has
// the whole register file: two sets of chunk results for the software
// pipeline below), 32 cells a wave; lane (l32, h) holds cell l32 of its
// wave and, in an operand of k-step t, features 16 t + 8 h .. + 7. Per
// 32-unit chunk j:
//   g^T, u^T = Wg[j], Wu[j] . x^T,  g_A^T = WdT[j] . bf16(G)^T  (k = features)
//   g_x^T += WuT[:, j] . g_u^T + WgT[:, j] . g_g^T                (k = units)
// with every fragment's weight rows in the bits-2-and-3-swapped order, so the
// three results of a unit sit in the same lane (the adjoints are lane-local),
// g_u and g_g pack lane-locally into the last products' operands, and g_x
// lands in the layout of x (the LN adjoint is lane-local plus one exchange
// with lane l32 + 32). Step j of a tile issues chunk j + 1's three products
// beside chunk j's adjoints (independent work, so the vector instructions
// issue under the matrix products), then chunk j's g_x products. The
// chunks' 40 weight fragments stream through a ring of three LDS buffers,
// across tiles. The pair state is formed from the fp32 projections,
// z = a[row] + b[col] (Equation 3 inverted per lane), as in the forward,
// and formed again for the LN adjoint at the tile's end. The bf16 outputs
// are chunk-major (column m of row k at ((m / 32) rows + k) 32 + m % 32), so
// the two stores of a wave's chunk cover 2 KiB of contiguous memory (in the
// row-major layout each 16-byte store of a lane went to another row, and
// the line writes came out 1.4 times the bytes), and padded to whole tiles,
// so the stores need no guard (a guard inside the chunk loop splits it, and
// the compiler then waits for every outstanding memory operation at the
// join).
//
// dgamma and dbeta: each wave sums its 32 cells' terms with a
// reduce-scatter over the lanes, the waves' sums are added in wave order and
// kept per workgroup over its tiles in a fixed order; the workgroup sums are
// added in order afterwards. The grid is fixed (kSbGrid workgroups, fewer
// for small inputs), so the order, and the result, depend on the cells only.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kSbWaves = 4;  // one wave per SIMD
constexpr int kSbThreads = kSbWaves * 64;
constexpr int kSbTile = kSbWaves * 32;  // cells per tile
constexpr int kSbCz = 128, kSbKt = 8, kSbFb = 4;
constexpr int kSbFrags = 5 * kSbKt * 64;  // 16-byte pieces per chunk (40 fragments)
constexpr int kSbPer = kSbFrags / kSbThreads;
constexpr int kSbGrid = 256;
static_assert(kSampleIndexSpan % kSbTile == 0, "tiles nest in the sample index");
static_assert(kSbFrags % kSbThreads == 0, "chunk staging splits evenly");

__device__ __forceinline__ f32x16 sb_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// MFMA row rho of a 32-row block holds weight row sb_perm(rho): bits 2 and 3
// swapped, so result element 8 s + e of lane half h is row 16 s + 8 h + e.
__device__ __forceinline__ int sb_perm(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// One reduce-scatter step over the lanes l32 ^ M: of n values the lane keeps
// the half selected by its bit M and adds the partner's copy of that half.
template <int N, int M>
__device__ __forceinline__ void sb_scatter_step(float (&v)[128], int l32) {
  const bool upper = (l32 & M) != 0;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float send = upper ? v[i] : v[N / 2 + i];
    const float keep = upper ? v[N / 2 + i] : v[i];
    v[i] = keep + __shfl_xor(send, M);
  }
}

__global__ __launch_bounds__(kSbThreads, 1) void k_swiglu_bwd32(
    const float* __restrict__ a, const float* __restrict__ b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int64_t* __restrict__ col_offsets, const int32_t* __restrict__ col_lengths,
    const int32_t* __restrict__ tile_sample, const float* __restrict__ gamma,
    const float* __restrict__ beta, const bf16* __restrict__ Wg, const bf16* __restrict__ Wu,
    const bf16* __restrict__ WdT, const bf16* __restrict__ WuT, const bf16* __restrict__ WgT,
    float* G, bf16* __restrict__ X2, bf16* __restrict__ G2, bf16* __restrict__ Ab,
    bf16* __restrict__ GUb, bf16* __restrict__ GGb, float* __restrict__ lnpart, int64_t cells,
    int64_t ntiles, int hidden, float eps) {
  constexpr int CZ = kSbCz, KT = kSbKt, FB = kSbFb, PER = kSbPer;
  __shared__ bf16x8 wbuf[3][kSbFrags];
  __shared__ f32x4 red[kSbWaves][2][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int nchunks = hidden / 32;
  const int64_t rows = ntiles * kSbTile;  // rows of the chunk-major outputs

  // piece p of chunk j: fragment p / 64 (Wg, Wu, WdT by k-step; then WuT,
  // WgT by (feature block, k-step)), lane p % 64
  auto piece_src = [&](int j, int p) -> const bf16* {
    const int F = p >> 6, L = p & 63, r = sb_perm(L & 31), hh = L >> 5;
    if (F < 3 * KT) {
      const bf16* W = F < KT ? Wg : (F < 2 * KT ? Wu : WdT);
      return W + (int64_t)(32 * j + r) * CZ + 16 * (F % KT) + 8 * hh;
    }
    const int i = F - 3 * KT;
    const bf16* W = i < 2 * FB ? WuT : WgT;
    const int q = i % (2 * FB), fb = q >> 1, s = q & 1;
    return W + (int64_t)(32 * fb + r) * hidden + 32 * j + 16 * s + 8 * hh;
  };
  auto load_chunk = [&](int j, bf16x8 (&st)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      st[k] = *reinterpret_cast<const bf16x8*>(piece_src(j, tid + k * kSbThreads));
  };
  auto store_chunk = [&](int buf, const bf16x8 (&st)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k) wbuf[buf][tid + k * kSbThreads] = st[k];
  };
  // the lane's fragments of buffer bb, the byte offset opaque so fragment
  // offsets stay immediates of the LDS reads
  auto lane_frags = [&](int bb) -> const bf16x8* {
    int off = (bb * kSbFrags + lane) * (int)sizeof(bf16x8);
    asm volatile("" : "+v"(off));
    return reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(&wbuf[0][0]) + off);
  };

  bf16x8 stg[PER];
  load_chunk(0, stg);
  store_chunk(0, stg);
  load_chunk(1 % nchunks, stg);
  store_chunk(1, stg);
  load_chunk(2 % nchunks, stg);
  __syncthreads();
  int qb = 0;              // ring buffer of the tile's chunk 0
  float ln_acc = 0.f;      // thread tid < 256: entry tid of this workgroup's sums

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t c0 = tile * kSbTile + wave * 32 + l32;
    const bool live = c0 < cells;
    const int64_t cell = live ? c0 : cells - 1;  // past the end: the last cell, not stored
    int i = tile_sample[tile * kSbTile / kSampleIndexSpan];
    while (pair_offsets[i + 1] <= cell) ++i;
    const int64_t m = col_lengths[i], local = cell - pair_offsets[i];
    const int64_t r = local / m;
    const int64_t arow = (single_offsets[i] + r) * CZ + 8 * h;
    const int64_t bcol = (col_offsets[i] + (local - r * m)) * CZ + 8 * h;
    // opaque per-tile copies of the affine and row offsets (hoisted out of
    // the tile loop they would hold registers across it)
    int ao = 8 * h;
    asm volatile("" : "+v"(ao));

    // G's loads go out first, beside the gathers below: issued after LN
    // and the x stores, their latency added to the gathers'
    f32x4 gv[KT][2];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        gv[t][q] = *reinterpret_cast<const f32x4*>(G + cell * CZ + 16 * t + 8 * h + 4 * q);
    // ---- x = LN(z) (bf16 operand, and hi + lo for the weight gradients)
    bf16x8 xb[KT];
    float mu, rstd;
    {
      float zf[KT][8];
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 va = *reinterpret_cast<const f32x4*>(a + arow + 16 * t + 4 * q);
          const f32x4 vb = *reinterpret_cast<const f32x4*>(b + bcol + 16 * t + 4 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) zf[t][4 * q + e] = va[e] + vb[e];
        }
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += zf[t][e];
      s += __shfl_xor(s, 32);
      mu = s * (1.f / CZ);
      float q2 = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = zf[t][e] - mu;
          q2 += d * d;
        }
      q2 += __shfl_xor(q2, 32);
      rstd = 1.f / sqrtf(q2 * (1.f / CZ) + eps);
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(beta + ao + 16 * t);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(beta + ao + 16 * t + 4);
        bf16x8 lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (zf[t][e] - mu) * rstd * (e < 4 ? g0[e] : g1[e - 4]) +
                          (e < 4 ? b0[e] : b1[e - 4]);
          xb[t][e] = (bf16)x;
          lo[e] = (bf16)(x - (float)xb[t][e]);
        }
        *reinterpret_cast<bf16x8*>(X2 + ((t >> 1) * rows + c0) * 32 + 16 * (t & 1) + 8 * h) =
            xb[t];
        *reinterpret_cast<bf16x8*>(X2 + ((KT / 2 + (t >> 1)) * rows + c0) * 32 + 16 * (t & 1) +
                                   8 * h) = lo;
      }
    }
    // ---- G as the bf16 operand of g_A, and hi + lo for dWd
    bf16x8 gb[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      bf16x8 lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = gv[t][e >> 2][e & 3];
        gb[t][e] = (bf16)v;
        lo[e] = (bf16)(v - (float)gb[t][e]);
      }
      *reinterpret_cast<bf16x8*>(G2 + ((t >> 1) * rows + c0) * 32 + 16 * (t & 1) + 8 * h) =
          gb[t];
      *reinterpret_cast<bf16x8*>(G2 + ((KT / 2 + (t >> 1)) * rows + c0) * 32 + 16 * (t & 1) +
                                 8 * h) = lo;
    }

    // the x and G operands wait in AGPRs (the products read them there), so
    // the chunk results stay in VGPRs for the adjoints (the file is built
    // with the VGPR form of the products): 29 instead of 48 moves between
    // the two register files a chunk, 1% faster
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      asm volatile("" : "+a"(xb[t]));
      asm volatile("" : "+a"(gb[t]));
    }
    // ---- the chunks, software-pipelined (see above)
    f32x16 gx[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) gx[fb] = f32x16{};
    // chunk products: g^T, u^T (k = features of x) and g_A^T (of bf16 G)
    auto prod = [&](const bf16x8* wb, f32x16& gt, f32x16& up, f32x16& ga) {
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        gt = sb_mfma(wb[64 * t], xb[t], t ? gt : f32x16{});
        up = sb_mfma(wb[64 * (KT + t)], xb[t], t ? up : f32x16{});
        ga = sb_mfma(wb[64 * (2 * KT + t)], gb[t], t ? ga : f32x16{});
      }
    };
    // the adjoints of result element r (unit 32 j + 16 (r / 8) + 8 h + r % 8
    // of the lane's cell)
    auto adjoint = [&](int r, const f32x16& gt, const f32x16& up, const f32x16& ga,
                       bf16x8 (&av)[2], bf16x8 (&gu)[2], bf16x8 (&gg)[2]) {
      const float g = gt[r], u = up[r], gA = ga[r];
      const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-g));
      const float silu = g * sg;
      av[r >> 3][r & 7] = (bf16)(silu * u);
      gu[r >> 3][r & 7] = (bf16)(gA * silu);
      gg[r >> 3][r & 7] = (bf16)(gA * u * sg * (1.f + g * (1.f - sg)));
    };
    // step j: chunk j + 1's products, each k-step followed by two elements'
    // adjoints of chunk j (the issue order is pinned: left alone, the
    // compiler puts all of the adjoints before the products), then chunk j's
    // g_x products and its stores; then chunk j + 2 written into the buffer
    // chunk j - 1 used and chunk j + 3 loaded. Fragments are read one group
    // ahead of their products.
    auto step = [&](int j, const f32x16& gc, const f32x16& uc, const f32x16& ac, f32x16& gn,
                    f32x16& un, f32x16& an, bool next) {
      const bf16x8* wn = lane_frags((qb + j + 1) % 3);
      const bf16x8* wc = lane_frags((qb + j) % 3);
      bf16x8 av[2], gu[2], gg[2];
      bf16x8 f0{}, f1{}, f2{};
      if (next) {
        f0 = wn[0];
        f1 = wn[64 * KT];
        f2 = wn[64 * 2 * KT];
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        bf16x8 n0{}, n1{}, n2{};
        if (next && t + 1 < KT) {
          n0 = wn[64 * (t + 1)];
          n1 = wn[64 * (KT + t + 1)];
          n2 = wn[64 * (2 * KT + t + 1)];
        }
        if (next) {
          gn = sb_mfma(f0, xb[t], t ? gn : f32x16{});
          un = sb_mfma(f1, xb[t], t ? un : f32x16{});
          an = sb_mfma(f2, gb[t], t ? an : f32x16{});
        }
        adjoint(2 * t, gc, uc, ac, av, gu, gg);
        adjoint(2 * t + 1, gc, uc, ac, av, gu, gg);
        __builtin_amdgcn_sched_barrier(0);
        f0 = n0;
        f1 = n1;
        f2 = n2;
      }
      // g_x^T += WuT[:, j] g_u^T + WgT[:, j] g_g^T: fragment q = 2 fb + s of
      // each, read one product ahead
      bf16x8 pu = wc[64 * (3 * KT)], pg = wc[64 * (3 * KT + 2 * FB)];
#pragma unroll
      for (int q = 0; q < 2 * FB; ++q) {
        bf16x8 nu{}, ng{};
        if (q + 1 < 2 * FB) {
          nu = wc[64 * (3 * KT + q + 1)];
          ng = wc[64 * (3 * KT + 2 * FB + q + 1)];
        }
        gx[q >> 1] = sb_mfma(pu, gu[q & 1], gx[q >> 1]);
        gx[q >> 1] = sb_mfma(pg, gg[q & 1], gx[q >> 1]);
        if (q < 2) {
          const int64_t o = ((int64_t)j * rows + c0) * 32 + 16 * q + 8 * h;
          *reinterpret_cast<bf16x8*>(Ab + o) = av[q];
          *reinterpret_cast<bf16x8*>(GUb + o) = gu[q];
          *reinterpret_cast<bf16x8*>(GGb + o) = gg[q];
        }
        __builtin_amdgcn_sched_barrier(0);
        pu = nu;
        pg = ng;
      }
      store_chunk((qb + j + 2) % 3, stg);
      load_chunk((j + 3) % nchunks, stg);
      __syncthreads();
    };
    f32x16 gA, uA, aA, gB, uB, aB;
    prod(lane_frags(qb), gA, uA, aA);
    int j = 0;
    for (; j + 2 < nchunks; j += 2) {
      step(j, gA, uA, aA, gB, uB, aB, true);
      step(j + 1, gB, uB, aB, gA, uA, aA, true);
    }
    step(j, gA, uA, aA, gB, uB, aB, true);  // j = nchunks - 2
    // the last chunk: its adjoints and g_x products only; the ring moves on
    // to the next tile's chunk 1 (its chunk 0 was written by the step above)
    step(j + 1, gB, uB, aB, gA, uA, aA, false);
    qb = (qb + nchunks) % 3;

    // ---- LN's adjoint: element 8 (t % 2) + e of gx[t / 2] is feature 16 t + 8 h + e.
    // G (the residual) and the pair state's singles are loaded again, all at
    // once
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        gv[t][q] = *reinterpret_cast<const f32x4*>(G + cell * CZ + 16 * t + 8 * h + 4 * q);
    float xh[KT][8];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 va = *reinterpret_cast<const f32x4*>(a + arow + 16 * t + 4 * q);
        const f32x4 vb = *reinterpret_cast<const f32x4*>(b + bcol + 16 * t + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) xh[t][4 * q + e] = (va[e] + vb[e] - mu) * rstd;
      }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gxh = gx[t >> 1][8 * (t & 1) + e] * (e < 4 ? g0[e] : g1[e - 4]);
        s1 += gxh;
        s2 += gxh * xh[t][e];
      }
    }
    s1 += __shfl_xor(s1, 32);
    s2 += __shfl_xor(s2, 32);
    const float m1 = s1 * (1.f / CZ), m2 = s2 * (1.f / CZ);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + ao + 16 * t + 4);
      float* gp = G + cell * CZ + 16 * t + 8 * h;
      f32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gxh = gx[t >> 1][8 * (t & 1) + e] * (e < 4 ? g0[e] : g1[e - 4]);
        const float gz = gv[t][e >> 2][e & 3] + rstd * (gxh - m1 - xh[t][e] * m2);
        if (e < 4) o0[e] = gz; else o1[e - 4] = gz;
      }
      if (live) {
        *reinterpret_cast<f32x4*>(gp) = o0;
        *reinterpret_cast<f32x4*>(gp + 4) = o1;
      }
    }

    // ---- dgamma, dbeta terms of the wave's cells: v[8 t + e] = g_x xhat,
    // v[64 + 8 t + e] = g_x (zero past the end), summed over the 32 cells
    float v[128];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = live ? gx[t >> 1][8 * (t & 1) + e] : 0.f;
        v[8 * t + e] = gv * xh[t][e];
        v[64 + 8 * t + e] = gv;
      }
    sb_scatter_step<128, 16>(v, l32);
    sb_scatter_step<64, 8>(v, l32);
    sb_scatter_step<32, 4>(v, l32);
    sb_scatter_step<16, 2>(v, l32);
    sb_scatter_step<8, 1>(v, l32);
    // the lane now holds entries 4 l32 .. 4 l32 + 3 of its half's 128
    red[wave][h][l32] = f32x4{v[0], v[1], v[2], v[3]};
    __syncthreads();
    if (tid < 256) {
      const int hh = tid >> 7, idx = tid & 127;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kSbWaves; ++w) sum += red[w][hh][idx >> 2][idx & 3];
      ln_acc += sum;
    }
  }
  // entry (hh, idx): array idx / 64 (dgamma, dbeta), feature
  // 16 ((idx % 64) / 8) + 8 hh + idx % 8
  if (tid < 256) {
    const int hh = tid >> 7, idx = tid & 127;
    const int arr = idx >> 6, k = idx & 63;
    const int f = 16 * (k >> 3) + 8 * hh + (k & 7);
    lnpart[((int64_t)arr * gridDim.x + blockIdx.x) * CZ + f] = ln_acc;
  }
}

}  // namespace

bool swiglu_bwd32_supported(int c_z, int hidden, nt_dtype dtype) {
  // hidden a multiple of 128: the weight contractions take 128 x 128 tiles
  return dtype == NT_BF16 && c_z == kSbCz && hidden > 0 && hidden % 128 == 0;
}

int64_t swiglu_bwd32_rows(int64_t cells) {
  return (cells + kSbTile - 1) / kSbTile * kSbTile;
}

int swiglu_bwd32_grid(int64_t cells) {
  const int64_t tiles = (cells + kSbTile - 1) / kSbTile;
  return (int)(tiles < kSbGrid ? tiles : kSbGrid);
}

hipError_t launch_swiglu_bwd32(const nt_partition& p, const float* a, const float* b,
                               const float* gamma, const float* beta, const void* Wg,
                               const void* Wu, const void* WdT, const void* WuT, const void* WgT,
                               float* G, void* X2, void* G2, void* A, void* GU, void* GG,
                               float* lnpart, int hidden, float eps, hipStream_t stream) {
  if (p.cells == 0) return hipSuccess;
  const int64_t tiles = (p.cells + kSbTile - 1) / kSbTile;
  hipLaunchKernelGGL(k_swiglu_bwd32, dim3((unsigned)swiglu_bwd32_grid(p.cells)),
                     dim3(kSbThreads), 0, stream, a, b, p.pair_offsets, p.single_offsets,
                     p.col_offsets, p.col_lengths, p.tile_sample, gamma, beta,
                     static_cast<const bf16*>(Wg), static_cast<const bf16*>(Wu),
                     static_cast<const bf16*>(WdT), static_cast<const bf16*>(WuT),
                     static_cast<const bf16*>(WgT), G, static_cast<bf16*>(X2),
                     static_cast<bf16*>(G2), static_cast<bf16*>(A), static_cast<bf16*>(GU),
                     static_cast<bf16*>(GG), lnpart, p.cells, tiles, hidden, eps);
  return hipGetLastError();
}

}  // namespace nt
