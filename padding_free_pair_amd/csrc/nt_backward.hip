// Backward pass of the packed single-pair-single block and its loss
// (DanLing NestedTensor, arXiv 2609.30379): the sample-weighted squared loss
// of Appendix A.1, Equation 5, and the adjoints of Equation 1's steps - the
// column mean, the broadcast and the residual ReLU transition - over the
// packed cells. Section 4 measures forward, loss and backward together.
//
// Kernels here are the HBM-bound adjoints and the generic (any width, fp32
// or bf16) forms of the transition's gradient; the MFMA forms of the
// transition's gradient live in nt_transition_bwd.hip.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Adjoint of the column mean: every cell of pair row r receives
// g_m[r] / M_i, plus the incoming gradient of the pair state when there is
// one. The row's cells are row_splits[r] .. row_splits[r + 1], so M_i is
// their count and no sample lookup is needed. One workgroup per row.
__global__ __launch_bounds__(kThreads) void k_mean_backward(
    const float* __restrict__ g_m, const float* g_in, float* G,
    const int64_t* __restrict__ row_splits, int64_t T_rows, int c_z) {
  const int q4 = c_z / 4;             // float4s per cell
  const int cpp = kThreads / q4;      // cells per pass (c_z <= 512: at least 2)
  const int tc = threadIdx.x / q4, f = 4 * (threadIdx.x % q4);
  if (tc >= cpp) return;
  for (int64_t r = blockIdx.x; r < T_rows; r += gridDim.x) {
    const int64_t c0 = row_splits[r], n = row_splits[r + 1] - c0;
    if (n == 0) continue;
    const float nf = (float)n;
    const f32x4 gm = *reinterpret_cast<const f32x4*>(g_m + r * c_z + f);
    f32x4 d;
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = gm[e] / nf;
    for (int64_t c = tc; c < n; c += cpp) {
      const int64_t off = (c0 + c) * c_z + f;
      f32x4 v = d;
      if (g_in) {
        const f32x4 gi = *reinterpret_cast<const f32x4*>(g_in + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = d[e] + gi[e];
      }
      *reinterpret_cast<f32x4*>(G + off) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Column adjoint of the broadcast: g_b[mu_i + c] = sum_r g_z[o_i + r M_i + c].
// A pair row of sample i is M_i c_z contiguous floats, and float4 q of it is
// float4 q of g_b's block for the sample, so each thread sums one float4
// position down the sample's N_i rows, in row order. A column is a long
// dependent walk and there are few of them, so each thread keeps
// kColUnroll rows' loads in flight (with four, the whole grid held about
// 4 MB in flight and read at about 3 TB/s). STREAM: nontemporal loads, for
// a g_z above the last-level cache (long_square_x4: row and column sums
// 301 -> 287 us; on high_variation_x4's 208 MB, which fits, 10% slower).
constexpr int kColUnroll = 16;

template <bool STREAM>
__device__ __forceinline__ f32x4 load_col4(const float* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return *reinterpret_cast<const f32x4*>(p);
}

template <bool STREAM>
__global__ __launch_bounds__(kThreads) void k_col_sums(
    const float* __restrict__ g_z, float* __restrict__ g_b,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ col_offsets,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ col_lengths, int per_sample,
    int c_z) {
  const int i = blockIdx.x / per_sample, part = blockIdx.x % per_sample;
  const int64_t N = lengths[i], M = col_lengths[i];
  const int64_t width = M * c_z / 4;
  const int64_t step = (int64_t)M * c_z;  // floats between rows
  const float* base = g_z + pair_offsets[i] * c_z;
  float* dst = g_b + col_offsets[i] * c_z;
  for (int64_t q = (int64_t)part * kThreads + threadIdx.x; q < width;
       q += (int64_t)per_sample * kThreads) {
    const float* src = base + 4 * q;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    int64_t r = 0;
    for (; r + kColUnroll <= N; r += kColUnroll) {
      f32x4 v[kColUnroll];
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u)
        v[u] = load_col4<STREAM>(src + (r + u) * step);
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[u][e];
    }
    for (; r < N; ++r) {
      const f32x4 v = load_col4<STREAM>(src + r * step);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    *reinterpret_cast<f32x4*>(dst + 4 * q) = acc;
  }
}

// ---------------------------------------------------------------------------
// Equation 5, one workgroup per single row r (sample i = row_sample[r]): the
// squares of x[r] and of the cells of pair row r, summed in fp32 lanes and
// an fp32 tree, weighted by alpha_i / d1 and beta_i / d2 into partial[r]
// (fp64); the gradients 2 alpha_i x / d1 and 2 beta_i pz / d2 in fp32.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

constexpr int kLossUnroll = 4;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_loss_rows(
    const T* __restrict__ x, int c_s, const T* __restrict__ pz, int c_z,
    const int64_t* __restrict__ row_splits, const int32_t* __restrict__ row_sample, int B,
    int64_t T_rows, double inv_d1, double inv_d2, double* __restrict__ partial,
    float* __restrict__ g_x, float* __restrict__ g_pz) {
  constexpr int VEC = Vec16<T>::N;
  __shared__ float red[kThreads / 64];
  for (int64_t r = blockIdx.x; r < T_rows; r += gridDim.x) {
    const int i = row_sample[r];
    const double alpha = 1.0 + (double)i / B, beta = 1.5 - (double)i / (2.0 * B);
    const float gxs = (float)(2.0 * alpha * inv_d1), gps = (float)(2.0 * beta * inv_d2);
    float sx = 0.f, sp = 0.f;
    for (int f = threadIdx.x * VEC; f < c_s; f += kThreads * VEC) {
      const Vec16<T> v = load16(x + r * c_s + f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float xv = v.get(e);
        sx += xv * xv;
        if (g_x) g_x[r * c_s + f + e] = gxs * xv;
      }
    }
    // the pair row's vectors, kLossUnroll loads in flight per thread; each
    // thread still adds its squares in element order
    const int64_t e0 = row_splits[r] * c_z, e1 = row_splits[r + 1] * c_z;
    constexpr int64_t step = (int64_t)kThreads * VEC;
    auto use = [&](const Vec16<T>& v, int64_t e) {
      float g[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float pv = v.get(k);
        sp += pv * pv;
        g[k] = gps * pv;
      }
      if (g_pz) {
#pragma unroll
        for (int k = 0; k < VEC; k += 4)
          *reinterpret_cast<f32x4*>(g_pz + e + k) = f32x4{g[k], g[k + 1], g[k + 2], g[k + 3]};
      }
    };
    int64_t e = e0 + (int64_t)threadIdx.x * VEC;
    for (; e + (kLossUnroll - 1) * step < e1; e += kLossUnroll * step) {
      Vec16<T> v[kLossUnroll];
#pragma unroll
      for (int u = 0; u < kLossUnroll; ++u) v[u] = load16(pz + e + u * step);
#pragma unroll
      for (int u = 0; u < kLossUnroll; ++u) use(v[u], e + u * step);
    }
    for (; e < e1; e += step) use(load16(pz + e), e);
    sx = block_sum(sx, red);
    sp = block_sum(sp, red);
    if (threadIdx.x == 0) partial[r] = alpha * (double)sx * inv_d1 + beta * (double)sp * inv_d2;
  }
}

// Sum of the per-row terms in fp64, one workgroup, fixed order.
__global__ __launch_bounds__(kThreads) void k_loss_final(const double* __restrict__ partial,
                                                         int64_t n, double* __restrict__ loss) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < n; k += kThreads) s += partial[k];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = red[0];
}

// ---------------------------------------------------------------------------
// dst [C, R] = src [R, C]^T through a 32 x 33 LDS tile (weights only).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_transpose(const T* __restrict__ src,
                                                        T* __restrict__ dst, int R, int C) {
  __shared__ T tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  for (int k = ty; k < 32; k += 8) {
    const int r = r0 + k, c = c0 + tx;
    if (r < R && c < C) tile[k][tx] = src[(int64_t)r * C + c];
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k, r = r0 + tx;
    if (r < R && c < C) dst[(int64_t)c * R + r] = tile[tx][k];
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient contraction over rows: C[m, n] = sum_k A[k, m] B[k, n],
// A [K, M] and B [K, N] row-major (bf16 inputs widened), fp32 products and
// accumulation on v_mfma_f32_32x32x2_f32, whose operands hold one k per
// lane: lane (l % 32, l / 32) takes A[k + l / 32][m0 + l % 32], so the loads
// of a K-major operand stay coalesced. Each workgroup owns a 32 x 32 tile of
// C and one of `gridDim.z` slices of K (a multiple of 32 rows); its four
// waves take interleaved pairs of rows and add their tiles through LDS; the
// partial tile is written and k_sum_splits adds the slices in order.
template <typename TA, typename TB>
__global__ __launch_bounds__(kThreads) void k_gemm_tn(const TA* __restrict__ A,
                                                      const TB* __restrict__ Bm,
                                                      float* __restrict__ part, int64_t K, int M,
                                                      int N, int64_t kchunk) {
  __shared__ float red[kThreads / 64][32 * 33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int64_t kb = (int64_t)blockIdx.z * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
  const int m = m0 + l32, n = n0 + l32;
  const bool mok = m < M, nok = n < N;
  f32x16 acc = f32x16{};
  // wave w takes the row pairs kb + 2 w + 8 u (u = 0, 1, ...), lane half h row + h
  for (int64_t k0 = kb + 2 * wave; k0 < ke; k0 += 32) {
    float av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t k = k0 + 8 * u + h;
      const bool kin = k < ke;
      av[u] = (kin && mok) ? to_f32(A[k * M + m]) : 0.f;
      bv[u] = (kin && nok) ? to_f32(Bm[k * N + n]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], acc, 0, 0, 0);
  }
  // element r of the tile: row 8 (r / 4) + 4 h + r % 4, column l32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][(8 * (r / 4) + 4 * h + r % 4) * 33 + l32] = acc[r];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + kThreads * q, row = idx >> 5, col = idx & 31;
    const float v = red[0][row * 33 + col] + red[1][row * 33 + col] + red[2][row * 33 + col] +
                    red[3][row * 33 + col];
    if (m0 + row < M && n0 + col < N)
      part[((int64_t)blockIdx.z * M + m0 + row) * N + n0 + col] = v;
  }
}

__global__ __launch_bounds__(kThreads) void k_sum_splits(const float* __restrict__ part,
                                                         float* __restrict__ C, int S,
                                                         int64_t MN) {
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < MN;
       idx += (int64_t)gridDim.x * kThreads) {
    float s = 0.f;
    for (int z = 0; z < S; ++z) s += part[(int64_t)z * MN + idx];
    C[idx] = s;
  }
}

// The same sum, four outputs a thread (MN a multiple of 4, 16-byte aligned),
// eight slices' loads in flight, added in slice order.
__global__ __launch_bounds__(64) void k_sum_splits4(const f32x4* __restrict__ part,
                                                    f32x4* __restrict__ C, int S, int64_t MN4) {
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (idx >= MN4) return;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  int z = 0;
  for (; z + 8 <= S; z += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(z + u) * MN4 + idx];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[u][e];
  }
  for (; z < S; ++z) {
    const f32x4 v = part[(int64_t)z * MN4 + idx];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  C[idx] = acc;
}

// ---------------------------------------------------------------------------
// Transition gradient, any width, one workgroup per cell (grid-stride):
//   pre = z W1^T; H = relu(pre); g_H = (G W2) * [pre > 0];
//   g_z = G + g_H W1.
// With bf16 storage the products read G and g_H rounded to bf16 (as the
// matrix-core form does). H, g_H and G are stored for the weight
// gradients dW2 = Gb^T H and dW1 = g_H^T z, Gb holding G in the storage
// type (dW2 runs after g_z may have overwritten G). g_z may alias G: a cell's
// G is read into LDS before its g_z is written. g_H is read back from GH
// after the barrier, so LDS stays 3 c_z floats.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_transition_backward_generic(
    const T* __restrict__ z, const float* G, const T* __restrict__ W1, const T* __restrict__ W2,
    float* g_z, T* __restrict__ H, T* __restrict__ GH, T* __restrict__ Gb, int64_t cells,
    int c_z, int hid) {
  extern __shared__ float sm[];
  float* zs = sm;
  float* gs = zs + c_z;
  float* gq = gs + c_z;
  const int tid = threadIdx.x;
  for (int64_t cell = blockIdx.x; cell < cells; cell += gridDim.x) {
    for (int f = tid; f < c_z; f += kThreads) {
      zs[f] = to_f32(z[cell * c_z + f]);
      const float g = G[cell * c_z + f];
      gs[f] = g;
      const T gt = from_f32<T>(g);
      gq[f] = to_f32(gt);
      if (Gb) Gb[cell * c_z + f] = gt;
    }
    __syncthreads();
    for (int u = tid; u < hid; u += kThreads) {
      float pre = 0.f, gh = 0.f;
      for (int f = 0; f < c_z; ++f) {
        pre += zs[f] * to_f32(W1[(int64_t)u * c_z + f]);
        gh += gq[f] * to_f32(W2[(int64_t)f * hid + u]);
      }
      H[cell * hid + u] = from_f32<T>(pre > 0.f ? pre : 0.f);
      GH[cell * hid + u] = from_f32<T>(pre > 0.f ? gh : 0.f);
    }
    __syncthreads();  // this cell's GH row is visible to the workgroup
    for (int f = tid; f < c_z; f += kThreads) {
      float acc = gs[f];
      for (int u = 0; u < hid; ++u)
        acc += to_f32(GH[cell * hid + u]) * to_f32(W1[(int64_t)u * c_z + f]);
      g_z[cell * c_z + f] = acc;
    }
    __syncthreads();
  }
}

template <typename T>
hipError_t launch_loss_t(const nt_partition& p, const void* x, int c_s, const void* pz, int c_z,
                         double inv_d1, double inv_d2, double* partial, float* g_x, float* g_pz,
                         hipStream_t s) {
  const int64_t grid = p.T < 65536 ? p.T : 65536;
  hipLaunchKernelGGL((k_loss_rows<T>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     static_cast<const T*>(x), c_s, static_cast<const T*>(pz), c_z, p.row_splits,
                     p.row_sample, p.B, p.T, inv_d1, inv_d2, partial, g_x, g_pz);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Both adjoints of the broadcast from one read of g_z (square partitions of
// at most kAdjSamples samples): g_a[eta_i + r] = sum_c g_z[o_i + r N_i + c]
// and g_b[eta_i + c] = sum_r g_z[o_i + r N_i + c]. A workgroup takes a tile
// of kAdjR rows x C columns of one sample (C = kAdjKC columns per thread);
// thread (f, cl) owns float4 f of columns c0 + cl + cpp u. Each tile writes
// its row sums to prow[column tile][row] and its column sums to
// pcol[row tile][column]; k_adj_sum then adds a row's (column's) tiles in
// tile order, so results are deterministic.
constexpr int kAdjSamples = 256;
constexpr int kAdjR = 16;   // rows of a tile
constexpr int kAdjKC = 16;  // columns of a tile per thread

template <bool STREAM>
__global__ __launch_bounds__(kThreads) void k_bcast_adj(
    const float* __restrict__ g_z, float* __restrict__ prow, float* __restrict__ pcol,
    const int64_t* __restrict__ pair_offsets, const int64_t* __restrict__ single_offsets,
    const int32_t* __restrict__ lengths, int B, int W, int64_t T) {
  __shared__ int64_t tile_end[kAdjSamples];  // inclusive prefix of tiles per sample
  __shared__ int64_t wave_sum[kThreads / 64];
  __shared__ f32x4 rsum[kAdjR][kThreads];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = W / 4, cpp = kThreads / q4, C = cpp * kAdjKC;
  int64_t v = 0;
  if (tid < B) {
    const int64_t n = lengths[tid];
    v = ((n + kAdjR - 1) / kAdjR) * ((n + C - 1) / C);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wave_sum[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += wave_sum[w];
  tile_end[tid] = v;
  __syncthreads();
  const int64_t g = blockIdx.x;
  if (B == 0 || g >= tile_end[B - 1]) return;  // the grid is an upper bound
  int lo = 0, hi = B - 1;  // first sample with tile_end > g
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tile_end[mid] > g) hi = mid; else lo = mid + 1;
  }
  const int i = lo;
  const int64_t local = g - (i > 0 ? tile_end[i - 1] : 0);
  const int64_t n = lengths[i], nct = (n + C - 1) / C;
  const int64_t rt = local / nct, ct = local - rt * nct;
  const int64_t r0 = rt * kAdjR, c0 = ct * C;
  const int f = tid % q4, cl = tid / q4;
  const bool act = cl < cpp;
  const int64_t eta = single_offsets[i], o = pair_offsets[i];
  f32x4 colp[kAdjKC];
#pragma unroll
  for (int u = 0; u < kAdjKC; ++u) colp[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kAdjR; ++k) {
    const int64_t r = r0 + k;
    f32x4 rs = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r < n && act) {
      const float* row = g_z + (o + r * n) * W + 4 * f;
      f32x4 x[kAdjKC];
#pragma unroll
      for (int u = 0; u < kAdjKC; ++u) {
        const int64_t c = c0 + cl + (int64_t)cpp * u;
        x[u] = c < n ? load_col4<STREAM>(row + c * W) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kAdjKC; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          colp[u][e] += x[u][e];
          rs[e] += x[u][e];
        }
    }
    rsum[k][tid] = rs;
  }
  __syncthreads();
  // the tile's row sums: row k, float4 ff, over the cpp column lanes in order
  for (int idx = tid; idx < kAdjR * q4; idx += kThreads) {
    const int k = idx / q4, ff = idx - k * q4;
    const int64_t r = r0 + k;
    if (r >= n) continue;
    f32x4 sum = rsum[k][ff];
    for (int c2 = 1; c2 < cpp; ++c2) {
      const f32x4 t = rsum[k][c2 * q4 + ff];
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += t[e];
    }
    *reinterpret_cast<f32x4*>(prow + ((int64_t)ct * T + eta + r) * W + 4 * ff) = sum;
  }
  if (act) {
#pragma unroll
    for (int u = 0; u < kAdjKC; ++u) {
      const int64_t c = c0 + cl + (int64_t)cpp * u;
      if (c < n) *reinterpret_cast<f32x4*>(pcol + ((int64_t)rt * T + eta + c) * W + 4 * f) = colp[u];
    }
  }
}

// out[x] = sum over the ceil(n / span) tiles t of part[t][x] in tile order, for
// every row (column) x of T; n is the length of x's sample.
__global__ __launch_bounds__(kThreads) void k_adj_sum(const float* __restrict__ part,
                                                      float* __restrict__ out,
                                                      const int32_t* __restrict__ row_sample,
                                                      const int32_t* __restrict__ lengths,
                                                      int64_t T, int W, int span) {
  const int q4 = W / 4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= T * q4) return;
  const int64_t x = idx / q4;
  const int f = (int)(idx - x * q4);
  const int64_t n = lengths[row_sample[x]], cnt = (n + span - 1) / span;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t t = 0; t < cnt; ++t) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (t * T + x) * W + 4 * f);
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] += v[e];
  }
  *reinterpret_cast<f32x4*>(out + x * W + 4 * f) = sum;
}

}  // namespace

hipError_t launch_mean_backward(const nt_partition& p, const float* g_m, const float* g_in,
                                float* G, int c_z, hipStream_t s) {
  if (p.T == 0 || p.cells == 0) return hipSuccess;
  const int64_t grid = p.T < 65536 ? p.T : 65536;
  hipLaunchKernelGGL(k_mean_backward, dim3((unsigned)grid), dim3(kThreads), 0, s, g_m, g_in, G,
                     p.row_splits, p.T, c_z);
  return hipGetLastError();
}

hipError_t launch_col_sums(const nt_partition& p, const float* g_z, float* g_b, int c_z,
                           hipStream_t s) {
  if (p.T_cols == 0 || p.B == 0) return hipSuccess;
  // a workgroup covers 256 float4s of a row; samples take at most 128 of them
  const int64_t widest = (p.col_offsets == p.single_offsets ? (int64_t)p.n_max : p.T_cols);
  int64_t per = (widest * c_z / 4 + kThreads - 1) / kThreads;
  per = per < 1 ? 1 : (per > 128 ? 128 : per);
  const bool stream_g = p.cells * c_z * (int64_t)sizeof(float) > kStreamBytes;
  hipLaunchKernelGGL(stream_g ? k_col_sums<true> : k_col_sums<false>, dim3((unsigned)(p.B * per)),
                     dim3(kThreads), 0, s, g_z, g_b,
                     p.pair_offsets, p.col_offsets, p.lengths, p.col_lengths, (int)per, c_z);
  return hipGetLastError();
}

bool bcast_adj_fused(const nt_partition& p, int W) {
  return p.col_offsets == p.single_offsets && p.B <= kAdjSamples && W % 4 == 0 && W / 4 <= kThreads;
}

size_t bcast_adj_ws_bytes(const nt_partition& p, int W) {
  if (!bcast_adj_fused(p, W)) return 0;
  const int64_t C = (int64_t)(kThreads / (W / 4)) * kAdjKC;
  const int64_t CT = (p.n_max + C - 1) / C, RT = ((int64_t)p.n_max + kAdjR - 1) / kAdjR;
  return (size_t)(CT + RT) * p.T * W * sizeof(float);
}

hipError_t launch_bcast_adj(const nt_partition& p, const float* g_z, float* g_a, float* g_b,
                            int W, float* ws, hipStream_t s) {
  if (!bcast_adj_fused(p, W)) {
    hipError_t e = launch_reduce(p, g_z, g_a, W, NT_F32, s, false);
    return e != hipSuccess ? e : launch_col_sums(p, g_z, g_b, W, s);
  }
  if (p.T == 0) return hipSuccess;
  const int64_t C = (int64_t)(kThreads / (W / 4)) * kAdjKC;
  const int64_t CT = (p.n_max + C - 1) / C;
  float* prow = ws;
  float* pcol = ws + CT * p.T * W;
  // an upper bound of the tiles, sum ceil(N_i / R) ceil(N_i / C) <=
  // sum (N_i / R + 1)(N_i / C + 1); workgroups past the last tile return at once
  const int64_t tiles = (p.cells + kAdjR * C - 1) / (kAdjR * C) + (p.T + kAdjR - 1) / kAdjR +
                        (p.T + C - 1) / C + p.B;
  const bool stream_g = p.cells * W * (int64_t)sizeof(float) > kStreamBytes;
  hipLaunchKernelGGL(stream_g ? k_bcast_adj<true> : k_bcast_adj<false>, dim3((unsigned)tiles),
                     dim3(kThreads), 0, s, g_z, prow, pcol, p.pair_offsets, p.single_offsets,
                     p.lengths, p.B, W, p.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = p.T * (W / 4);
  const dim3 grid((unsigned)((n4 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(k_adj_sum, grid, dim3(kThreads), 0, s, prow, g_a, p.row_sample, p.lengths,
                     p.T, W, (int)C);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_adj_sum, grid, dim3(kThreads), 0, s, pcol, g_b, p.row_sample, p.lengths,
                     p.T, W, kAdjR);
  return hipGetLastError();
}

hipError_t launch_loss_eq5(const nt_partition& p, const void* x, int c_s, const void* pz, int c_z,
                           int S, nt_dtype dtype, double* partial, double* loss, float* g_x,
                           float* g_pz, hipStream_t s) {
  // rows hold S slices of c_s (c_z) values: the divisors count every value
  const double d1 = (double)S * c_s * (double)p.T;
  const double d2 = (double)S * c_z * (double)p.cells;
  const double inv_d1 = d1 > 0 ? 1.0 / d1 : 0.0, inv_d2 = d2 > 0 ? 1.0 / d2 : 0.0;
  if (p.T > 0) {
    hipError_t e = dtype == NT_BF16
                       ? launch_loss_t<bf16>(p, x, S * c_s, pz, S * c_z, inv_d1, inv_d2, partial,
                                             g_x, g_pz, s)
                       : launch_loss_t<float>(p, x, S * c_s, pz, S * c_z, inv_d1, inv_d2, partial,
                                              g_x, g_pz, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(kThreads), 0, s, partial, p.T, loss);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int R, int C, nt_dtype dtype,
                            hipStream_t s) {
  const dim3 grid((unsigned)((C + 31) / 32), (unsigned)((R + 31) / 32));
  if (dtype == NT_BF16)
    hipLaunchKernelGGL(k_transpose<bf16>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16*>(src), static_cast<bf16*>(dst), R, C);
  else
    hipLaunchKernelGGL(k_transpose<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(src), static_cast<float*>(dst), R, C);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, float* C, int S, int64_t MN, hipStream_t s) {
  if (MN % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(C) % 16 == 0) {
    const int64_t MN4 = MN / 4;
    hipLaunchKernelGGL(k_sum_splits4, dim3((unsigned)((MN4 + 63) / 64)), dim3(64), 0, s,
                       reinterpret_cast<const f32x4*>(part), reinterpret_cast<f32x4*>(C), S,
                       MN4);
    return hipGetLastError();
  }
  int64_t g = (MN + kThreads - 1) / kThreads;
  g = g > 4096 ? 4096 : (g < 1 ? 1 : g);
  hipLaunchKernelGGL(k_sum_splits, dim3((unsigned)g), dim3(kThreads), 0, s, part, C, S, MN);
  return hipGetLastError();
}

int gemm_tn_splits(int64_t K, int M, int N) {
  const int64_t tiles = (int64_t)((M + 31) / 32) * ((N + 31) / 32);
  int64_t S = (1024 + tiles - 1) / tiles;         // about 1024 workgroups
  const int64_t kmax = (K + 255) / 256;           // at least 256 rows a slice
  if (S > kmax) S = kmax;
  if (S > 256) S = 256;
  return (int)(S < 1 ? 1 : S);
}

hipError_t launch_gemm_tn(const void* A, nt_dtype a_dtype, const void* B, nt_dtype b_dtype,
                          float* C, float* partial, int64_t K, int M, int N, int splits,
                          hipStream_t s) {
  const int64_t MN = (int64_t)M * N;
  int64_t g = (MN + kThreads - 1) / kThreads;
  g = g > 4096 ? 4096 : g;
  if (K == 0) {  // no rows: C = 0 (a sum over no slices; a kernel, not a memset)
    hipLaunchKernelGGL(k_sum_splits, dim3((unsigned)g), dim3(kThreads), 0, s, partial, C, 0, MN);
    return hipGetLastError();
  }
  const int64_t kchunk = ((K + splits - 1) / splits + 31) / 32 * 32;
  const int S = (int)((K + kchunk - 1) / kchunk);
  const dim3 grid((unsigned)((M + 31) / 32), (unsigned)((N + 31) / 32), (unsigned)S);
#define NT_TN(TA, TB)                                                                        \
  hipLaunchKernelGGL((k_gemm_tn<TA, TB>), grid, dim3(kThreads), 0, s,                       \
                     static_cast<const TA*>(A), static_cast<const TB*>(B), partial, K, M, N, \
                     kchunk)
  if (a_dtype == NT_BF16 && b_dtype == NT_BF16) NT_TN(bf16, bf16);
  else if (a_dtype == NT_BF16) NT_TN(bf16, float);
  else if (b_dtype == NT_BF16) NT_TN(float, bf16);
  else NT_TN(float, float);
#undef NT_TN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum_splits, dim3((unsigned)g), dim3(kThreads), 0, s, partial, C, S, MN);
  return hipGetLastError();
}

hipError_t launch_transition_backward_generic(const nt_partition& p, const void* z,
                                              const float* G, const void* W1, const void* W2,
                                              float* g_z, void* H, void* GH, void* Gb, int c_z,
                                              int hidden, nt_dtype dtype, hipStream_t s) {
  if (p.cells == 0) return hipSuccess;
  const int64_t grid = p.cells < 65536 ? p.cells : 65536;
  const size_t lds = 3 * (size_t)c_z * sizeof(float);
  if (dtype == NT_BF16)
    hipLaunchKernelGGL(k_transition_backward_generic<bf16>, dim3((unsigned)grid), dim3(kThreads),
                       lds, s, static_cast<const bf16*>(z), G, static_cast<const bf16*>(W1),
                       static_cast<const bf16*>(W2), g_z, static_cast<bf16*>(H),
                       static_cast<bf16*>(GH), static_cast<bf16*>(Gb), p.cells, c_z, hidden);
  else
    hipLaunchKernelGGL(k_transition_backward_generic<float>, dim3((unsigned)grid),
                       dim3(kThreads), lds, s, static_cast<const float*>(z), G,
                       static_cast<const float*>(W1), static_cast<const float*>(W2), g_z,
                       static_cast<float*>(H), static_cast<float*>(GH), static_cast<float*>(Gb),
                       p.cells, c_z, hidden);
  return hipGetLastError();
}

}  // namespace nt
