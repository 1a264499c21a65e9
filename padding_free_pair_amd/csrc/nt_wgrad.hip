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
// 32x32x16 MFMA operand wants 8 values of k per lane: the step's 64 x 128
// rows of each operand are copied as they are into LDS ([k][m]), and the
// fragments are read with gfx950's transposing LDS read (ds_read_b64_tr_b16,
// two reads a fragment; both operands take the same k order within a step,
// so the contraction is unchanged). The next step's rows are loaded while
// the current step's products run, into the other of two LDS buffers.
#include "nt_device.hpp"
#include "nt_internal.hpp"

namespace nt {
namespace {

constexpr int kWgThreads = 256;
constexpr int kWgTile = 128;   // C tile edge
constexpr int kWgK = 64;       // k per step
constexpr int kWgRow = kWgTile + 8;  // LDS row pitch in elements (272 bytes)

typedef short wg_i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 wg_bf16x4 __attribute__((ext_vector_type(4)));

// Four bf16 by the transposing LDS read (within each 16 lanes, lane j's
// element e is element j mod 4 of the 8 bytes at the address of lane
// 4 e + j / 4); p is this lane's 8-byte address.
__device__ __forceinline__ wg_bf16x4 wg_read_tr(const bf16* p) {
  const wg_i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) wg_i16x4*)(p));
  return __builtin_bit_cast(wg_bf16x4, v);
}

__device__ __forceinline__ f32x16 wg_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup b takes tile t and K slice y (the slice [y kchunk, min(K,
// (y + 1) kchunk)), kchunk a multiple of kWgK), numbered so that the tiles
// of one slice run on one XCD (workgroups go to the XCDs round robin, b to
// XCD b mod 8): b = 8 (tiles q + t) + x with y = 8 q + x; they then read the
// slice's rows through one L2 (numbered tile-fastest, the tiles of a slice
// went to different XCDs and each fetched the slice from HBM: 2.7 times the
// operand bytes). Workgroups with y >= S return. The tile of C is (tm, tn) =
// (t % tiles_m, t / tiles_m); waves own 64 x 64 quadrants of it. Each thread
// stages four 16-byte pieces of each operand per step.
// CHUNKED: both operands in the chunk-major layout, element (k, m) at
// ((m / 32) rows + k) 32 + m % 32 (rows >= K: 32-column chunks of rows).
template <bool CHUNKED>
__global__ __launch_bounds__(kWgThreads, 2) void k_wgrad(const bf16* __restrict__ A,
                                                         const bf16* __restrict__ B,
                                                         float* __restrict__ part, int64_t K,
                                                         int M, int N, int64_t kchunk,
                                                         int64_t rows, int S) {
  __shared__ bf16 lds[2][2][kWgK * kWgRow];  // [buffer][operand][k * pitch + m]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_m = M / kWgTile, tiles = tiles_m * (N / kWgTile);
  const int q = blockIdx.x / 8, t = q % tiles;
  const int y = (q / tiles) * 8 + blockIdx.x % 8;
  if (y >= S) return;
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int64_t kb = (int64_t)y * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;

  // staging: piece p = tid + 256 u of an operand's 64 x 128 step tile is row
  // pk[u], columns pm[u] .. + 7 (chunk-major: 64 contiguous bytes a row and
  // chunk, so four lanes cover a chunk's row; row-major: 16 lanes a row)
  int pk[4], pm[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + kWgThreads * u;
    if (CHUNKED) {
      pk[u] = (p & 255) >> 2;
      pm[u] = 32 * (p >> 8) + 8 * (p & 3);
    } else {
      pk[u] = p >> 4;
      pm[u] = 8 * (p & 15);
    }
  }
  const bf16* base[2] = {A, B};
  const int col0[2] = {tm * kWgTile, tn * kWgTile};
  const int ld[2] = {M, N};
  auto gaddr = [&](int op, int64_t k, int m) -> const bf16* {
    const int c = col0[op] + m;
    return CHUNKED ? base[op] + (((int64_t)(c >> 5) * rows + k) * 32 + (c & 31))
                   : base[op] + (k * ld[op] + c);
  };
  bf16x8 nxt[2][4];
  // the rows of the step at k0; rows past the slice read its last row (in
  // bounds, no branch) and are zeroed
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t k = k0 + pk[u];
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(gaddr(op, k < ke ? k : ke - 1, pm[u]));
        nxt[op][u] = k < ke ? v : bf16x8{};
      }
  };
  auto put = [&](int bb) {
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<bf16x8*>(&lds[bb][op][pk[u] * kWgRow + pm[u]]) = nxt[op][u];
  };

  const int wm = wave & 1, wn = wave >> 1;  // quadrant of the C tile
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  // this lane's transposing-read address: within its 16-lane group (columns
  // 16 (g mod 2) .., rows 4 h ..), lane l' points at row 4 h + l' / 4,
  // column + 4 (l' mod 4); the fragment of a 32-column block then holds, for
  // column l32, rows 4 h + (0..3) and 8 + 4 h + (0..3) of a 16-row k-step
  const int lq = lane & 15, lg = lane >> 4;
  const int tr_off = (4 * h + (lq >> 2)) * kWgRow + 16 * (lg & 1) + 4 * (lq & 3);
  auto frag = [&](const bf16* T, int s, int m0) -> bf16x8 {
    const int off = tr_off + 16 * s * kWgRow + m0;
    const wg_bf16x4 v0 = wg_read_tr(T + off);
    const wg_bf16x4 v1 = wg_read_tr(T + off + 8 * kWgRow);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = v0[e];
      f[4 + e] = v1[e];
    }
    return f;
  };

  fetch(kb);
  put(0);
  __syncthreads();
  int bb = 0;
  for (int64_t k0 = kb; k0 < ke; k0 += kWgK) {
    fetch(k0 + kWgK);  // past the slice: clamped reads, not used
    const bf16* TA = lds[bb][0];
    const bf16* TB = lds[bb][1];
#pragma unroll
    for (int s = 0; s < kWgK / 16; ++s) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = frag(TA, s, 64 * wm + 32 * i);
        bfr[i] = frag(TB, s, 64 * wn + 32 * i);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = wg_mfma(af[i], bfr[j], acc[i][j]);
    }
    // the other buffer was last read in the previous step, before its barrier
    put(bb ^ 1);
    __syncthreads();
    bb ^= 1;
  }
  // partial tile: element r of block (i, j) is row 8 (r / 4) + 4 h + r % 4,
  // column l32 of that 32 x 32 block
  float* out = part + (int64_t)y * M * N;
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

// ---------------------------------------------------------------------------
// The transition's weight gradients recomputed from z and bf16(G), without
// materialising H or g_H: for hidden chunk j (32 units),
//   pre^T = z W1[j]^T, gh^T = bf16(G) W2T[j]^T     (cells x units, k = features)
//   g_H = gh * [pre > 0], H = relu(pre)            (lane-local)
//   dW1[j] += g_H^T z,  dW2[:, j] += bf16(G)^T H    (k = cells)
// Workgroup (slice, group): eight waves, two per SIMD, walk the same 64-cell
// blocks of the slice; waves w and w + 4 own chunk 4 group + w % 4, the
// first for the block's first 32 cells, the second for the other 32, and
// their sums are added (first + second) at the end. Workgroups are handed to the
// XCDs round robin (workgroup b to XCD b mod 8), so the index is split as
// b = 8 (GROUPS q + group) + x with slice 8 q + x: the GROUPS workgroups of a
// slice run on one XCD at the same time and read its cells through one L2
// (one HBM fetch instead of GROUPS). In the first two products the
// lane holds a unit and 16 cells, so the packed g_H and H are already the
// MFMA operands of the contractions over cells (k-step s takes result
// elements 8 s .. 8 s + 7, cells 16 s + 8 (e / 4) + 4 h + e % 4); the other
// operand, z or bf16(G) with a feature per lane, is read from the same
// row-major LDS copy with gfx950's transposing read (ds_read_b64_tr_b16:
// within each 16 lanes, lane j's element e is element j mod 4 of the 8 bytes
// at the address of lane 4 e + j / 4), two reads per fragment. The next
// block's rows are loaded into registers while the current block's products
// run and are written after them. The chunk weights (the B operands of the
// first two products) are read from LDS, not held in registers: a wave's
// accumulators then fit its 256 VGPRs (the file is built with the VGPR form
// of the products), with no moves between AGPRs and VGPRs around them, and
// two waves share each SIMD. Each chunk's first wave writes its partial dW1
// rows and dW2 columns for the slice; the slices are added in order
// afterwards.
constexpr int kRcCells = 64;              // cells per block (two 32-cell halves)
constexpr int kRcRow = 128 + 8;          // [cell][feature] pitch in elements (272 bytes)

typedef short rc_i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 rc_bf16x4 __attribute__((ext_vector_type(4)));

// Four bf16 by the transposing LDS read; p is this lane's 8-byte address.
__device__ __forceinline__ rc_bf16x4 rc_read_tr(const bf16* p) {
  const rc_i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) rc_i16x4*)(p));
  return __builtin_bit_cast(rc_bf16x4, v);
}

template <int CZ, int HID>
__global__ __launch_bounds__(512, 2) void k_wgrad_rc(
    const bf16* __restrict__ z, const bf16* __restrict__ Gb, const bf16* __restrict__ W1,
    const bf16* __restrict__ W2T, float* __restrict__ part1, float* __restrict__ part2,
    int64_t cells, int64_t slice_cells, int64_t slices) {
  constexpr int KT = CZ / 16, FB = CZ / 32, GROUPS = HID / 128;
  static_assert(CZ == 128, "row staging assumes 128 features");
  // [buffer][operand: 0 z, 1 G]
  __shared__ bf16 rm[2][2][kRcCells * kRcRow];
  // each chunk's weights as B fragments: [chunk of the group][matrix][t][lane]
  __shared__ bf16x8 wl[4][2][KT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int cw = wave & 3, hb = wave >> 2;  // chunk of the group, half of each block
  const int64_t q = blockIdx.x / 8;
  const int group = (int)(q % GROUPS);
  const int64_t slice = 8 * (q / GROUPS) + blockIdx.x % 8;
  if (slice >= slices) return;  // the grid is rounded up to whole XCD rounds
  const int j = 4 * group + cw;
  const int64_t cb0 = slice * slice_cells;
  const int64_t cb1 = cb0 + slice_cells < cells ? cb0 + slice_cells : cells;

  // chunk j's weights as the B operand: unit 32 j + l32, features 16 t + 8 h ..
  // (in LDS, read by the chunk's two waves)
  if (hb == 0) {
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      wl[cw][0][t][lane] =
          *reinterpret_cast<const bf16x8*>(W1 + (int64_t)(32 * j + l32) * CZ + 16 * t + 8 * h);
      wl[cw][1][t][lane] =
          *reinterpret_cast<const bf16x8*>(W2T + (int64_t)(32 * j + l32) * CZ + 16 * t + 8 * h);
    }
  }
  f32x16 acc1[FB], acc2[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    acc1[f] = f32x16{};
    acc2[f] = f32x16{};
  }

  // staging: thread -> operand (tid < 256: z, else G), cell cp, 16-byte
  // pieces sp0 .. sp0 + 3 of it
  const int op = tid >> 8, st = tid & 255, cp = st >> 2, sp0 = 4 * (st & 3);
  const bf16* ssrc = op == 0 ? z : Gb;
  bf16x8 nxt[4];
  auto load_rows = [&](int64_t c0) {
    const int64_t c = c0 + cp;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      nxt[k] = c < cb1 ? *reinterpret_cast<const bf16x8*>(ssrc + c * CZ + 8 * (sp0 + k))
                       : bf16x8{};
  };
  auto write_rows = [&](int buf) {
    bf16* R = rm[buf][op];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<bf16x8*>(R + cp * kRcRow + 8 * (sp0 + k)) = nxt[k];
  };
  // this lane's transposing-read address in a 32-cell half: within its
  // 16-lane group (features 32 f + 16 (g mod 2) .., cells 4 h ..), lane l'
  // points at cell 4 h + l' / 4, features + 4 (l' mod 4)
  const int lq = lane & 15, lg = lane >> 4;
  const int tr_off = (4 * h + (lq >> 2)) * kRcRow + 16 * (lg & 1) + 4 * (lq & 3);

  int buf = 0;
  if (cb0 < cb1) {
    load_rows(cb0);
    write_rows(0);
  }
  __syncthreads();
  for (int64_t c0 = cb0; c0 < cb1; c0 += kRcCells) {
    const bool more = c0 + kRcCells < cb1;
    if (more) load_rows(c0 + kRcCells);  // in flight during this block's products
    const bf16* Rz = rm[buf][0];
    const bf16* Rg = rm[buf][1];
    f32x16 pre = f32x16{}, gh = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int r = (32 * hb + l32) * kRcRow + 16 * t + 8 * h;
      const bf16x8 za = *reinterpret_cast<const bf16x8*>(Rz + r);
      const bf16x8 ga = *reinterpret_cast<const bf16x8*>(Rg + r);
      pre = wg_mfma(za, wl[cw][0][t][lane], pre);
      gh = wg_mfma(ga, wl[cw][1][t][lane], gh);
    }
    // relu and the mask on the bits: a float is > 0 exactly when its bits
    // are a positive integer (finite inputs), and max(bits, 0) is relu
    bf16x8 hk[2], gk[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pi = __float_as_int(pre[8 * s + e]);
        hk[s][e] = (bf16)__int_as_float(pi > 0 ? pi : 0);
        gk[s][e] = (bf16)(pi > 0 ? gh[8 * s + e] : 0.f);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        // cells 32 hb + 16 s + 4 h + (0..3) and + 8, feature 32 f + l32
        const int off = tr_off + (32 * hb + 16 * s) * kRcRow + 32 * f;
        const rc_bf16x4 z0 = rc_read_tr(Rz + off);
        const rc_bf16x4 z1 = rc_read_tr(Rz + off + 8 * kRcRow);
        const rc_bf16x4 g0 = rc_read_tr(Rg + off);
        const rc_bf16x4 g1 = rc_read_tr(Rg + off + 8 * kRcRow);
        bf16x8 zf, gf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          zf[e] = z0[e];
          zf[4 + e] = z1[e];
          gf[e] = g0[e];
          gf[4 + e] = g1[e];
        }
        acc1[f] = wg_mfma(gk[s], zf, acc1[f]);  // dW1[j] (units x features)
        acc2[f] = wg_mfma(gf, hk[s], acc2[f]);  // dW2[:, j] (features x units)
      }
    // the other buffer was last read two blocks ago, before the previous barrier
    if (more) write_rows(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // the second half's sums join the first's through LDS (over the row
  // buffers, free after the last barrier), dW1's then dW2's, in that order
  float* xch = reinterpret_cast<float*>(&rm[0][0][0]);  // [chunk][f][r][lane]
  static_assert(sizeof(rm) >= sizeof(float) * 4 * FB * 16 * 64, "exchange fits");
#pragma unroll
  for (int mat = 0; mat < 2; ++mat) {
    f32x16 (&acc)[FB] = mat == 0 ? acc1 : acc2;
    if (hb == 1) {
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[((cw * FB + f) * 16 + r) * 64 + lane] = acc[f][r];
    }
    __syncthreads();
    if (hb == 0) {
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[f][r] += xch[((cw * FB + f) * 16 + r) * 64 + lane];
    }
    __syncthreads();
  }
  if (hb == 1) return;
  // partials: acc1[f] element r is unit 8 (r / 4) + 4 h + r % 4, feature 32 f + l32;
  // acc2[f] element r is feature 32 f + 8 (r / 4) + 4 h + r % 4, unit l32
  float* o1 = part1 + slice * HID * CZ;
  float* o2 = part2 + slice * CZ * HID;
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r / 4) + 4 * h + r % 4;
      o1[(int64_t)(32 * j + i) * CZ + 32 * f + l32] = acc1[f][r];
      o2[(int64_t)(32 * f + i) * HID + 32 * j + l32] = acc2[f][r];
    }
}

}  // namespace

bool wgrad_rc_supported(int c_z, int hidden, nt_dtype dtype) {
  return dtype == NT_BF16 && c_z == 128 && hidden == 512;
}

// Slices of the cells: one workgroup per (slice, group of four chunks), about
// one workgroup per CU of a 256-CU part, at least 256 cells a slice.
int wgrad_rc_slices(int64_t cells) {
  int64_t S = 256 / 4;
  const int64_t smax = (cells + 255) / 256;
  if (S > smax) S = smax;
  return (int)(S < 1 ? 1 : S);
}

hipError_t launch_wgrad_rc(const void* z, const void* Gb, const void* W1, const void* W2T,
                           float* dW1, float* dW2, float* part, int64_t cells, int slices,
                           hipStream_t stream) {
  constexpr int CZ = 128, HID = 512;
  const int64_t MN = (int64_t)CZ * HID;
  if (cells == 0) {
    hipError_t e = launch_sum_splits(part, dW1, 0, MN, stream);
    return e != hipSuccess ? e : launch_sum_splits(part, dW2, 0, MN, stream);
  }
  int64_t slice_cells = (cells + slices - 1) / slices;
  slice_cells = (slice_cells + kRcCells - 1) / kRcCells * kRcCells;
  const int64_t S = (cells + slice_cells - 1) / slice_cells;
  float* part1 = part;
  float* part2 = part + S * MN;
  const int64_t S8 = (S + 7) / 8 * 8;
  hipLaunchKernelGGL((k_wgrad_rc<CZ, HID>), dim3((unsigned)(S8 * (HID / 128))), dim3(512), 0,
                     stream, static_cast<const bf16*>(z), static_cast<const bf16*>(Gb),
                     static_cast<const bf16*>(W1), static_cast<const bf16*>(W2T), part1, part2,
                     cells, slice_cells, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_sum_splits(part1, dW1, (int)S, MN, stream);
  return e != hipSuccess ? e : launch_sum_splits(part2, dW2, (int)S, MN, stream);
}

int wgrad_splits(int64_t K, int M, int N) {
  const int64_t tiles = (int64_t)(M / kWgTile) * (N / kWgTile);
  int64_t S = (512 + tiles - 1) / tiles;  // about 512 workgroups (two per CU of a 256-CU part)
  const int64_t kmax = (K + 4 * kWgK - 1) / (4 * kWgK);  // at least four steps a slice
  if (S > kmax) S = kmax;
  return (int)(S < 1 ? 1 : (S > 512 ? 512 : S));
}

bool wgrad_supported(int M, int N) { return M % kWgTile == 0 && N % kWgTile == 0; }

hipError_t launch_wgrad(const void* A, const void* B, float* C, float* part, int64_t K, int M,
                        int N, int splits, hipStream_t stream, int64_t chunked_rows) {
  if (K == 0) return launch_sum_splits(part, C, 0, (int64_t)M * N, stream);
  int64_t kchunk = (K + splits - 1) / splits;
  kchunk = (kchunk + kWgK - 1) / kWgK * kWgK;
  const int64_t S = (K + kchunk - 1) / kchunk;
  const int64_t tiles = (int64_t)(M / kWgTile) * (N / kWgTile);
  const int64_t grid = 8 * tiles * ((S + 7) / 8);
  auto kern = chunked_rows > 0 ? k_wgrad<true> : k_wgrad<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWgThreads), 0, stream,
                     static_cast<const bf16*>(A), static_cast<const bf16*>(B), part, K, M, N,
                     kchunk, chunked_rows, (int)S);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_splits(part, C, (int)S, (int64_t)M * N, stream);
}

}  // namespace nt
