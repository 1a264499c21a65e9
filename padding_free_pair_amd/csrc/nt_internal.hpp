// Internal definitions shared by the gfx950 kernels and the host API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nt_pair.h"

namespace nt {

constexpr uint32_t kPartitionMagic = 0x4E545031u;  // "NTP1"

// Widths the library accepts (all multiples of 8).
constexpr int kMaxCz = 512;
constexpr int kMaxCs = 16384;
constexpr int kMaxHidden = 16384;

// ---------------------------------------------------------------------------
// Column-mean schedule. Rows of one sample all have N_i cells. A row of at
// least kLongRow cells is one work item, reduced by a whole workgroup; shorter
// rows are grouped, rows_per_item(N) at a time, and each wave of the
// workgroup reduces whole rows. Items never cross samples, so the item of a
// workgroup is found by a search over per-sample item offsets.
constexpr int64_t kLongRow = 256;
constexpr int64_t kItemCells = 512;

// m: cells per pair row (M_i; N_i for square pairs). Rows without cells
// (M_i = 0) are grouped 64 to an item; their mean is 0/0.
__host__ __device__ inline int64_t rows_per_item(int64_t m) {
  if (m >= kLongRow) return 1;
  if (m <= 0) return 64;
  int64_t k = kItemCells / (4 * m);
  return 4 * (k < 1 ? 1 : k);
}

// Work items of a sample with n pair rows of m cells each.
__host__ __device__ inline int64_t items_of(int64_t n, int64_t m) {
  if (n <= 0) return 0;
  const int64_t r = rows_per_item(m);
  return (n + r - 1) / r;
}

// The last-level cache (MALL) of one MI355X. An array larger than this that
// one kernel writes and the next reads once cannot still be cached, so the
// reading kernel streams it with nontemporal loads, which do not allocate.
constexpr int64_t kStreamBytes = int64_t(256) << 20;

// Cells per entry of the tile_sample execution index.
constexpr int64_t kSampleIndexSpan = 256;
inline int64_t sample_index_entries(int64_t cells) {
  return (cells + kSampleIndexSpan - 1) / kSampleIndexSpan;
}

// Byte layout of the partition buffer: each array starts 256-byte aligned.
struct PartitionLayout {
  size_t lengths, single_offsets, pair_offsets, item_offsets, row_splits, row_sample, tile_sample,
      col_lengths, col_offsets, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Square partitions alias the column arrays to the row arrays (rect false).
inline PartitionLayout partition_layout(int64_t B, int64_t T, int64_t cells, bool rect = false) {
  PartitionLayout L;
  size_t off = 0;
  L.lengths = off;        off = align256(off + sizeof(int32_t) * (B > 0 ? B : 1));
  L.single_offsets = off; off = align256(off + sizeof(int64_t) * (B + 1));
  L.pair_offsets = off;   off = align256(off + sizeof(int64_t) * (B + 1));
  L.item_offsets = off;   off = align256(off + sizeof(int64_t) * (B + 1));
  L.row_splits = off;     off = align256(off + sizeof(int64_t) * (T + 1));
  L.row_sample = off;     off = align256(off + sizeof(int32_t) * (T > 0 ? T : 1));
  const int64_t K = sample_index_entries(cells);
  L.tile_sample = off;    off = align256(off + sizeof(int32_t) * (K > 0 ? K : 1));
  if (rect) {
    L.col_lengths = off;  off = align256(off + sizeof(int32_t) * (B > 0 ? B : 1));
    L.col_offsets = off;  off = align256(off + sizeof(int64_t) * (B + 1));
  } else {
    L.col_lengths = L.lengths;
    L.col_offsets = L.single_offsets;
  }
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip sources). Each returns the launch's
// hipError_t; arguments are validated by the host API beforehand.
// p.lengths and p.col_lengths (device) hold N and M; mu is written only
// when it is a separate array (rectangular partitions).
hipError_t launch_partition(const nt_partition& p, int64_t* single_offsets, int64_t* col_offsets,
                            int64_t* pair_offsets, int64_t* item_offsets, int64_t* row_splits,
                            int32_t* row_sample, int32_t* tile_sample, hipStream_t stream);
// Batches of at most kArgSamples samples: one launch, lengths passed by value
// from host memory (read before the call returns).
constexpr int kArgSamples = 256;
hipError_t launch_partition_small(const int32_t* lengths_host, const int32_t* cols_host,
                                  const nt_partition& p, int32_t* lengths, int32_t* col_lengths,
                                  int64_t* single_offsets, int64_t* col_offsets,
                                  int64_t* pair_offsets, int64_t* item_offsets,
                                  int64_t* row_splits, int32_t* row_sample, int32_t* tile_sample,
                                  hipStream_t stream);
hipError_t launch_decode(const nt_partition& p, int32_t* sample, int32_t* row, int32_t* col,
                         hipStream_t stream);
// f32_inputs: a and b are fp32 whatever dtype is (the projections' results).
hipError_t launch_broadcast(const nt_partition& p, const void* a, const void* b, void* z, int c_z,
                            nt_dtype dtype, hipStream_t stream, bool f32_inputs = false);
// z_in == nullptr selects the fused form: z is formed from fp32 a and b in
// the prologue (a, b are fp32 [T, c_z] whatever the storage dtype).
bool transition_has_mfma(int c_z, int hidden, nt_dtype dtype);
// Pre-normalised SwiGLU transition (bf16, c_z in {64, 128}, hidden % 32 == 0).
// z_in == nullptr selects the fused form: z = a[row] + b[col] from the fp32
// projections (needs the tile_sample index).
bool transition_swiglu_supported(int c_z, int hidden, nt_dtype dtype);
hipError_t launch_transition_swiglu(const nt_partition& p, const void* z_in, const void* a,
                                    const void* b, void* z_out, const float* gamma,
                                    const float* beta, const void* Wg, const void* Wu,
                                    const void* Wd, int c_z, int hidden, float eps,
                                    hipStream_t stream);
// Fused broadcast + transition for c_z = 128, hidden = 512 with both weights
// held in registers (one hidden quarter per wave) over 32-row blocks; needs
// the tile_sample index and T S < 2^22. S > 1: the non-leading layout, S
// slices of c_z per pair cell and per single row (a, b: [T S, c_z]).
hipError_t launch_transition_ws(const nt_partition& p, const void* a, const void* b, void* z_out,
                                const void* W1, const void* W2, int cus, hipStream_t stream,
                                int S = 1);
// The fused non-leading form: the weight-stationary kernel over S slices
// per cell (bf16, c_z 128, hidden 512, T S < 2^22); false when the shape or
// size does not allow it.
bool transition_ws_slices_supported(const nt_partition& p, int c_z, int hidden, nt_dtype dtype,
                                    int S);
hipError_t launch_transition(const nt_partition& p, const void* z_in, const void* a, const void* b,
                             void* z_out, const void* W1, const void* W2, int c_z, int hidden,
                             nt_dtype dtype, hipStream_t stream);
// mean == false: row sums instead of means (the broadcast's row adjoint).
hipError_t launch_reduce(const nt_partition& p, const void* z, float* m, int c_z, nt_dtype dtype,
                         hipStream_t stream, bool mean = true);
// C[M, N] = (R ? R : 0) + A[M, K] W[N, K]^T with fp32 accumulation. R has
// C's type. Supported (A, W, C) types: (bf16, bf16, f32), (f32, bf16, bf16),
// (f32, bf16, f32), (f32, f32, f32). R may equal C (each element is read and
// written by one thread).
hipError_t launch_linear(const void* A, nt_dtype a_dtype, const void* W, nt_dtype w_dtype,
                         const void* R, void* C, nt_dtype c_dtype, int64_t M, int N, int K,
                         hipStream_t stream);
// Two projections of one left operand in one launch: C0 = A W0^T, C1 = A W1^T
// (fp32 results; A and the weights are `a_dtype`).
hipError_t launch_linear2(const void* A, nt_dtype a_dtype, const void* W0, const void* W1,
                          void* C0, void* C1, int64_t M, int N, int K, hipStream_t stream);

// ---- backward (nt_backward.hip, nt_transition_bwd.hip)
// G = g_in (or 0) + g_m[row] / M_i on every cell; G may equal g_in.
hipError_t launch_mean_backward(const nt_partition& p, const float* g_m, const float* g_in,
                                float* G, int c_z, hipStream_t stream);
// g_b[mu_i + c] = sum_r g_z[o_i + r M_i + c] (fp32).
hipError_t launch_col_sums(const nt_partition& p, const float* g_z, float* g_b, int c_z,
                           hipStream_t stream);
// Both broadcast adjoints, g_a (row sums) and g_b (column sums) of g_z with
// rows of W floats, from one read of g_z when bcast_adj_fused (square
// partitions, B <= 256): tile partial sums go to ws (bcast_adj_ws_bytes)
// and are added in tile order. Otherwise the row and column kernels run
// (ws unused).
bool bcast_adj_fused(const nt_partition& p, int W);
size_t bcast_adj_ws_bytes(const nt_partition& p, int W);
hipError_t launch_bcast_adj(const nt_partition& p, const float* g_z, float* g_a, float* g_b,
                            int W, float* ws, hipStream_t stream);
// Equation 5: rows of x hold S * c_s values, rows of pz S * c_z; partial
// [max(T, 1)] fp64 scratch, loss one fp64; g_x, g_pz may be null.
hipError_t launch_loss_eq5(const nt_partition& p, const void* x, int c_s, const void* pz, int c_z,
                           int S, nt_dtype dtype, double* partial, double* loss, float* g_x,
                           float* g_pz, hipStream_t stream);
hipError_t launch_transpose(const void* src, void* dst, int R, int C, nt_dtype dtype,
                            hipStream_t stream);
// C[M, N] = sum_k A[k, M] B[k, N]; partial holds splits * M * N floats.
int gemm_tn_splits(int64_t K, int M, int N);
hipError_t launch_gemm_tn(const void* A, nt_dtype a_dtype, const void* B, nt_dtype b_dtype,
                          float* C, float* partial, int64_t K, int M, int N, int splits,
                          hipStream_t stream);
// C = sum of S partials [S][MN] in slice order (S = 0: C = 0).
hipError_t launch_sum_splits(const float* part, float* C, int S, int64_t MN, hipStream_t stream);
// Matrix-core form of launch_gemm_tn for bf16 A, B with M, N multiples of
// 128; part holds wgrad_splits(K, M, N) * M * N floats. With chunked_rows
// > 0 both operands are chunk-major: element (k, m) at
// ((m / 32) chunked_rows + k) 32 + m % 32, chunked_rows >= K.
bool wgrad_supported(int M, int N);
int wgrad_splits(int64_t K, int M, int N);
hipError_t launch_wgrad(const void* A, const void* B, float* C, float* part, int64_t K, int M,
                        int N, int splits, hipStream_t stream, int64_t chunked_rows = 0);
// Weight gradients recomputed from z and bf16(G) (bf16, c_z 128, hidden 512):
// part holds 2 * wgrad_rc_slices(cells) * c_z * hidden floats.
bool wgrad_rc_supported(int c_z, int hidden, nt_dtype dtype);
int wgrad_rc_slices(int64_t cells);
hipError_t launch_wgrad_rc(const void* z, const void* Gb, const void* W1, const void* W2T,
                           float* dW1, float* dW2, float* part, int64_t cells, int slices,
                           hipStream_t stream);
// Static scratch of nt_pair_block_noalloc (nt_static.hip): bytes per
// device, and its device address on the current device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void** ptr);
// ---- Fused SwiGLU transition gradient (nt_swiglu_bwd32.hip): c_z 128, hidden
// a multiple of 128, bf16. From the fp32 projections a, b (the pair state is
// formed per cell) and G (fp32 [cells, c_z], replaced by g_z): X2 and G2 get
// x = LN(z) and G as bf16 pairs (hi in columns 0 .. c_z - 1, lo in c_z ..
// 2 c_z - 1), A, GU, GG get A, g_u, g_g (hidden columns) in bf16, all
// chunk-major (column m of row k at ((m / 32) rows + k) 32 + m % 32, so a
// wave's stores of a chunk are contiguous), with rows =
// swiglu_bwd32_rows(cells) (whole tiles; the rows past the cells hold
// garbage), lnpart the
// workgroups' dgamma and dbeta sums [2][swiglu_bwd32_grid(cells)][c_z].
// WdT is Wd transposed [hidden, c_z]; WuT, WgT are Wu, Wg transposed
// [c_z, hidden].
bool swiglu_bwd32_supported(int c_z, int hidden, nt_dtype dtype);
int64_t swiglu_bwd32_rows(int64_t cells);
int swiglu_bwd32_grid(int64_t cells);
hipError_t launch_swiglu_bwd32(const nt_partition& p, const float* a, const float* b,
                               const float* gamma, const float* beta, const void* Wg,
                               const void* Wu, const void* WdT, const void* WuT, const void* WgT,
                               float* G, void* X2, void* G2, void* A, void* GU, void* GG,
                               float* lnpart, int hidden, float eps, hipStream_t stream);
// ---- SwiGLU transition gradient pieces (nt_swiglu_bwd.hip), c_z 64 or 128
// x = LN(z) row by row, fp32 (z fp32 [rows, c_z]).
hipError_t launch_ln_rows(const float* z, const float* gamma, const float* beta, float* x,
                          int64_t rows, int c_z, float eps, hipStream_t s);
// A = silu(g) u, g_u = g_A silu(g), g_g = g_A u silu'(g), all bf16; n elements.
hipError_t launch_swiglu_gate_bwd(const float* g, const float* u, const float* gA, void* A,
                                  void* gu, void* gg, int64_t n, hipStream_t s);
// G += LN's adjoint of gx (in place); dgamma, dbeta [c_z] from per-workgroup
// partials (part_gamma, part_beta: ln_backward_blocks(rows, c_z) x c_z floats).
int ln_backward_blocks(int64_t rows, int c_z);
hipError_t launch_ln_backward(const float* z, const float* gamma, const float* gx, float* G,
                              float* part_gamma, float* part_beta, float* dgamma, float* dbeta,
                              int64_t rows, int c_z, float eps, hipStream_t s);
// Compute units of the current device (cached per device).
int device_cu_count();
// Matrix-core transition gradient (bf16, c_z = 128, hidden = 512): W2T =
// W2^T [hidden, c_z] and W1T = W1^T [c_z, hidden] are prepared by the caller.
// H and GH may be null (then they are not written). With g_m non-null, G is
// not read: it is formed per cell as g_m[row] / M_i (+ g_in[cell] when
// g_in is non-null), exactly as launch_mean_backward forms it; the quotients
// go to gm_rows [T, c_z] first.
bool transition_backward_has_mfma(int c_z, int hidden, nt_dtype dtype);
hipError_t launch_transition_backward_mfma(const nt_partition& p, const void* z, const float* G,
                                           const float* g_m, const float* g_in, const void* W1,
                                           const void* W2T, const void* W1T, float* g_z,
                                           void* H, void* GH, void* Gb, float* gm_rows,
                                           int cus, hipStream_t stream);
// Transition gradient without weight gradients: g_z, and H, GH and Gb (G in
// the storage type) for them. g_z may equal G.
hipError_t launch_transition_backward_generic(const nt_partition& p, const void* z,
                                              const float* G, const void* W1, const void* W2,
                                              float* g_z, void* H, void* GH, void* Gb, int c_z,
                                              int hidden, nt_dtype dtype, hipStream_t stream);

}  // namespace nt
