/*
 * nt_pair.h - packed single-pair-single block on AMD Instinct MI355X (gfx950).
 *
 * The operation is the single-pair-single block of the DanLing NestedTensor
 * paper (arXiv 2609.30379, Section 3, Equation 1), run on packed
 * multi-ragged storage instead of a B x N_max^2 envelope:
 *
 *   a = s Wa^T,  b = s Wb^T                    (single projections)
 *   z[o_i + r N_i + c] = a[eta_i + r] + b[eta_i + c]        (broadcast)
 *   z~ = z + relu(z W1^T) W2^T                  (residual cell transition)
 *   m[eta_i + r] = (1/N_i) sum_c z~[o_i + r N_i + c]        (column mean)
 *   s~ = s + m Wo^T                             (output projection, residual)
 *
 * eta_i = sum_{k<i} N_k are the single offsets and o_i = sum_{k<i} N_k^2 the
 * pair offsets (Section 3.1, Equation 2); the packed row of pair cell (r, c)
 * of sample i is Equation 3's o_i + r N_i + c; the column sum is Equation 4.
 *
 * Conventions for every call:
 *  - Memory: every array argument is device memory owned by the caller and
 *    must stay alive until the work enqueued on `stream` has finished. The
 *    library allocates no device memory and keeps no state except a
 *    thread-local error message.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream). Every device call is asynchronous on it.
 *  - Layout: row-major, contiguous, feature dimension innermost. Singles are
 *    [T, c_s], pair states [cells, c_z]. Weights are [out, in] (the layout of
 *    the paper's V W^T, Section 3.3), without bias:
 *       Wa, Wb: [c_z, c_s]  W1: [hidden, c_z]  W2: [c_z, hidden]  Wo: [c_s, c_z]
 *  - Element type: NT_BF16 (storage bf16, accumulation fp32, results rounded
 *    to nearest-even) or NT_F32 (fp32 throughout). The column mean m is always
 *    fp32.
 *  - Widths c_s, c_z and hidden must be positive multiples of 8, with
 *    c_z <= 512 and c_s, hidden <= 16384.
 *  - Alignment: every array pointer must be 16-byte aligned.
 *  - Errors: arguments are checked on the host before anything is enqueued;
 *    a validation failure enqueues nothing and leaves outputs untouched.
 *    NT_ERR_HIP means the runtime rejected a launch; stages of the same call
 *    before it may already be enqueued. nt_last_error() describes the
 *    failure. Faults inside kernels surface at the caller's next
 *    synchronisation, as with any HIP launch. No call aborts or throws.
 */
#ifndef NT_PAIR_H
#define NT_PAIR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nt_status {
  NT_OK = 0,
  NT_ERR_NULL = 1,      /* a required pointer is NULL */
  NT_ERR_INVALID = 2,   /* bad length, width, partition, or overlapping buffers */
  NT_ERR_OVERFLOW = 3,  /* a size does not fit the index types */
  NT_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  NT_ERR_WORKSPACE = 5, /* buffer or workspace smaller than required */
  NT_ERR_DTYPE = 6,     /* unknown element type */
  NT_ERR_HIP = 7        /* the HIP runtime rejected a launch */
} nt_status;

typedef enum nt_dtype { NT_F32 = 0, NT_BF16 = 1 } nt_dtype;

/*
 * A pair partition (Section 3.1 "Structural metadata"; Figure 2; Appendix A
 * "Structural invariants"): square, N_i x N_i (nt_make_partition), or
 * rectangular, N_i x M_i (nt_make_partition_rect; Section 3.1 packs
 * (N_i, M_i, C) pairs as (sum N_i M_i, C)). Host scalars are canonical; the
 * arrays are device mirrors inside the caller's partition buffer. Read-only
 * for callers. N_i counts pair rows (lengths), M_i pair columns
 * (col_lengths); a square partition has M_i = N_i and its column arrays
 * point at the row arrays.
 *
 *   single_offsets [B+1]  eta_i over N_i (the row singles), eta_B = T
 *   col_offsets    [B+1]  mu_i over M_i (the column singles), mu_B = T_cols
 *   pair_offsets   [B+1]  o_i over N_i M_i, o_B = cells; empty samples repeat
 *   row_splits     [T+1]  second-level splits: pair row r of sample i starts
 *                         at o_i + r M_i; row_splits[T] = cells
 *   row_sample     [T]    sample index of each pair row
 *   item_offsets   [B+1]  execution index of the column-mean schedule: sample
 *                         i owns work items [item_offsets[i], item_offsets[i+1])
 *   tile_sample    [ceil(cells / 256)]  execution index of the pair kernels:
 *                         the sample holding cell 256 k (the non-empty one)
 */
typedef struct nt_partition {
  uint32_t magic;       /* set by nt_make_partition */
  int32_t B;            /* samples */
  int32_t n_max;        /* max_i N_i (0 if every sample is empty) */
  int32_t reserved;
  int64_t T;            /* sum_i N_i */
  int64_t cells;        /* sum_i N_i M_i (sum_i N_i^2 when square) */
  int64_t n_items;      /* item_offsets[B] */
  const int32_t* lengths;
  const int64_t* single_offsets;
  const int64_t* pair_offsets;
  const int64_t* row_splits;
  const int32_t* row_sample;
  const int64_t* item_offsets;
  const int32_t* tile_sample;
  int64_t T_cols;                /* sum_i M_i (== T when square) */
  const int32_t* col_lengths;    /* [B] M_i (== lengths when square) */
  const int64_t* col_offsets;    /* [B+1] mu_i (== single_offsets when square) */
} nt_partition;

/* The five weights of one block; see the layout convention above. */
typedef struct nt_block_weights {
  const void* Wa;
  const void* Wb;
  const void* W1;
  const void* W2;
  const void* Wo;
} nt_block_weights;

/*
 * Host only. Validates lengths and reports the partition's sizes and the
 * device buffer nt_make_partition needs. lengths: host int32 [B], N_i >= 0
 * (NULL allowed only when B == 0). Any output pointer may be NULL.
 * Errors: NT_ERR_INVALID (B < 0 or a negative length), NT_ERR_NULL,
 * NT_ERR_OVERFLOW (sum N_i^2 exceeds int64, or T exceeds INT32_MAX).
 */
nt_status nt_partition_sizes(const int32_t* lengths, int32_t B, int64_t* T, int64_t* cells,
                             int32_t* n_max, size_t* buffer_bytes);

/*
 * Builds the partition of Section 3.1 / Figure 2 for square pairs on the
 * device: the exclusive scans giving eta, o and the item offsets, then
 * row_splits and row_sample. The host lengths reach the device as kernel
 * arguments when B <= 256 (one launch; the lengths are read before the call
 * returns); larger batches copy them into `buffer` on `stream` first
 * (pageable memory is read before the call returns; page-locked memory is
 * read asynchronously and must stay unchanged until the stream passes this
 * call) and use two launches. `out` receives the host
 * scalars and pointers into `buffer` immediately; the device arrays are
 * valid once the stream reaches this point. The partition stays valid while
 * `buffer` lives. buffer: device, at least nt_partition_sizes' buffer_bytes,
 * 256-byte aligned. Errors: as nt_partition_sizes, plus NT_ERR_WORKSPACE,
 * NT_ERR_ALIGN, NT_ERR_HIP.
 */
nt_status nt_make_partition(const int32_t* lengths, int32_t B, void* buffer, size_t buffer_bytes,
                            void* stream, nt_partition* out);

/*
 * Rectangular pairs (Section 3.1: (N_i, M_i, C) packs as (sum N_i M_i, C);
 * Appendix A.1's rectangular variant). Host only, like nt_partition_sizes:
 * rows, cols: host int32 [B], N_i, M_i >= 0. T = sum N_i, T_cols = sum M_i,
 * cells = sum N_i M_i. Errors as nt_partition_sizes (T_cols is bounded like
 * T).
 */
nt_status nt_partition_sizes_rect(const int32_t* rows, const int32_t* cols, int32_t B, int64_t* T,
                                  int64_t* T_cols, int64_t* cells, size_t* buffer_bytes);

/*
 * Builds a rectangular partition on the device, as nt_make_partition does a
 * square one: eta over N_i, mu over M_i, o over N_i M_i, the column-mean
 * item offsets, row_splits[eta_i + r] = o_i + r M_i, row_sample and the tile
 * index. Every stage entry point accepts the result: the broadcast reads row
 * singles a [T, c_z] and column singles b [T_cols, c_z], the column mean
 * divides each row's sum by M_i (a row with M_i = 0 has no cells and its mean
 * is 0/0, NaN). Host memory and buffer rules as nt_make_partition.
 */
nt_status nt_make_partition_rect(const int32_t* rows, const int32_t* cols, int32_t B, void* buffer,
                                 size_t buffer_bytes, void* stream, nt_partition* out);

/*
 * Test hook: materialises the decode of every packed cell t into its
 * (sample, row, col) with t = o_sample + row * N_sample + col (Equation 3
 * inverted). sample, row, col: device int32 [cells]. The hot kernels decode
 * on the fly and never build these maps.
 */
nt_status nt_decode_cells(const nt_partition* p, int32_t* sample, int32_t* row, int32_t* col,
                          void* stream);

/*
 * Broadcast (Equation 1, first line; Section 3.2 "Creating axes through
 * broadcasting"): z[o_i + r M_i + c, :] = a[eta_i + r, :] + b[mu_i + c, :]
 * (M_i = N_i and mu = eta for square pairs). a: [T, c_z]; b: [T_cols, c_z];
 * z: [cells, c_z], all of `dtype`. The sum is formed in fp32 and rounded once
 * to the storage type. z must not overlap a or b.
 */
nt_status nt_pair_broadcast(const nt_partition* p, const void* a, const void* b, void* z,
                            int32_t c_z, nt_dtype dtype, void* stream);

/*
 * Residual pair transition (Equation 1, second line, with a two-layer ReLU
 * MLP as the feature update; Section 3.3 "Dense work across valid
 * positions": it runs over the sum N_i^2 packed cells only):
 *   z_out = z_in + relu(z_in W1^T) W2^T, cell by cell.
 * z_in, z_out: [cells, c_z]; W1: [hidden, c_z]; W2: [c_z, hidden]. In bf16
 * the hidden activations are rounded to bf16 before the second product and
 * both products accumulate in fp32. z_out may equal z_in (in place); other
 * overlaps are rejected.
 */
nt_status nt_pair_transition(const nt_partition* p, const void* z_in, void* z_out, const void* W1,
                             const void* W2, int32_t c_z, int32_t hidden, nt_dtype dtype,
                             void* stream);

/*
 * Broadcast fused into the transition (Equation 1's first two lines in one
 * kernel): z_out[o_i + r M_i + c] = z + relu(z W1^T) W2^T with
 * z = a[eta_i + r] + b[mu_i + c] formed on chip and never written to
 * memory. a: fp32 [T, c_z], b: fp32 [T_cols, c_z] whatever `dtype` is (the projections' fp32
 * results); z_out: [cells, c_z] of `dtype`; W1, W2 as for
 * nt_pair_transition. With NT_BF16 the MLP reads z rounded to bf16 while the
 * residual adds z in fp32, so the pair state is rounded once, on output.
 * This is the kernel nt_pair_block runs for these two stages. z_out must not
 * overlap a, b or the weights.
 */
nt_status nt_pair_broadcast_transition(const nt_partition* p, const void* a, const void* b,
                                       void* z_out, const void* W1, const void* W2, int32_t c_z,
                                       int32_t hidden, nt_dtype dtype, void* stream);

/*
 * The paper's own transition: a residual, pre-normalised SwiGLU update
 * (Equation 1, second line, P~ = P + h(LN(P)); Appendix A.1, "transition
 * expansion four"), cell by cell over the packed cells:
 *   x = (z - mean) / sqrt(var + ln_eps) * ln_gamma + ln_beta,
 *       mean and biased var over the c_z features of the cell;
 *   z_out = z_in + (silu(x W_gate^T) * (x W_up^T)) W_down^T,
 *       silu(g) = g / (1 + exp(-g)).
 * z_in, z_out: [cells, c_z] bf16; ln_gamma, ln_beta: fp32 [c_z];
 * W_gate, W_up: bf16 [hidden, c_z]; W_down: bf16 [c_z, hidden]. Statistics
 * and products accumulate in fp32; x and the gated activations are rounded
 * to bf16 before the products that read them; the residual adds z in fp32
 * and rounds once.
 * Supported: dtype NT_BF16 (else NT_ERR_DTYPE), c_z 64 or 128 and hidden a
 * positive multiple of 32 (else NT_ERR_INVALID), ln_eps finite and >= 0.
 * z_out may equal z_in (in place); other overlaps are rejected.
 */
nt_status nt_pair_transition_swiglu(const nt_partition* p, const void* z_in, void* z_out,
                                    const float* ln_gamma, const float* ln_beta,
                                    const void* W_gate, const void* W_up, const void* W_down,
                                    int32_t c_z, int32_t hidden, float ln_eps, nt_dtype dtype,
                                    void* stream);

/*
 * Column mean (Equation 1, third line; Equation 4 divided by M_i, which is
 * N_i for square pairs):
 *   m[eta_i + r, :] = (1/M_i) sum_{c < M_i} z[o_i + r M_i + c, :].
 * z: [cells, c_z] of `dtype`; m: fp32 [T, c_z]. Deterministic: a row of at
 * least 256 cells is summed by one workgroup, a shorter row by one wave,
 * each in a fixed order, with no atomics.
 */
nt_status nt_pair_reduce(const nt_partition* p, const void* z, float* m, int32_t c_z,
                         nt_dtype dtype, void* stream);

/*
 * Workspace bytes nt_pair_block needs for this partition and widths.
 */
nt_status nt_block_workspace_bytes(const nt_partition* p, int32_t c_s, int32_t c_z,
                                   int32_t hidden, nt_dtype dtype, size_t* bytes);

/*
 * One whole block (Equation 1; Figure 3's three lines): projections, the
 * broadcast fused into the transition's prologue, the column mean and the
 * output projection with its residual. Returns both outputs, as the paper's
 * block does: s_out [T, c_s] and z_out [cells, c_z]. s_out may equal s_in.
 * workspace: device, at least nt_block_workspace_bytes, 16-byte aligned;
 * it holds a, b (fp32, unrounded projections) and m (fp32) between stages.
 */
nt_status nt_pair_block(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                        const nt_block_weights* w, int32_t c_s, int32_t c_z, int32_t hidden,
                        nt_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nt_pair_block without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The workspace nt_pair_block
 * takes (fp32 a, b and m, nt_block_workspace_bytes) lives in a static device
 * array of 16 MiB that every GPU the library runs on holds until the process
 * ends: 3 x (T * c_z * 4 bytes, rounded up to 256) <= 16 MiB, so T <= 10,922
 * single rows at c_z = 128. The call itself allocates nothing and clears nothing (every
 * launch writes the scratch before reading it); the first call on a device
 * looks up the array's address there. Calls on one GPU share the array, so
 * calls that overlap in time on one GPU (other streams, other threads) race;
 * serialise them. Square partitions. Inputs, outputs and errors as
 * nt_pair_block, plus NT_ERR_WORKSPACE when the partition needs more scratch
 * than the array holds (checked before anything is enqueued).
 */
nt_status nt_pair_block_noalloc(const nt_partition* p, const void* s_in, void* s_out,
                                void* z_out, const nt_block_weights* w, int32_t c_s, int32_t c_z,
                                int32_t hidden, nt_dtype dtype, void* stream);

/*
 * Workspace bytes nt_pair_chain needs: the block's, plus one [T, c_s] buffer
 * of singles (in `dtype`) when nblocks >= 2.
 */
nt_status nt_chain_workspace_bytes(const nt_partition* p, int32_t nblocks, int32_t c_s,
                                   int32_t c_z, int32_t hidden, nt_dtype dtype, size_t* bytes);

/*
 * nblocks blocks in sequence (Section 4.3, "A larger pair application": the
 * singles of each block feed the next, whose pair state is rebuilt from
 * them). w points to nblocks weight sets in host memory; the weights
 * themselves are on the device. s_out [T, c_s] receives the last block's
 * singles, z_out [cells, c_z] the last block's pair state (every block
 * writes it in turn). s_out may equal s_in. Square partitions only.
 * The blocks run nt_pair_block's launches in turn, and the results are
 * those of chained nt_pair_block calls, bit for bit.
 * workspace: device, at least nt_chain_workspace_bytes, 16-byte aligned,
 * disjoint from every other array. Errors as nt_pair_block; nothing is
 * launched when a check fails.
 */
nt_status nt_pair_chain(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                        const nt_block_weights* w, int32_t nblocks, int32_t c_s, int32_t c_z,
                        int32_t hidden, nt_dtype dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * The rectangular block (Appendix A.1's rectangular variant of Equation 1):
 * pair rows are built from s_rows [T, c_s], pair columns from s_cols
 * [T_cols, c_s]: a = s_rows Wa^T, b = s_cols Wb^T, z~ = transition(a[row] +
 * b[col]), m = column mean (divided by M_i), s_out = s_rows + m Wo^T. The
 * partition comes from nt_make_partition_rect (a square one works too, with
 * s_cols = s_rows giving nt_pair_block). s_out may equal s_rows, not s_cols.
 * Workspace as nt_pair_block (nt_block_workspace_bytes accounts for T_cols).
 */
nt_status nt_pair_block_rect(const nt_partition* p, const void* s_rows, const void* s_cols,
                             void* s_out, void* z_out, const nt_block_weights* w, int32_t c_s,
                             int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Blocks with the transition named explicitly (Equation 1, second line:
 * P~ = P + h(LN_{C_p}(P))). NT_TRANSITION_RELU_MLP is the two-layer ReLU
 * MLP without normalisation that nt_pair_block runs (the measured
 * workloads' update); NT_TRANSITION_LN_SWIGLU is the paper's own update, a
 * residual pre-normalised SwiGLU (Appendix A.1, expansion four):
 *   x = (z - mean) / sqrt(var + ln_eps) * ln_gamma + ln_beta
 *       (mean and biased var over the c_z features of a cell),
 *   z~ = z + (silu(x W_gate^T) * (x W_up^T)) W_down^T,  silu(g) = g / (1 + e^-g).
 * In the block z = a[row] + b[col] is formed in fp32 and never stored: LN
 * takes its statistics on it, x and the gated activations are rounded to
 * bf16 before the products that read them, and the residual adds z in fp32
 * (the pair state is rounded once, on output). NT_TRANSITION_LN_SWIGLU
 * needs dtype NT_BF16, c_z 64 or 128, hidden a multiple of 32 and a
 * finite ln_eps >= 0 (else NT_ERR_DTYPE / NT_ERR_INVALID).
 * ------------------------------------------------------------------------ */
typedef enum nt_transition_kind {
  NT_TRANSITION_RELU_MLP = 0,
  NT_TRANSITION_LN_SWIGLU = 1
} nt_transition_kind;

/*
 * One block's parameters. Wa, Wb, Wo as in nt_block_weights. RELU_MLP reads
 * W1 [hidden, c_z] and W2 [c_z, hidden]; LN_SWIGLU reads ln_gamma, ln_beta
 * (fp32 [c_z]), W_gate, W_up ([hidden, c_z]) and W_down ([c_z, hidden]), all
 * other weights in the block's dtype. Pointers the kind does not read may be
 * NULL.
 */
typedef struct nt_block_params {
  int32_t kind; /* nt_transition_kind */
  float ln_eps;
  const void* Wa;
  const void* Wb;
  const void* Wo;
  const void* W1;
  const void* W2;
  const float* ln_gamma;
  const float* ln_beta;
  const void* W_gate;
  const void* W_up;
  const void* W_down;
} nt_block_params;

/* fp32 gradients, shaped like the parameters; those the kind has no
 * parameter for are not written and may be NULL. */
typedef struct nt_block_param_grads {
  float* Wa;
  float* Wb;
  float* Wo;
  float* W1;
  float* W2;
  float* ln_gamma;
  float* ln_beta;
  float* W_gate;
  float* W_up;
  float* W_down;
} nt_block_param_grads;

/*
 * nt_pair_block with the transition of w->kind: projections, the broadcast
 * fused into the transition, the column mean, the output projection.
 * Workspace as nt_pair_block (nt_block_workspace_bytes); square or
 * rectangular partitions (rectangular: s_cols [T_cols, c_s] gives the
 * columns, s_cols = NULL means s_in). Other arguments and errors as
 * nt_pair_block.
 */
nt_status nt_pair_block_ex(const nt_partition* p, const void* s_in, const void* s_cols,
                           void* s_out, void* z_out, const nt_block_params* w, int32_t c_s,
                           int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * nt_pair_chain with nblocks parameter sets (each block's kind may differ).
 * Workspace as nt_pair_chain (nt_chain_workspace_bytes). Square partitions.
 */
nt_status nt_pair_chain_ex(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                           const nt_block_params* w, int32_t nblocks, int32_t c_s, int32_t c_z,
                           int32_t hidden, nt_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward pass and loss (Section 4: the measured step is forward, loss and
 * backward; Section 3.4: gradients reach the projections, the pair update
 * and the reduction of Equation 1 through the packed storage). Gradients
 * are fp32 whatever the storage type. With NT_BF16 the transition's products
 * read their operands rounded to bf16 (G, the hidden gradient g_H, the
 * hidden activations H) and accumulate in fp32, as the forward does.
 * ------------------------------------------------------------------------ */

/* The weight gradients of one block (fp32, [out, in] like the weights). */
typedef struct nt_block_grads {
  float* Wa;
  float* Wb;
  float* W1;
  float* W2;
  float* Wo;
} nt_block_grads;

/*
 * Workspace bytes nt_pair_loss_eq5 needs: one fp64 per single row.
 */
nt_status nt_loss_workspace_bytes(const nt_partition* p, size_t* bytes);

/*
 * The sample-weighted squared loss of Appendix A.1, Equation 5, over a
 * block's returned singles x [T, S, c_s] and pair state pz [cells, S, c_z]:
 *   L = sum_i alpha_i |x_i|^2 / (S c_s sum_i N_i)
 *     + sum_i beta_i |pz_i|^2 / (S c_z sum_i N_i M_i),
 *   alpha_i = 1 + i / B, beta_i = 1.5 - i / (2 B), i = 0 .. B - 1,
 * S is the static leading axis of the non-leading (S, N_i, C) layout, packed
 * inside each row (Eq. 2), 1 <= S <= 64; S = 1 is the leading layout. The
 * squares accumulate in fp32 per row and the rows' terms in fp64 into
 * *loss (device, one double). g_x [T, S, c_s] and g_pz [cells, S, c_z]
 * (fp32, either may be NULL) receive 2 alpha_i x / (S c_s sum N) and
 * 2 beta_i pz / (S c_z sum N M). Deterministic. workspace: device, at least
 * nt_loss_workspace_bytes, 16-byte aligned.
 */
nt_status nt_pair_loss_eq5(const nt_partition* p, const void* x, int32_t c_s, const void* pz,
                           int32_t c_z, int32_t S, nt_dtype dtype, double* loss, float* g_x,
                           float* g_pz, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Adjoint of the column mean (Equation 4 divided by M_i): every cell of pair
 * row r of sample i receives g_m[eta_i + r] / M_i, added to g_z_in when it
 * is not NULL:  G[o_i + r M_i + c] = g_z_in[...] + g_m[eta_i + r] / M_i.
 * g_m: fp32 [T, c_z]; g_z_in, G: fp32 [cells, c_z]; G may equal g_z_in.
 */
nt_status nt_pair_reduce_backward(const nt_partition* p, const float* g_m, const float* g_z_in,
                                  float* G, int32_t c_z, void* stream);

/*
 * Adjoint of the broadcast (Equation 1, first line): the row singles'
 * gradient sums each pair row over its columns and the column singles'
 * gradient sums each pair column over its rows:
 *   g_a[eta_i + r] = sum_c g_z[o_i + r M_i + c],
 *   g_b[mu_i + c]  = sum_r g_z[o_i + r M_i + c].
 * g_z: fp32 [cells, c_z]; g_a: fp32 [T, c_z]; g_b: fp32 [T_cols, c_z].
 * Deterministic (fixed summation order, no atomics).
 */
nt_status nt_pair_broadcast_backward(const nt_partition* p, const float* g_z, float* g_a,
                                     float* g_b, int32_t c_z, void* stream);

/*
 * Workspace bytes nt_pair_transition_backward needs.
 */
nt_status nt_transition_backward_workspace_bytes(const nt_partition* p, int32_t c_z,
                                                 int32_t hidden, nt_dtype dtype, size_t* bytes);

/*
 * Gradient of the residual transition z' = z + relu(z W1^T) W2^T for an
 * incoming G = dL/dz' (fp32 [cells, c_z]):
 *   pre = z W1^T, g_H = (G W2) * [pre > 0]   (relu'(0) = 0),
 *   g_z = G + g_H W1,  dW1 = g_H^T z,  dW2 = G^T relu(pre).
 * z: [cells, c_z] of `dtype` (the transition's input); W1: [hidden, c_z];
 * W2: [c_z, hidden]; g_z: fp32 [cells, c_z], may equal G; dW1: fp32
 * [hidden, c_z] and dW2: fp32 [c_z, hidden] are overwritten. The weight
 * gradients are contractions over all cells, summed in fixed order.
 * workspace: device, at least nt_transition_backward_workspace_bytes,
 * 16-byte aligned (it holds H and g_H per cell).
 */
nt_status nt_pair_transition_backward(const nt_partition* p, const void* z, const float* G,
                                      const void* W1, const void* W2, float* g_z, float* dW1,
                                      float* dW2, int32_t c_z, int32_t hidden, nt_dtype dtype,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes nt_pair_block_backward needs.
 */
nt_status nt_block_backward_workspace_bytes(const nt_partition* p, int32_t c_s, int32_t c_z,
                                            int32_t hidden, nt_dtype dtype, size_t* bytes);

/*
 * Backward of one square block (nt_pair_block) by the chain rule, step by
 * step in reverse: for incoming g_s_out = dL/ds~ (fp32 [T, c_s]) and,
 * optionally, g_z_out = dL/dz~ (fp32 [cells, c_z], NULL when the loss does
 * not read the pair state):
 *   g_m = g_s_out Wo,             dWo = g_s_out^T m,
 *   G = g_z_out + g_m[row] / N_i  (the mean's adjoint),
 *   g_z, dW1, dW2 = transition backward at z = a[row] + b[col],
 *   g_a, g_b = row and column sums of g_z,
 *   g_s_in = g_s_out + g_a Wa + g_b Wb,  dWa = g_a^T s,  dWb = g_b^T s.
 * s_in: the block's input singles [T, c_s]; z_out: its returned pair state
 * [cells, c_z] (m is recomputed from it); weights as for nt_pair_block.
 * g_s_in: fp32 [T, c_s], may equal g_s_out; grads: fp32 outputs,
 * overwritten. a, b and z are recomputed from s_in. workspace: device, at
 * least nt_block_backward_workspace_bytes, 16-byte aligned.
 */
nt_status nt_pair_block_backward(const nt_partition* p, const void* s_in, const void* z_out,
                                 const nt_block_weights* w, const float* g_s_out,
                                 const float* g_z_out, float* g_s_in, const nt_block_grads* grads,
                                 int32_t c_s, int32_t c_z, int32_t hidden, nt_dtype dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes nt_pair_block_backward_ex needs for a transition kind.
 */
nt_status nt_block_backward_ex_workspace_bytes(const nt_partition* p, int32_t kind, int32_t c_s,
                                               int32_t c_z, int32_t hidden, nt_dtype dtype,
                                               size_t* bytes);

/*
 * Backward of nt_pair_block_ex on a square partition, as
 * nt_pair_block_backward with the transition of w->kind. For
 * NT_TRANSITION_LN_SWIGLU the transition's adjoint, for G = dL/dz~, is
 * (g = x W_gate^T, u = x W_up^T, s = sigmoid(g), A = g s u):
 *   dW_down = G^T A,  g_A = G W_down,  g_u = g_A g s,  g_g = g_A u s (1 + g (1 - s)),
 *   dW_up = g_u^T x,  dW_gate = g_g^T x,  g_x = g_u W_up + g_g W_gate,
 *   dln_gamma = sum g_x xhat,  dln_beta = sum g_x,
 *   g_z = G + (g_xhat - mean(g_xhat) - xhat mean(g_xhat xhat)) / sqrt(var + ln_eps),
 *   g_xhat = g_x ln_gamma,  xhat = (z - mean) / sqrt(var + ln_eps),
 * with z re-formed in fp32 from the recomputed projections. At c_z 128,
 * hidden a multiple of 128 and bf16, the gate, value and g_A products read
 * x and G rounded to bf16 (the forward's operands) and the weight
 * contractions read them as bf16 pairs hi + lo (unrounded to about 2^-17);
 * other shapes read x and G unrounded in every product. A, g_u and g_g are
 * rounded to bf16; every product accumulates in fp32. The weight
 * gradients are sums over all cells in a fixed order. grads: the kind's
 * gradients, fp32, overwritten.
 */
nt_status nt_pair_block_backward_ex(const nt_partition* p, const void* s_in, const void* z_out,
                                    const nt_block_params* w, const float* g_s_out,
                                    const float* g_z_out, float* g_s_in,
                                    const nt_block_param_grads* grads, int32_t c_s, int32_t c_z,
                                    int32_t hidden, nt_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The non-leading layout (Appendix A.1's non-leading variant; Section 3.1,
 * Eq. 2: a sample with a static leading axis, singles (S, N_i, C) and pairs
 * (S, N_i, N_i, C_p), packs its ragged axes first, so every single row holds
 * S slices of c_s values and every pair cell S slices of c_z). Projections,
 * the transition and the output projection act per slice on the last axis,
 * the broadcast adds along the pair axes and the mean runs over columns, so
 * no step mixes the slices; the weights are shared by all of them. Square
 * partitions; 1 <= S <= 64 and S * c_z <= 512. With S > 1 the broadcast and
 * the transition run as two kernels (z rounded to the storage type between
 * them), the residual adding that rounded z.
 * ------------------------------------------------------------------------ */

/* Workspace bytes nt_pair_block_nl needs. */
nt_status nt_block_nl_workspace_bytes(const nt_partition* p, int32_t S, int32_t c_s, int32_t c_z,
                                      int32_t hidden, nt_dtype dtype, size_t* bytes);

/*
 * One block on the non-leading layout: s_in, s_out [T, S, c_s]; z_out
 * [cells, S, c_z]; weights as for nt_pair_block. s_out may equal s_in.
 * Errors as nt_pair_block, plus NT_ERR_INVALID for S out of range or a
 * rectangular partition.
 */
nt_status nt_pair_block_nl(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                           const nt_block_weights* w, int32_t S, int32_t c_s, int32_t c_z,
                           int32_t hidden, nt_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Workspace bytes nt_pair_block_backward_nl needs. */
nt_status nt_block_backward_nl_workspace_bytes(const nt_partition* p, int32_t S, int32_t c_s,
                                               int32_t c_z, int32_t hidden, nt_dtype dtype,
                                               size_t* bytes);

/*
 * Backward of nt_pair_block_nl, as nt_pair_block_backward with every single
 * array [T, S, ...] and pair array [cells, S, ...]; the weight gradients sum
 * over the slices.
 */
nt_status nt_pair_block_backward_nl(const nt_partition* p, const void* s_in, const void* z_out,
                                    const nt_block_weights* w, const float* g_s_out,
                                    const float* g_z_out, float* g_s_in,
                                    const nt_block_grads* grads, int32_t S, int32_t c_s,
                                    int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* nt_last_error(void);

/* Library ABI version: 1. */
int32_t nt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NT_PAIR_H */
