// C-ABI entry points: host-side validation, partition sizing, launch order.
// Every check runs before anything is enqueued, so a non-OK status leaves
// the stream and all outputs untouched.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "nt_internal.hpp"

namespace {

thread_local std::string g_last_error;

nt_status fail(nt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

nt_status ok() {
  g_last_error.clear();
  return NT_OK;
}

// Largest cell count accepted: keeps every launch grid within 2^31 blocks
// (a 2^34-cell pair state is 256 GiB even at 8 bf16 features per cell).
constexpr int64_t kMaxCells = int64_t(1) << 34;

size_t esize(nt_dtype d) { return d == NT_BF16 ? 2 : 4; }

nt_status check_dtype(nt_dtype d) {
  if (d != NT_F32 && d != NT_BF16) return fail(NT_ERR_DTYPE, "unknown dtype %d", (int)d);
  return NT_OK;
}

nt_status check_width(const char* name, int32_t v, int max) {
  if (v <= 0 || v % 8 != 0 || v > max)
    return fail(NT_ERR_INVALID, "%s = %d must be a positive multiple of 8 and at most %d", name,
                (int)v, max);
  return NT_OK;
}

// A device array of `bytes` bytes: NULL only when empty, 16-byte aligned.
nt_status check_array(const char* name, const void* ptr, uint64_t bytes) {
  if (bytes == 0) return NT_OK;
  if (!ptr) return fail(NT_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(NT_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return NT_OK;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

nt_status check_partition(const nt_partition* p) {
  if (!p) return fail(NT_ERR_NULL, "partition is NULL");
  if (p->magic != nt::kPartitionMagic)
    return fail(NT_ERR_INVALID, "partition was not built by nt_make_partition");
  if (p->B < 0 || p->T < 0 || p->cells < 0 || p->cells > kMaxCells || p->T > INT32_MAX)
    return fail(NT_ERR_INVALID, "partition sizes are corrupt");
  if (p->T_cols < 0 || p->T_cols > INT32_MAX)
    return fail(NT_ERR_INVALID, "partition sizes are corrupt");
  if (!p->single_offsets || !p->pair_offsets || !p->row_splits || !p->item_offsets ||
      !p->col_offsets || (p->B > 0 && (!p->lengths || !p->col_lengths)) ||
      (p->T > 0 && !p->row_sample) || (p->cells > 0 && !p->tile_sample))
    return fail(NT_ERR_NULL, "partition arrays are NULL");
  return NT_OK;
}

nt_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(NT_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return ok();
}

#define NT_TRY(expr)                      \
  do {                                    \
    const nt_status s_ = (expr);          \
    if (s_ != NT_OK) return s_;           \
  } while (0)

struct BlockWorkspace {
  uint64_t a, b, m, total;
};

// a and b are kept in fp32 (the projections' accumulators, unrounded), m too;
// b has one row per column single (T_cols, which is T for square pairs). In
// the non-leading layout every single row holds S slices.
BlockWorkspace block_workspace(int64_t T, int64_t T_cols, int c_z, nt_dtype, int S = 1) {
  BlockWorkspace w;
  const uint64_t a = nt::align256((size_t)T * S * c_z * sizeof(float));
  const uint64_t b = nt::align256((size_t)T_cols * S * c_z * sizeof(float));
  w.a = 0;
  w.b = a;
  w.m = a + b;
  w.total = a + b + a;
  return w;
}

// Totals of a partition with N_i = rows[i] pair rows of M_i = cols[i] cells
// (cols == rows for square pairs). Any output may be NULL.
nt_status partition_totals(const int32_t* rows, const int32_t* cols, int32_t B, int64_t* T_out,
                           int64_t* T_cols_out, int64_t* cells_out, int32_t* n_max_out) {
  if (B < 0) return fail(NT_ERR_INVALID, "B = %d is negative", (int)B);
  if (B > 0 && !rows) return fail(NT_ERR_NULL, "lengths is NULL");
  int64_t T = 0, T_cols = 0, cells = 0;
  int32_t n_max = 0;
  for (int32_t i = 0; i < B; ++i) {
    const int64_t n = rows[i], m = cols[i];
    if (n < 0) return fail(NT_ERR_INVALID, "length %d of sample %d is negative", (int)n, (int)i);
    if (m < 0)
      return fail(NT_ERR_INVALID, "column length %d of sample %d is negative", (int)m, (int)i);
    T += n;
    T_cols += m;
    if (T > INT32_MAX || T_cols > INT32_MAX)
      return fail(NT_ERR_OVERFLOW, "sum of lengths exceeds INT32_MAX");
    if (m > 0 && n > (kMaxCells - cells) / m)
      return fail(NT_ERR_OVERFLOW, "sum of pair cells exceeds %lld cells", (long long)kMaxCells);
    cells += n * m;
    if (n > n_max) n_max = (int32_t)n;
  }
  if (T_out) *T_out = T;
  if (T_cols_out) *T_cols_out = T_cols;
  if (cells_out) *cells_out = cells;
  if (n_max_out) *n_max_out = n_max;
  return ok();
}

nt_status make_partition(const int32_t* rows, const int32_t* cols, int32_t B, bool rect,
                         void* buffer, size_t buffer_bytes, void* stream, nt_partition* out) {
  if (!out) return fail(NT_ERR_NULL, "out is NULL");
  int64_t T = 0, T_cols = 0, cells = 0;
  int32_t n_max = 0;
  NT_TRY(partition_totals(rows, cols, B, &T, &T_cols, &cells, &n_max));
  const nt::PartitionLayout L = nt::partition_layout(B, T, cells, rect);
  if (!buffer) return fail(NT_ERR_NULL, "buffer is NULL");
  if (reinterpret_cast<uintptr_t>(buffer) % 256 != 0)
    return fail(NT_ERR_ALIGN, "partition buffer is not 256-byte aligned");
  if (buffer_bytes < L.total)
    return fail(NT_ERR_WORKSPACE, "partition buffer has %zu bytes, needs %zu", buffer_bytes,
                L.total);
  int64_t items = 0;
  for (int32_t i = 0; i < B; ++i) items += nt::items_of(rows[i], cols[i]);

  char* base = static_cast<char*>(buffer);
  nt_partition p;
  std::memset(&p, 0, sizeof(p));
  p.magic = nt::kPartitionMagic;
  p.B = B;
  p.n_max = n_max;
  p.T = T;
  p.T_cols = T_cols;
  p.cells = cells;
  p.n_items = items;
  int32_t* d_lengths = reinterpret_cast<int32_t*>(base + L.lengths);
  int32_t* d_cols = reinterpret_cast<int32_t*>(base + L.col_lengths);
  int64_t* d_eta = reinterpret_cast<int64_t*>(base + L.single_offsets);
  int64_t* d_mu = reinterpret_cast<int64_t*>(base + L.col_offsets);
  int64_t* d_o = reinterpret_cast<int64_t*>(base + L.pair_offsets);
  int64_t* d_items = reinterpret_cast<int64_t*>(base + L.item_offsets);
  int64_t* d_splits = reinterpret_cast<int64_t*>(base + L.row_splits);
  int32_t* d_rows = reinterpret_cast<int32_t*>(base + L.row_sample);
  int32_t* d_tiles = reinterpret_cast<int32_t*>(base + L.tile_sample);
  p.lengths = d_lengths;
  p.col_lengths = d_cols;
  p.single_offsets = d_eta;
  p.col_offsets = d_mu;
  p.pair_offsets = d_o;
  p.item_offsets = d_items;
  p.row_splits = d_splits;
  p.row_sample = d_rows;
  p.tile_sample = d_tiles;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B <= nt::kArgSamples) {
    NT_TRY(hip_status(nt::launch_partition_small(rows, cols, p, d_lengths, d_cols, d_eta, d_mu,
                                                 d_o, d_items, d_splits, d_rows, d_tiles, s),
                      "partition kernel"));
  } else {
    hipError_t e =
        hipMemcpyAsync(d_lengths, rows, sizeof(int32_t) * B, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && rect)
      e = hipMemcpyAsync(d_cols, cols, sizeof(int32_t) * B, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_status(e, "copying lengths");
    NT_TRY(hip_status(nt::launch_partition(p, d_eta, d_mu, d_o, d_items, d_splits, d_rows,
                                           d_tiles, s),
                      "partition kernels"));
  }
  *out = p;
  return ok();
}

// The partition seen by a cell-local kernel over rows of width c_z when each
// cell holds S of them (the non-leading layout): cells * S rows, no sample
// index (cell-local kernels without the fused broadcast do not decode).
nt_partition rows_view(const nt_partition& p, int S) {
  nt_partition v = p;
  v.cells = p.cells * S;
  v.tile_sample = nullptr;
  return v;
}

nt_status check_static_axis(int32_t S, int32_t c_z) {
  if (S < 1 || S > 64)
    return fail(NT_ERR_INVALID, "S = %d must be in [1, 64]", (int)S);
  if ((int64_t)S * c_z > nt::kMaxCz)
    return fail(NT_ERR_INVALID, "S * c_z = %d exceeds %d", (int)(S * c_z), nt::kMaxCz);
  return NT_OK;
}

// The ReLU-MLP weights of nt_block_weights as block parameters.
nt_block_params relu_params(const nt_block_weights& w) {
  nt_block_params q;
  std::memset(&q, 0, sizeof(q));
  q.kind = NT_TRANSITION_RELU_MLP;
  q.Wa = w.Wa;
  q.Wb = w.Wb;
  q.Wo = w.Wo;
  q.W1 = w.W1;
  q.W2 = w.W2;
  return q;
}

// The arrays a block's parameters consist of, by kind; checked for NULL and
// alignment, and returned for the overlap checks (at most 8).
struct ParamArrays {
  const char* name[8];
  const void* ptr[8];
  uint64_t bytes[8];
  int n = 0;
  void add(const char* nm, const void* p, uint64_t b) {
    name[n] = nm;
    ptr[n] = p;
    bytes[n] = b;
    ++n;
  }
};

nt_status check_params(const nt_block_params* w, int32_t c_s, int32_t c_z, int32_t hidden,
                       nt_dtype dtype, ParamArrays* out) {
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  const size_t es = esize(dtype);
  const uint64_t proj = (uint64_t)c_z * c_s * es, mlp = (uint64_t)c_z * hidden * es;
  ParamArrays a;
  a.add("Wa", w->Wa, proj);
  a.add("Wb", w->Wb, proj);
  a.add("Wo", w->Wo, proj);
  if (w->kind == NT_TRANSITION_RELU_MLP) {
    a.add("W1", w->W1, mlp);
    a.add("W2", w->W2, mlp);
  } else if (w->kind == NT_TRANSITION_LN_SWIGLU) {
    if (dtype != NT_BF16) return fail(NT_ERR_DTYPE, "the SwiGLU transition runs in bf16 only");
    if (!nt::transition_swiglu_supported(c_z, hidden, dtype))
      return fail(NT_ERR_INVALID, "SwiGLU transition needs c_z 64 or 128 and hidden a positive "
                                  "multiple of 32 (got c_z %d, hidden %d)", (int)c_z, (int)hidden);
    if (!(w->ln_eps >= 0.f) || w->ln_eps > 3.0e38f)
      return fail(NT_ERR_INVALID, "ln_eps must be finite and >= 0");
    a.add("ln_gamma", w->ln_gamma, (uint64_t)c_z * sizeof(float));
    a.add("ln_beta", w->ln_beta, (uint64_t)c_z * sizeof(float));
    a.add("W_gate", w->W_gate, mlp);
    a.add("W_up", w->W_up, mlp);
    a.add("W_down", w->W_down, mlp);
  } else {
    return fail(NT_ERR_INVALID, "unknown transition kind %d", (int)w->kind);
  }
  for (int k = 0; k < a.n; ++k) NT_TRY(check_array(a.name[k], a.ptr[k], a.bytes[k]));
  if (out) *out = a;
  return NT_OK;
}

// The transition of a block over its pair state: fused (z = a[row] + b[col]
// formed on chip) for S = 1, either kind, and for S slices per cell (ReLU)
// where the weight-stationary kernel takes the shape; else the broadcast
// over rows of S slices followed by the cell-local transition in place over
// cells * S rows.
nt_status block_transition(const nt_partition& p, const nt_block_params& w, const void* a,
                           const void* b, void* z_out, int32_t c_z, int32_t hidden,
                           nt_dtype dtype, int32_t S, hipStream_t s) {
  const bool swiglu = w.kind == NT_TRANSITION_LN_SWIGLU;
  if (S == 1) {
    if (swiglu)
      return hip_status(nt::launch_transition_swiglu(p, nullptr, a, b, z_out, w.ln_gamma,
                                                     w.ln_beta, w.W_gate, w.W_up, w.W_down, c_z,
                                                     hidden, w.ln_eps, s),
                        "fused broadcast + SwiGLU transition");
    return hip_status(nt::launch_transition(p, nullptr, a, b, z_out, w.W1, w.W2, c_z, hidden,
                                            dtype, s),
                      "fused broadcast + transition");
  }
  // S > 1: the non-leading layout, ReLU MLP only (checked by pair_block)
  if (nt::transition_ws_slices_supported(p, c_z, hidden, dtype, S))
    return hip_status(nt::launch_transition_ws(p, a, b, z_out, w.W1, w.W2, nt::device_cu_count(),
                                               s, S),
                      "fused broadcast + transition over slices");
  NT_TRY(hip_status(nt::launch_broadcast(p, a, b, z_out, S * c_z, dtype, s, true), "broadcast"));
  const nt_partition v = rows_view(p, S);
  return hip_status(nt::launch_transition(v, z_out, nullptr, nullptr, z_out, w.W1, w.W2, c_z,
                                          hidden, dtype, s),
                    "transition");
}

// One block; s_cols is s_rows for square partitions. S > 1: the non-leading
// layout (square partitions), rows of S slices.
nt_status pair_block(const nt_partition* p, const void* s_rows, const void* s_cols, void* s_out,
                     void* z_out, const nt_block_params* w, int32_t c_s, int32_t c_z,
                     int32_t hidden, nt_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* stream, int32_t S = 1) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  NT_TRY(check_static_axis(S, c_z));
  ParamArrays pa;
  NT_TRY(check_params(w, c_s, c_z, hidden, dtype, &pa));
  if (w->kind == NT_TRANSITION_LN_SWIGLU && S != 1)
    return fail(NT_ERR_INVALID, "the SwiGLU block takes the leading layout (S = 1)");
  const size_t es = esize(dtype);
  const uint64_t sbytes = (uint64_t)p->T * S * c_s * es;
  const uint64_t cbytes = (uint64_t)p->T_cols * S * c_s * es;
  const uint64_t pair = (uint64_t)p->cells * S * c_z * es;
  NT_TRY(check_array("s_rows", s_rows, sbytes));
  NT_TRY(check_array("s_cols", s_cols, cbytes));
  NT_TRY(check_array("s_out", s_out, sbytes));
  NT_TRY(check_array("z_out", z_out, pair));
  const BlockWorkspace ws = block_workspace(p->T, p->T_cols, c_z, dtype, S);
  if (ws.total > 0) {
    NT_TRY(check_array("workspace", workspace, ws.total));
    if (workspace_bytes < ws.total)
      return fail(NT_ERR_WORKSPACE, "workspace has %zu bytes, needs %llu", workspace_bytes,
                  (unsigned long long)ws.total);
  }
  if (s_rows != s_out && overlaps(s_rows, sbytes, s_out, sbytes))
    return fail(NT_ERR_INVALID, "s_out partially overlaps s_in");
  if (s_cols != s_rows && overlaps(s_out, sbytes, s_cols, cbytes))
    return fail(NT_ERR_INVALID, "s_out overlaps s_cols");
  if (overlaps(z_out, pair, s_rows, sbytes) || overlaps(z_out, pair, s_cols, cbytes) ||
      overlaps(z_out, pair, workspace, ws.total) || overlaps(s_out, sbytes, workspace, ws.total))
    return fail(NT_ERR_INVALID, "an output overlaps an input or the workspace");
  for (int k = 0; k < pa.n; ++k)
    if (overlaps(z_out, pair, pa.ptr[k], pa.bytes[k]) ||
        overlaps(s_out, sbytes, pa.ptr[k], pa.bytes[k]) ||
        overlaps(workspace, ws.total, pa.ptr[k], pa.bytes[k]))
      return fail(NT_ERR_INVALID, "an output or the workspace overlaps %s", pa.name[k]);
  if (overlaps(z_out, pair, s_out, sbytes))
    return fail(NT_ERR_INVALID, "z_out overlaps s_out");
  if (p->T == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  void* a = base + ws.a;
  void* b = base + ws.b;
  float* m = reinterpret_cast<float*>(base + ws.m);
  const int64_t TS = p->T * S;  // single rows of c_s values
  if (s_cols == s_rows && p->T_cols == p->T) {
    NT_TRY(hip_status(nt::launch_linear2(s_rows, dtype, w->Wa, w->Wb, a, b, TS, c_z, c_s, s),
                      "projections a, b"));
  } else {
    NT_TRY(hip_status(nt::launch_linear(s_rows, dtype, w->Wa, dtype, nullptr, a, NT_F32, p->T,
                                        c_z, c_s, s),
                      "projection a"));
    NT_TRY(hip_status(nt::launch_linear(s_cols, dtype, w->Wb, dtype, nullptr, b, NT_F32,
                                        p->T_cols, c_z, c_s, s),
                      "projection b"));
  }
  if (p->cells > 0) NT_TRY(block_transition(*p, *w, a, b, z_out, c_z, hidden, dtype, S, s));
  NT_TRY(hip_status(nt::launch_reduce(*p, z_out, m, S * c_z, dtype, s), "column mean"));
  return hip_status(nt::launch_linear(m, NT_F32, w->Wo, dtype, s_rows, s_out, dtype, TS, c_s,
                                      c_z, s),
                    "output projection");
}

// ---------------------------------------------------------------------------
// Backward helpers.

// One array of a call: outputs must not overlap anything else of the call.
struct Arr {
  const char* name;
  const void* ptr;
  uint64_t bytes;
  bool out;
};

// Every output is disjoint from every other array, except the pairs listed
// in `same` (index pairs that may be the identical pointer, e.g. in-place).
nt_status check_disjoint(const Arr* a, int n, const int (*same)[2] = nullptr, int nsame = 0) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j) {
      if (!a[i].out && !a[j].out) continue;
      bool allowed = false;
      for (int k = 0; k < nsame; ++k)
        if (((same[k][0] == i && same[k][1] == j) || (same[k][0] == j && same[k][1] == i)) &&
            a[i].ptr == a[j].ptr)
          allowed = true;
      if (!allowed && overlaps(a[i].ptr, a[i].bytes, a[j].ptr, a[j].bytes))
        return fail(NT_ERR_INVALID, "%s overlaps %s", a[i].name, a[j].name);
    }
  return NT_OK;
}

nt_status check_workspace(const void* ws, size_t have, uint64_t need) {
  if (need == 0) return NT_OK;
  NT_TRY(check_array("workspace", ws, need));
  if (have < need)
    return fail(NT_ERR_WORKSPACE, "workspace has %zu bytes, needs %llu", have,
                (unsigned long long)need);
  return NT_OK;
}

// Transition backward workspace: H and g_H per cell (storage type), G in the
// storage type (dW2 reads it after g_z may have overwritten G), the
// transposed weights, and the split partials of the weight gradients (both
// are hidden x c_z contractions over the cells).
struct TransBwdWs {
  uint64_t H, GH, Gb, W1T, W2T, part, gm_rows, total;
  int splits;
  bool mfma;  // the weight gradients run on the matrix cores
  bool rc;    // ... recomputing H and g_H from z and bf16(G) (no H, GH buffers)
};

// mean_rows: the pair rows whose mean adjoint the matrix-core kernel forms
// (T when called with g_m, else 0); their quotients g_m / M_i come last.
TransBwdWs transition_backward_ws(int64_t cells, int c_z, int hidden, nt_dtype dtype,
                                  int64_t mean_rows = 0) {
  TransBwdWs w;
  const uint64_t es = esize(dtype);
  w.rc = nt::wgrad_rc_supported(c_z, hidden, dtype);
  const uint64_t hb = w.rc ? 0 : nt::align256((size_t)cells * hidden * es);
  uint64_t off = 0;
  w.H = off;    off += hb;
  w.GH = off;   off += hb;
  w.Gb = off;   off += nt::align256((size_t)cells * c_z * es);
  w.W1T = off;  off += nt::align256((size_t)hidden * c_z * es);
  w.W2T = off;  off += nt::align256((size_t)hidden * c_z * es);
  w.mfma = dtype == NT_BF16 && nt::wgrad_supported(hidden, c_z);
  if (w.rc) {
    w.splits = nt::wgrad_rc_slices(cells);
    w.part = off; off += nt::align256((size_t)2 * w.splits * hidden * c_z * sizeof(float));
  } else {
    w.splits = w.mfma ? nt::wgrad_splits(cells, hidden, c_z)
                      : nt::gemm_tn_splits(cells, hidden, c_z);
    w.part = off; off += nt::align256((size_t)w.splits * hidden * c_z * sizeof(float));
  }
  w.gm_rows = off;
  if (nt::transition_backward_has_mfma(c_z, hidden, dtype))
    off += nt::align256((size_t)mean_rows * c_z * sizeof(float));
  w.total = off;
  return w;
}

// G given, or (g_m non-null) formed from the mean's adjoint g_m / M_i (+ g_in)
// by the matrix-core kernel; the generic path forms it first, into g_z.
nt_status transition_backward(const nt_partition* p, const void* z, const float* G,
                              const void* W1, const void* W2, float* g_z, float* dW1, float* dW2,
                              int c_z, int hidden, nt_dtype dtype, char* ws, hipStream_t s,
                              const float* g_m = nullptr, const float* g_in = nullptr) {
  const TransBwdWs w = transition_backward_ws(p->cells, c_z, hidden, dtype, g_m ? p->T : 0);
  void* H = w.rc ? nullptr : ws + w.H;
  void* GH = w.rc ? nullptr : ws + w.GH;
  void* Gb = ws + w.Gb;
  float* part = reinterpret_cast<float*>(ws + w.part);
  if (nt::transition_backward_has_mfma(c_z, hidden, dtype)) {
    void* W1T = ws + w.W1T;
    void* W2T = ws + w.W2T;
    NT_TRY(hip_status(nt::launch_transpose(W2, W2T, c_z, hidden, dtype, s), "transpose W2"));
    NT_TRY(hip_status(nt::launch_transpose(W1, W1T, hidden, c_z, dtype, s), "transpose W1"));
    NT_TRY(hip_status(nt::launch_transition_backward_mfma(
                          *p, z, G, g_m, g_in, W1, W2T, W1T, g_z, H, GH, Gb,
                          reinterpret_cast<float*>(ws + w.gm_rows), nt::device_cu_count(), s),
                      "transition backward"));
    if (w.rc)
      return hip_status(nt::launch_wgrad_rc(z, Gb, W1, W2T, dW1, dW2, part, p->cells, w.splits,
                                            s),
                        "weight gradients");
  } else {
    if (g_m) {
      NT_TRY(hip_status(nt::launch_mean_backward(*p, g_m, g_in, g_z, c_z, s), "mean backward"));
      G = g_z;
    }
    NT_TRY(hip_status(nt::launch_transition_backward_generic(*p, z, G, W1, W2, g_z, H, GH, Gb,
                                                             c_z, hidden, dtype, s),
                      "transition backward"));
  }
  // dW1 = g_H^T z ; dW2 = G^T H with G as stored in Gb
  if (w.mfma) {
    NT_TRY(hip_status(nt::launch_wgrad(GH, z, dW1, part, p->cells, hidden, c_z, w.splits, s),
                      "dW1 contraction"));
    return hip_status(nt::launch_wgrad(Gb, H, dW2, part, p->cells, c_z, hidden, w.splits, s),
                      "dW2 contraction");
  }
  NT_TRY(hip_status(nt::launch_gemm_tn(GH, dtype, z, dtype, dW1, part, p->cells, hidden, c_z,
                                       w.splits, s),
                    "dW1 contraction"));
  return hip_status(nt::launch_gemm_tn(Gb, dtype, H, dtype, dW2, part, p->cells, c_z, hidden,
                                       w.splits, s),
                    "dW2 contraction");
}

// SwiGLU transition gradient workspace (c_z 64 or 128, bf16): x = LN(z)
// (fp32), the gate and value pre-activations and the activation adjoint
// (fp32 [cells, hidden] each), their bf16 successors A, g_u, g_g, g_x
// (fp32), the transposed weights, and the partial sums of the weight
// gradients and of LN's parameter gradients.
struct SwigluBwdWs {
  uint64_t x, gp, up, ga, A, gu, gg, gx, WuT, WgT, WdT, wpart, lnpart, total;
  int wsplits, lnblocks;
};

SwigluBwdWs swiglu_backward_ws(int64_t cells, int c_z, int hidden) {
  SwigluBwdWs w;
  const uint64_t ch = (uint64_t)cells * hidden, cz = (uint64_t)cells * c_z;
  const uint64_t wbytes = nt::align256((size_t)hidden * c_z * 2);
  uint64_t off = 0;
  w.x = off;   off += nt::align256(cz * 4);
  w.gp = off;  off += nt::align256(ch * 4);
  w.up = off;  off += nt::align256(ch * 4);
  w.ga = off;  off += nt::align256(ch * 4);
  w.A = off;   off += nt::align256(ch * 2);
  w.gu = off;  off += nt::align256(ch * 2);
  w.gg = off;  off += nt::align256(ch * 2);
  w.gx = off;  off += nt::align256(cz * 4);
  w.WuT = off; off += wbytes;
  w.WgT = off; off += wbytes;
  w.WdT = off; off += wbytes;
  w.wsplits = nt::gemm_tn_splits(cells, c_z, hidden);
  w.wpart = off; off += nt::align256((size_t)w.wsplits * hidden * c_z * sizeof(float));
  w.lnblocks = nt::ln_backward_blocks(cells, c_z);
  w.lnpart = off; off += nt::align256((size_t)2 * w.lnblocks * c_z * sizeof(float));
  w.total = off;
  return w;
}

// Gradient of z~ = z + (silu(x Wg^T) * (x Wu^T)) Wd^T, x = LN(z), for G =
// dL/dz~ (fp32 [cells, c_z], replaced by g_z): z32 is the fp32 pair state.
// x and G enter the products unrounded (fp32 operands split into bf16 hi
// and lo parts on the matrix cores, fp32 contractions over the cells); the
// gate's outputs A, g_u, g_g are rounded to bf16.
nt_status swiglu_transition_backward(int64_t cells, const float* z32, float* G,
                                     const nt_block_params& w, const nt_block_param_grads& g,
                                     int c_z, int hidden, char* ws, hipStream_t s) {
  const SwigluBwdWs L = swiglu_backward_ws(cells, c_z, hidden);
  float* x = reinterpret_cast<float*>(ws + L.x);
  float* gp = reinterpret_cast<float*>(ws + L.gp);
  float* up = reinterpret_cast<float*>(ws + L.up);
  float* ga = reinterpret_cast<float*>(ws + L.ga);
  void *A = ws + L.A, *gu = ws + L.gu, *gg = ws + L.gg;
  float* gx = reinterpret_cast<float*>(ws + L.gx);
  void *WuT = ws + L.WuT, *WgT = ws + L.WgT, *WdT = ws + L.WdT;
  float* wpart = reinterpret_cast<float*>(ws + L.wpart);
  float* lnpart = reinterpret_cast<float*>(ws + L.lnpart);
  const float* gamma = w.ln_gamma;
  const int splits = L.wsplits;
  // forward pieces: x, then the gate and value pre-activations
  NT_TRY(hip_status(nt::launch_ln_rows(z32, gamma, w.ln_beta, x, cells, c_z, w.ln_eps, s),
                    "LN of the pair state"));
  NT_TRY(hip_status(nt::launch_linear(x, NT_F32, w.W_gate, NT_BF16, nullptr, gp, NT_F32, cells,
                                      hidden, c_z, s),
                    "gate product"));
  NT_TRY(hip_status(nt::launch_linear(x, NT_F32, w.W_up, NT_BF16, nullptr, up, NT_F32, cells,
                                      hidden, c_z, s),
                    "value product"));
  // g_A = G Wd, then the gate's adjoints
  NT_TRY(hip_status(nt::launch_transpose(w.W_down, WdT, c_z, hidden, NT_BF16, s),
                    "transpose W_down"));
  NT_TRY(hip_status(nt::launch_linear(G, NT_F32, WdT, NT_BF16, nullptr, ga, NT_F32, cells,
                                      hidden, c_z, s),
                    "g_A = G W_down"));
  NT_TRY(hip_status(nt::launch_swiglu_gate_bwd(gp, up, ga, A, gu, gg, cells * hidden, s),
                    "gate adjoints"));
  // the three weight gradients, contractions over the cells
  NT_TRY(hip_status(nt::launch_gemm_tn(G, NT_F32, A, NT_BF16, g.W_down, wpart, cells, c_z,
                                       hidden, splits, s),
                    "dW_down"));
  NT_TRY(hip_status(nt::launch_gemm_tn(gu, NT_BF16, x, NT_F32, g.W_up, wpart, cells, hidden, c_z,
                                       splits, s),
                    "dW_up"));
  NT_TRY(hip_status(nt::launch_gemm_tn(gg, NT_BF16, x, NT_F32, g.W_gate, wpart, cells, hidden,
                                       c_z, splits, s),
                    "dW_gate"));
  // g_x = g_u W_up + g_g W_gate
  NT_TRY(hip_status(nt::launch_transpose(w.W_up, WuT, hidden, c_z, NT_BF16, s),
                    "transpose W_up"));
  NT_TRY(hip_status(nt::launch_transpose(w.W_gate, WgT, hidden, c_z, NT_BF16, s),
                    "transpose W_gate"));
  NT_TRY(hip_status(nt::launch_linear(gu, NT_BF16, WuT, NT_BF16, nullptr, gx, NT_F32, cells, c_z,
                                      hidden, s),
                    "g_x = g_u W_up"));
  NT_TRY(hip_status(nt::launch_linear(gg, NT_BF16, WgT, NT_BF16, gx, gx, NT_F32, cells, c_z,
                                      hidden, s),
                    "g_x += g_g W_gate"));
  // LN's adjoint into G, and its parameters' gradients
  return hip_status(nt::launch_ln_backward(z32, gamma, gx, G, lnpart,
                                           lnpart + (size_t)L.lnblocks * c_z, g.ln_gamma,
                                           g.ln_beta, cells, c_z, w.ln_eps, s),
                    "LN backward");
}

// Workspace of the fused SwiGLU gradient (c_z 128, hidden a multiple of 128,
// bf16): the kernel's outputs x and G as bf16 pairs, A, g_u, g_g, the
// transposed weights, the LN parameters' workgroup sums, the weight
// contractions' split partials and their 2 c_z x hidden result.
struct SwigluBwd32Ws {
  uint64_t X2, G2, A, GU, GG, WdT, WuT, WgT, lnpart, wpart, ctmp, ttmp, total;
  int wsplits, grid;
};

SwigluBwd32Ws swiglu_backward32_ws(int64_t cells, int c_z, int hidden) {
  SwigluBwd32Ws w;
  // the kernel's outputs cover whole tiles
  const uint64_t rows = (uint64_t)nt::swiglu_bwd32_rows(cells);
  const uint64_t ch = rows * hidden, c2 = rows * 2 * c_z;
  const uint64_t wbytes = nt::align256((size_t)hidden * c_z * 2);
  const uint64_t mn2 = (uint64_t)2 * c_z * hidden;  // the [hi | lo] contractions
  uint64_t off = 0;
  w.X2 = off;  off += nt::align256(c2 * 2);
  w.G2 = off;  off += nt::align256(c2 * 2);
  w.A = off;   off += nt::align256(ch * 2);
  w.GU = off;  off += nt::align256(ch * 2);
  w.GG = off;  off += nt::align256(ch * 2);
  w.WdT = off; off += wbytes;
  w.WuT = off; off += wbytes;
  w.WgT = off; off += wbytes;
  w.grid = nt::swiglu_bwd32_grid(cells);
  w.lnpart = off; off += nt::align256((size_t)2 * (w.grid > 0 ? w.grid : 1) * c_z * 4);
  w.wsplits = nt::wgrad_splits(cells, 2 * c_z, hidden);
  w.wpart = off; off += nt::align256((size_t)w.wsplits * mn2 * 4);
  w.ctmp = off;  off += nt::align256(mn2 * 4);
  w.ttmp = off;  off += nt::align256((size_t)c_z * hidden * 4);
  w.total = off;
  return w;
}

// The fused SwiGLU gradient: G (fp32 [cells, c_z]) becomes g_z; a and b are
// the block's fp32 projections (the kernel forms the pair state per cell).
// The weight gradients are contractions over the cells on the matrix cores,
// with x and G as bf16 pairs: C = [hi; lo]^T B (2 c_z rows), then the two
// halves added (and transposed for dWu, dWg, whose rows are the units).
nt_status swiglu_transition_backward32(const nt_partition* p, const float* a, const float* b,
                                       float* G, const nt_block_params& w,
                                       const nt_block_param_grads& g, int c_z, int hidden,
                                       char* ws, hipStream_t s) {
  const SwigluBwd32Ws L = swiglu_backward32_ws(p->cells, c_z, hidden);
  void *X2 = ws + L.X2, *G2 = ws + L.G2, *A = ws + L.A, *GU = ws + L.GU, *GG = ws + L.GG;
  void *WdT = ws + L.WdT, *WuT = ws + L.WuT, *WgT = ws + L.WgT;
  float* lnpart = reinterpret_cast<float*>(ws + L.lnpart);
  float* wpart = reinterpret_cast<float*>(ws + L.wpart);
  float* ctmp = reinterpret_cast<float*>(ws + L.ctmp);
  float* ttmp = reinterpret_cast<float*>(ws + L.ttmp);
  const int64_t cz_h = (int64_t)c_z * hidden;
  NT_TRY(hip_status(nt::launch_transpose(w.W_down, WdT, c_z, hidden, NT_BF16, s),
                    "transpose W_down"));
  NT_TRY(hip_status(nt::launch_transpose(w.W_up, WuT, hidden, c_z, NT_BF16, s),
                    "transpose W_up"));
  NT_TRY(hip_status(nt::launch_transpose(w.W_gate, WgT, hidden, c_z, NT_BF16, s),
                    "transpose W_gate"));
  NT_TRY(hip_status(nt::launch_swiglu_bwd32(*p, a, b, w.ln_gamma, w.ln_beta, w.W_gate, w.W_up,
                                            WdT, WuT, WgT, G, X2, G2, A, GU, GG, lnpart, hidden,
                                            w.ln_eps, s),
                    "fused SwiGLU gradient"));
  const int grid = L.grid;
  NT_TRY(hip_status(nt::launch_sum_splits(lnpart, g.ln_gamma, grid, c_z, s), "dln_gamma"));
  NT_TRY(hip_status(nt::launch_sum_splits(lnpart + (size_t)grid * c_z, g.ln_beta, grid, c_z, s),
                    "dln_beta"));
  // dWd [c_z, hidden] = G^T A
  const int64_t rows = nt::swiglu_bwd32_rows(p->cells);  // the chunk-major operands
  NT_TRY(hip_status(nt::launch_wgrad(G2, A, ctmp, wpart, p->cells, 2 * c_z, hidden, L.wsplits,
                                     s, rows),
                    "dW_down contraction"));
  NT_TRY(hip_status(nt::launch_sum_splits(ctmp, g.W_down, 2, cz_h, s), "dW_down halves"));
  // dWu^T, dWg^T [c_z, hidden] = x^T g_u, x^T g_g
  const struct { void* B; float* out; const char* what; } wg[2] = {
      {GU, g.W_up, "dW_up"}, {GG, g.W_gate, "dW_gate"}};
  for (const auto& q : wg) {
    NT_TRY(hip_status(nt::launch_wgrad(X2, q.B, ctmp, wpart, p->cells, 2 * c_z, hidden,
                                       L.wsplits, s, rows),
                      q.what));
    NT_TRY(hip_status(nt::launch_sum_splits(ctmp, ttmp, 2, cz_h, s), q.what));
    NT_TRY(hip_status(nt::launch_transpose(ttmp, q.out, c_z, hidden, NT_F32, s), q.what));
  }
  return ok();
}

// Block backward workspace (square partitions): a, b (fp32), z (storage
// type), m, g_m, G (fp32; G becomes g_z in place), g_a, g_b (fp32), the
// transposed projection weights, the projections' split partials, then the
// transition backward's own workspace.
struct BlockBwdWs {
  uint64_t a, b, z, m, g_m, G, g_a, g_b, WoT, WaT, WbT, ppart, adj, trans, total;
  int psplits;
};

BlockBwdWs block_backward_ws(const nt_partition* p, int c_s, int c_z, int hidden,
                             nt_dtype dtype, int S = 1, int kind = NT_TRANSITION_RELU_MLP) {
  const bool swiglu = kind == NT_TRANSITION_LN_SWIGLU;
  BlockBwdWs w;
  const uint64_t es = esize(dtype);
  const int64_t TS = p->T * S, CS = p->cells * S;  // rows of c_s / c_z values
  const uint64_t single = nt::align256((size_t)TS * c_z * sizeof(float));
  const uint64_t proj = nt::align256((size_t)c_s * c_z * es);
  uint64_t off = 0;
  w.a = off;     off += single;
  w.b = off;     off += single;
  // the unfused SwiGLU gradient reads the pair state in fp32 (LN's
  // statistics); the fused one forms it per cell and needs none
  const bool fused = swiglu && S == 1 && nt::swiglu_bwd32_supported(c_z, hidden, dtype);
  w.z = off;     off += fused ? 0 : nt::align256((size_t)CS * c_z * (swiglu ? 4 : es));
  w.m = off;     off += single;
  w.g_m = off;   off += single;
  w.G = off;     off += nt::align256((size_t)CS * c_z * sizeof(float));
  w.g_a = off;   off += single;
  w.g_b = off;   off += single;
  w.WoT = off;   off += proj;
  w.WaT = off;   off += proj;
  w.WbT = off;   off += proj;
  w.psplits = nt::gemm_tn_splits(TS, c_z, c_s);
  w.ppart = off; off += nt::align256((size_t)w.psplits * c_s * c_z * sizeof(float));
  w.adj = off;   off += nt::align256(nt::bcast_adj_ws_bytes(*p, S * c_z));
  w.trans = off;
  off += fused    ? swiglu_backward32_ws(CS, c_z, hidden).total
         : swiglu ? swiglu_backward_ws(CS, c_z, hidden).total
                  : transition_backward_ws(CS, c_z, hidden, dtype, S == 1 ? p->T : 0).total;
  w.total = off;
  return w;
}

nt_status check_widths(int32_t c_s, int32_t c_z, int32_t hidden) {
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  return check_width("hidden", hidden, nt::kMaxHidden);
}

}  // namespace

extern "C" {

const char* nt_last_error(void) { return g_last_error.c_str(); }

int32_t nt_version(void) { return 1; }

nt_status nt_partition_sizes(const int32_t* lengths, int32_t B, int64_t* T_out, int64_t* cells_out,
                             int32_t* n_max_out, size_t* bytes_out) {
  int64_t T = 0, cells = 0;
  int32_t n_max = 0;
  NT_TRY(partition_totals(lengths, lengths, B, &T, nullptr, &cells, &n_max));
  if (T_out) *T_out = T;
  if (cells_out) *cells_out = cells;
  if (n_max_out) *n_max_out = n_max;
  if (bytes_out) *bytes_out = nt::partition_layout(B, T, cells).total;
  return ok();
}

nt_status nt_partition_sizes_rect(const int32_t* rows, const int32_t* cols, int32_t B,
                                  int64_t* T_out, int64_t* T_cols_out, int64_t* cells_out,
                                  size_t* bytes_out) {
  int64_t T = 0, T_cols = 0, cells = 0;
  NT_TRY(partition_totals(rows, cols, B, &T, &T_cols, &cells, nullptr));
  if (T_out) *T_out = T;
  if (T_cols_out) *T_cols_out = T_cols;
  if (cells_out) *cells_out = cells;
  if (bytes_out) *bytes_out = nt::partition_layout(B, T, cells, true).total;
  return ok();
}

nt_status nt_make_partition(const int32_t* lengths, int32_t B, void* buffer, size_t buffer_bytes,
                            void* stream, nt_partition* out) {
  return make_partition(lengths, lengths, B, false, buffer, buffer_bytes, stream, out);
}

nt_status nt_make_partition_rect(const int32_t* rows, const int32_t* cols, int32_t B, void* buffer,
                                 size_t buffer_bytes, void* stream, nt_partition* out) {
  if (B > 0 && !cols) return fail(NT_ERR_NULL, "cols is NULL");
  return make_partition(rows, cols, B, true, buffer, buffer_bytes, stream, out);
}

nt_status nt_decode_cells(const nt_partition* p, int32_t* sample, int32_t* row, int32_t* col,
                          void* stream) {
  NT_TRY(check_partition(p));
  const uint64_t bytes = (uint64_t)p->cells * sizeof(int32_t);
  NT_TRY(check_array("sample", sample, bytes));
  NT_TRY(check_array("row", row, bytes));
  NT_TRY(check_array("col", col, bytes));
  return hip_status(nt::launch_decode(*p, sample, row, col, static_cast<hipStream_t>(stream)),
                    "decode kernel");
}

nt_status nt_pair_broadcast(const nt_partition* p, const void* a, const void* b, void* z,
                            int32_t c_z, nt_dtype dtype, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  const uint64_t single = (uint64_t)p->T * c_z * esize(dtype);
  const uint64_t bsingle = (uint64_t)p->T_cols * c_z * esize(dtype);
  const uint64_t pair = (uint64_t)p->cells * c_z * esize(dtype);
  NT_TRY(check_array("a", a, single));
  NT_TRY(check_array("b", b, bsingle));
  NT_TRY(check_array("z", z, pair));
  if (overlaps(z, pair, a, single) || overlaps(z, pair, b, bsingle))
    return fail(NT_ERR_INVALID, "z overlaps a or b");
  return hip_status(
      nt::launch_broadcast(*p, a, b, z, c_z, dtype, static_cast<hipStream_t>(stream)),
      "broadcast kernel");
}

nt_status nt_pair_transition(const nt_partition* p, const void* z_in, void* z_out, const void* W1,
                             const void* W2, int32_t c_z, int32_t hidden, nt_dtype dtype,
                             void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  const uint64_t pair = (uint64_t)p->cells * c_z * esize(dtype);
  const uint64_t wbytes = (uint64_t)hidden * c_z * esize(dtype);
  NT_TRY(check_array("z_in", z_in, pair));
  NT_TRY(check_array("z_out", z_out, pair));
  NT_TRY(check_array("W1", W1, wbytes));
  NT_TRY(check_array("W2", W2, wbytes));
  if (z_in != z_out && overlaps(z_in, pair, z_out, pair))
    return fail(NT_ERR_INVALID, "z_out partially overlaps z_in");
  if (overlaps(z_out, pair, W1, wbytes) || overlaps(z_out, pair, W2, wbytes))
    return fail(NT_ERR_INVALID, "z_out overlaps a weight");
  if (p->cells == 0) return ok();
  return hip_status(nt::launch_transition(*p, z_in, nullptr, nullptr, z_out, W1, W2, c_z, hidden,
                                          dtype, static_cast<hipStream_t>(stream)),
                    "transition kernel");
}

nt_status nt_pair_transition_swiglu(const nt_partition* p, const void* z_in, void* z_out,
                                    const float* ln_gamma, const float* ln_beta,
                                    const void* W_gate, const void* W_up, const void* W_down,
                                    int32_t c_z, int32_t hidden, float ln_eps, nt_dtype dtype,
                                    void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  if (dtype != NT_BF16) return fail(NT_ERR_DTYPE, "the SwiGLU transition runs in bf16 only");
  if (!nt::transition_swiglu_supported(c_z, hidden, dtype))
    return fail(NT_ERR_INVALID, "SwiGLU transition needs c_z 64 or 128 and hidden a positive "
                                "multiple of 32 (got c_z %d, hidden %d)", (int)c_z, (int)hidden);
  if (!(ln_eps >= 0.f) || ln_eps > 3.0e38f)
    return fail(NT_ERR_INVALID, "ln_eps must be finite and >= 0");
  const uint64_t pair = (uint64_t)p->cells * c_z * esize(dtype);
  const uint64_t wbytes = (uint64_t)hidden * c_z * esize(dtype);
  const uint64_t lnbytes = (uint64_t)c_z * sizeof(float);
  NT_TRY(check_array("z_in", z_in, pair));
  NT_TRY(check_array("z_out", z_out, pair));
  NT_TRY(check_array("ln_gamma", ln_gamma, lnbytes));
  NT_TRY(check_array("ln_beta", ln_beta, lnbytes));
  NT_TRY(check_array("W_gate", W_gate, wbytes));
  NT_TRY(check_array("W_up", W_up, wbytes));
  NT_TRY(check_array("W_down", W_down, wbytes));
  if (z_in != z_out && overlaps(z_in, pair, z_out, pair))
    return fail(NT_ERR_INVALID, "z_out partially overlaps z_in");
  if (overlaps(z_out, pair, W_gate, wbytes) || overlaps(z_out, pair, W_up, wbytes) ||
      overlaps(z_out, pair, W_down, wbytes) || overlaps(z_out, pair, ln_gamma, lnbytes) ||
      overlaps(z_out, pair, ln_beta, lnbytes))
    return fail(NT_ERR_INVALID, "z_out overlaps a parameter");
  if (p->cells == 0) return ok();
  return hip_status(nt::launch_transition_swiglu(*p, z_in, nullptr, nullptr, z_out, ln_gamma,
                                                 ln_beta, W_gate, W_up, W_down, c_z, hidden,
                                                 ln_eps,
                                                 static_cast<hipStream_t>(stream)),
                    "SwiGLU transition kernel");
}

nt_status nt_pair_broadcast_transition(const nt_partition* p, const void* a, const void* b,
                                       void* z_out, const void* W1, const void* W2, int32_t c_z,
                                       int32_t hidden, nt_dtype dtype, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  const uint64_t single = (uint64_t)p->T * c_z * sizeof(float);
  const uint64_t bsingle = (uint64_t)p->T_cols * c_z * sizeof(float);
  const uint64_t pair = (uint64_t)p->cells * c_z * esize(dtype);
  const uint64_t wbytes = (uint64_t)hidden * c_z * esize(dtype);
  NT_TRY(check_array("a", a, single));
  NT_TRY(check_array("b", b, bsingle));
  NT_TRY(check_array("z_out", z_out, pair));
  NT_TRY(check_array("W1", W1, wbytes));
  NT_TRY(check_array("W2", W2, wbytes));
  if (overlaps(z_out, pair, a, single) || overlaps(z_out, pair, b, bsingle) ||
      overlaps(z_out, pair, W1, wbytes) || overlaps(z_out, pair, W2, wbytes))
    return fail(NT_ERR_INVALID, "z_out overlaps an input");
  if (p->cells == 0) return ok();
  return hip_status(nt::launch_transition(*p, nullptr, a, b, z_out, W1, W2, c_z, hidden, dtype,
                                          static_cast<hipStream_t>(stream)),
                    "fused broadcast + transition kernel");
}

nt_status nt_pair_reduce(const nt_partition* p, const void* z, float* m, int32_t c_z,
                         nt_dtype dtype, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  const uint64_t pair = (uint64_t)p->cells * c_z * esize(dtype);
  const uint64_t mbytes = (uint64_t)p->T * c_z * sizeof(float);
  NT_TRY(check_array("z", z, pair));
  NT_TRY(check_array("m", m, mbytes));
  if (overlaps(z, pair, m, mbytes)) return fail(NT_ERR_INVALID, "m overlaps z");
  return hip_status(nt::launch_reduce(*p, z, m, c_z, dtype, static_cast<hipStream_t>(stream)),
                    "reduce kernel");
}

nt_status nt_block_workspace_bytes(const nt_partition* p, int32_t c_s, int32_t c_z,
                                   int32_t hidden, nt_dtype dtype, size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = block_workspace(p->T, p->T_cols, c_z, dtype).total;
  return ok();
}

nt_status nt_pair_block(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                        const nt_block_weights* w, int32_t c_s, int32_t c_z, int32_t hidden,
                        nt_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  NT_TRY(check_partition(p));
  if (p->col_offsets != p->single_offsets)
    return fail(NT_ERR_INVALID, "rectangular partition: use nt_pair_block_rect");
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  const nt_block_params q = relu_params(*w);
  return pair_block(p, s_in, s_in, s_out, z_out, &q, c_s, c_z, hidden, dtype, workspace,
                    workspace_bytes, stream);
}

nt_status nt_pair_block_ex(const nt_partition* p, const void* s_in, const void* s_cols,
                           void* s_out, void* z_out, const nt_block_params* w, int32_t c_s,
                           int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  NT_TRY(check_partition(p));
  const bool rect = p->col_offsets != p->single_offsets;
  if (!s_cols) s_cols = s_in;
  if (!rect && s_cols != s_in)
    return fail(NT_ERR_INVALID, "s_cols must be NULL or s_in for a square partition");
  return pair_block(p, s_in, s_cols, s_out, z_out, w, c_s, c_z, hidden, dtype, workspace,
                    workspace_bytes, stream);
}

nt_status nt_pair_block_noalloc(const nt_partition* p, const void* s_in, void* s_out,
                                void* z_out, const nt_block_weights* w, int32_t c_s, int32_t c_z,
                                int32_t hidden, nt_dtype dtype, void* stream) {
  NT_TRY(check_partition(p));
  if (p->col_offsets != p->single_offsets)
    return fail(NT_ERR_INVALID, "rectangular partition: use nt_pair_block_rect");
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_widths(c_s, c_z, hidden));
  const uint64_t need = block_workspace(p->T, p->T_cols, c_z, dtype).total;
  if (need > nt::kStaticScratchBytes)
    return fail(NT_ERR_WORKSPACE,
                "the block needs %llu bytes of scratch (T = %lld rows of 3 x c_z fp32 values); "
                "the static scratch holds %zu: use nt_pair_block with a workspace",
                (unsigned long long)need, (long long)p->T, nt::kStaticScratchBytes);
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  const nt_block_params q = relu_params(*w);
  void* ws = nullptr;
  NT_TRY(hip_status(nt::static_scratch(&ws), "static scratch address"));
  return pair_block(p, s_in, s_in, s_out, z_out, &q, c_s, c_z, hidden, dtype, ws,
                    nt::kStaticScratchBytes, stream);
}

// Chain workspace: the block's, then (for two or more blocks) one bf16/fp32
// buffer of T x c_s singles that the chain alternates with s_out.
static uint64_t chain_workspace(const nt_partition* p, int32_t nblocks, int32_t c_s, int32_t c_z,
                         nt_dtype dtype) {
  const uint64_t blk = block_workspace(p->T, p->T_cols, c_z, dtype).total;
  return blk + (nblocks > 1 ? nt::align256((size_t)p->T * c_s * esize(dtype)) : 0);
}

nt_status nt_chain_workspace_bytes(const nt_partition* p, int32_t nblocks, int32_t c_s,
                                   int32_t c_z, int32_t hidden, nt_dtype dtype, size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  if (nblocks < 1) return fail(NT_ERR_INVALID, "nblocks = %d must be at least 1", (int)nblocks);
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = chain_workspace(p, nblocks, c_s, c_z, dtype);
  return ok();
}

// nblocks blocks in sequence; params(k) gives block k's parameters.
}  // extern "C"
template <typename Params>
nt_status pair_chain(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                     Params params, int32_t nblocks, int32_t c_s, int32_t c_z, int32_t hidden,
                     nt_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  if (p->col_offsets != p->single_offsets)
    return fail(NT_ERR_INVALID, "rectangular partition: chain nt_pair_block_rect calls");
  if (nblocks < 1) return fail(NT_ERR_INVALID, "nblocks = %d must be at least 1", (int)nblocks);
  const size_t es = esize(dtype);
  const uint64_t sbytes = (uint64_t)p->T * c_s * es;
  const uint64_t pair = (uint64_t)p->cells * c_z * es;
  const uint64_t blk = block_workspace(p->T, p->T_cols, c_z, dtype).total;
  const uint64_t need = chain_workspace(p, nblocks, c_s, c_z, dtype);
  NT_TRY(check_array("s_in", s_in, sbytes));
  NT_TRY(check_array("s_out", s_out, sbytes));
  NT_TRY(check_array("z_out", z_out, pair));
  if (need > 0) {
    NT_TRY(check_array("workspace", workspace, need));
    if (workspace_bytes < need)
      return fail(NT_ERR_WORKSPACE, "workspace has %zu bytes, needs %llu", workspace_bytes,
                  (unsigned long long)need);
  }
  if (s_in != s_out && overlaps(s_in, sbytes, s_out, sbytes))
    return fail(NT_ERR_INVALID, "s_out partially overlaps s_in");
  const void* outs[] = {s_out, z_out, workspace};
  const uint64_t outsz[] = {sbytes, pair, need};
  for (int k = 0; k < nblocks; ++k) {
    ParamArrays pa;
    const nt_block_params* q = params(k);
    if (!q) return fail(NT_ERR_NULL, "weights is NULL");
    NT_TRY(check_params(q, c_s, c_z, hidden, dtype, &pa));
    for (int j = 0; j < pa.n; ++j)
      for (int o = 0; o < 3; ++o)
        if (overlaps(outs[o], outsz[o], pa.ptr[j], pa.bytes[j]))
          return fail(NT_ERR_INVALID, "block %d's %s overlaps an output or the workspace", k,
                      pa.name[j]);
  }
  if (overlaps(z_out, pair, s_in, sbytes) || overlaps(z_out, pair, s_out, sbytes) ||
      overlaps(workspace, need, s_in, sbytes) || overlaps(workspace, need, s_out, sbytes) ||
      overlaps(workspace, need, z_out, pair))
    return fail(NT_ERR_INVALID, "z_out, the singles and the workspace must not overlap");
  if (p->T == 0) return ok();

  char* base = static_cast<char*>(workspace);
  void* sbuf = base + blk;
  // block k writes s_out when nblocks - 1 - k is even, else the workspace
  // buffer, so that the last block writes s_out
  auto dest = [&](int k) -> void* { return (nblocks - 1 - k) % 2 == 0 ? s_out : sbuf; };
  const void* cur = s_in;
  for (int k = 0; k < nblocks; ++k) {
    NT_TRY(pair_block(p, cur, cur, dest(k), z_out, params(k), c_s, c_z, hidden, dtype,
                      workspace, blk, stream));
    cur = dest(k);
  }
  return ok();
}
extern "C" {

nt_status nt_pair_chain(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                        const nt_block_weights* w, int32_t nblocks, int32_t c_s, int32_t c_z,
                        int32_t hidden, nt_dtype dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  if (nblocks < 1) return fail(NT_ERR_INVALID, "nblocks = %d must be at least 1", (int)nblocks);
  std::vector<nt_block_params> q(nblocks);
  for (int k = 0; k < nblocks; ++k) q[k] = relu_params(w[k]);
  return pair_chain(p, s_in, s_out, z_out, [&](int k) { return &q[k]; }, nblocks, c_s, c_z,
                    hidden, dtype, workspace, workspace_bytes, stream);
}

nt_status nt_pair_chain_ex(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                           const nt_block_params* w, int32_t nblocks, int32_t c_s, int32_t c_z,
                           int32_t hidden, nt_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  return pair_chain(p, s_in, s_out, z_out, [&](int k) { return &w[k]; }, nblocks, c_s, c_z,
                    hidden, dtype, workspace, workspace_bytes, stream);
}

nt_status nt_pair_block_rect(const nt_partition* p, const void* s_rows, const void* s_cols,
                             void* s_out, void* z_out, const nt_block_weights* w, int32_t c_s,
                             int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  const nt_block_params q = relu_params(*w);
  return pair_block(p, s_rows, s_cols, s_out, z_out, &q, c_s, c_z, hidden, dtype, workspace,
                    workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Backward pass and loss.

nt_status nt_loss_workspace_bytes(const nt_partition* p, size_t* bytes) {
  NT_TRY(check_partition(p));
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = nt::align256((size_t)(p->T > 0 ? p->T : 1) * sizeof(double));
  return ok();
}

nt_status nt_pair_loss_eq5(const nt_partition* p, const void* x, int32_t c_s, const void* pz,
                           int32_t c_z, int32_t S, nt_dtype dtype, double* loss, float* g_x,
                           float* g_pz, void* workspace, size_t workspace_bytes, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  if (S < 1) return fail(NT_ERR_INVALID, "S = %d must be at least 1", (int)S);
  if (S > 64) return fail(NT_ERR_INVALID, "S = %d must be at most 64", (int)S);
  const uint64_t es = esize(dtype);
  const uint64_t xw = (uint64_t)S * c_s, pw = (uint64_t)S * c_z;  // values per row
  const uint64_t xb = (uint64_t)p->T * xw * es, pb = (uint64_t)p->cells * pw * es;
  const uint64_t gxb = (uint64_t)p->T * xw * 4, gpb = (uint64_t)p->cells * pw * 4;
  const uint64_t need = nt::align256((size_t)(p->T > 0 ? p->T : 1) * sizeof(double));
  NT_TRY(check_array("x", x, xb));
  NT_TRY(check_array("pz", pz, pb));
  NT_TRY(check_array("loss", loss, sizeof(double)));
  if (g_x) NT_TRY(check_array("g_x", g_x, gxb));
  if (g_pz) NT_TRY(check_array("g_pz", g_pz, gpb));
  NT_TRY(check_workspace(workspace, workspace_bytes, need));
  const Arr arrs[] = {{"x", x, xb, false},           {"pz", pz, pb, false},
                      {"loss", loss, sizeof(double), true}, {"g_x", g_x, g_x ? gxb : 0, true},
                      {"g_pz", g_pz, g_pz ? gpb : 0, true}, {"workspace", workspace, need, true}};
  NT_TRY(check_disjoint(arrs, 6));
  return hip_status(nt::launch_loss_eq5(*p, x, c_s, pz, c_z, S, dtype,
                                        static_cast<double*>(workspace), loss, g_x, g_pz,
                                        static_cast<hipStream_t>(stream)),
                    "loss kernels");
}

nt_status nt_pair_reduce_backward(const nt_partition* p, const float* g_m, const float* g_z_in,
                                  float* G, int32_t c_z, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  const uint64_t mb = (uint64_t)p->T * c_z * 4, gb = (uint64_t)p->cells * c_z * 4;
  NT_TRY(check_array("g_m", g_m, mb));
  if (g_z_in) NT_TRY(check_array("g_z_in", g_z_in, gb));
  NT_TRY(check_array("G", G, gb));
  const Arr arrs[] = {{"g_m", g_m, mb, false}, {"g_z_in", g_z_in, g_z_in ? gb : 0, false},
                      {"G", G, gb, true}};
  const int same[][2] = {{1, 2}};
  NT_TRY(check_disjoint(arrs, 3, same, 1));
  return hip_status(
      nt::launch_mean_backward(*p, g_m, g_z_in, G, c_z, static_cast<hipStream_t>(stream)),
      "mean backward kernel");
}

nt_status nt_pair_broadcast_backward(const nt_partition* p, const float* g_z, float* g_a,
                                     float* g_b, int32_t c_z, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  const uint64_t zb = (uint64_t)p->cells * c_z * 4;
  const uint64_t ab = (uint64_t)p->T * c_z * 4, bb = (uint64_t)p->T_cols * c_z * 4;
  NT_TRY(check_array("g_z", g_z, zb));
  NT_TRY(check_array("g_a", g_a, ab));
  NT_TRY(check_array("g_b", g_b, bb));
  const Arr arrs[] = {{"g_z", g_z, zb, false}, {"g_a", g_a, ab, true}, {"g_b", g_b, bb, true}};
  NT_TRY(check_disjoint(arrs, 3));
  hipStream_t s = static_cast<hipStream_t>(stream);
  NT_TRY(hip_status(nt::launch_reduce(*p, g_z, g_a, c_z, NT_F32, s, false), "row sums"));
  return hip_status(nt::launch_col_sums(*p, g_z, g_b, c_z, s), "column sums");
}

nt_status nt_transition_backward_workspace_bytes(const nt_partition* p, int32_t c_z,
                                                 int32_t hidden, nt_dtype dtype, size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = transition_backward_ws(p->cells, c_z, hidden, dtype).total;
  return ok();
}

nt_status nt_pair_transition_backward(const nt_partition* p, const void* z, const float* G,
                                      const void* W1, const void* W2, float* g_z, float* dW1,
                                      float* dW2, int32_t c_z, int32_t hidden, nt_dtype dtype,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  const uint64_t es = esize(dtype);
  const uint64_t zb = (uint64_t)p->cells * c_z * es, fb = (uint64_t)p->cells * c_z * 4;
  const uint64_t wb = (uint64_t)hidden * c_z * es, db = (uint64_t)hidden * c_z * 4;
  const uint64_t need = transition_backward_ws(p->cells, c_z, hidden, dtype).total;
  NT_TRY(check_array("z", z, zb));
  NT_TRY(check_array("G", G, fb));
  NT_TRY(check_array("W1", W1, wb));
  NT_TRY(check_array("W2", W2, wb));
  NT_TRY(check_array("g_z", g_z, fb));
  NT_TRY(check_array("dW1", dW1, db));
  NT_TRY(check_array("dW2", dW2, db));
  NT_TRY(check_workspace(workspace, workspace_bytes, need));
  const Arr arrs[] = {{"z", z, zb, false},     {"G", G, fb, false},
                      {"W1", W1, wb, false},   {"W2", W2, wb, false},
                      {"g_z", g_z, fb, true},  {"dW1", dW1, db, true},
                      {"dW2", dW2, db, true},  {"workspace", workspace, need, true}};
  const int same[][2] = {{1, 4}};
  NT_TRY(check_disjoint(arrs, 8, same, 1));
  return transition_backward(p, z, G, W1, W2, g_z, dW1, dW2, c_z, hidden, dtype,
                             static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

nt_status nt_block_backward_workspace_bytes(const nt_partition* p, int32_t c_s, int32_t c_z,
                                            int32_t hidden, nt_dtype dtype, size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_widths(c_s, c_z, hidden));
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = block_backward_ws(p, c_s, c_z, hidden, dtype).total;
  return ok();
}

// The block backward; S > 1 is the non-leading layout (rows of S slices).
// The ReLU-MLP gradients of nt_block_grads as block parameter gradients.
static nt_block_param_grads relu_grads(const nt_block_grads& g) {
  nt_block_param_grads q;
  std::memset(&q, 0, sizeof(q));
  q.Wa = g.Wa;
  q.Wb = g.Wb;
  q.Wo = g.Wo;
  q.W1 = g.W1;
  q.W2 = g.W2;
  return q;
}

static nt_status block_backward_s(const nt_partition* p, const void* s_in, const void* z_out,
                                  const nt_block_params* w, const float* g_s_out,
                                  const float* g_z_out, float* g_s_in,
                                  const nt_block_param_grads* grads, int32_t c_s, int32_t c_z,
                                  int32_t hidden, nt_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream, int32_t S) {
  NT_TRY(check_partition(p));
  if (p->col_offsets != p->single_offsets)
    return fail(NT_ERR_INVALID, "the block backward takes square partitions");
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_widths(c_s, c_z, hidden));
  NT_TRY(check_static_axis(S, c_z));
  ParamArrays pa;
  NT_TRY(check_params(w, c_s, c_z, hidden, dtype, &pa));
  const bool swiglu = w->kind == NT_TRANSITION_LN_SWIGLU;
  if (swiglu && S != 1)
    return fail(NT_ERR_INVALID, "the SwiGLU block gradient takes the leading layout (S = 1)");
  if (!grads) return fail(NT_ERR_NULL, "grads is NULL");
  const uint64_t es = esize(dtype);
  const uint64_t TS = (uint64_t)p->T * S, CS = (uint64_t)p->cells * S;
  const uint64_t sb = TS * c_s * es, zb = CS * c_z * es;
  const uint64_t gsb = TS * c_s * 4, gzb = CS * c_z * 4;
  const uint64_t dproj = (uint64_t)c_z * c_s * 4, dmlp = (uint64_t)c_z * hidden * 4;
  const uint64_t dln = (uint64_t)c_z * 4;
  const BlockBwdWs L = block_backward_ws(p, c_s, c_z, hidden, dtype, S, w->kind);
  NT_TRY(check_array("s_in", s_in, sb));
  NT_TRY(check_array("z_out", z_out, zb));
  NT_TRY(check_array("g_s_out", g_s_out, gsb));
  if (g_z_out) NT_TRY(check_array("g_z_out", g_z_out, gzb));
  NT_TRY(check_array("g_s_in", g_s_in, gsb));
  Arr arrs[24];
  int n = 0;
  arrs[n++] = {"s_in", s_in, sb, false};
  arrs[n++] = {"z_out", z_out, zb, false};
  arrs[n++] = {"g_s_out", g_s_out, gsb, false};
  arrs[n++] = {"g_z_out", g_z_out, g_z_out ? gzb : 0, false};
  arrs[n++] = {"g_s_in", g_s_in, gsb, true};
  arrs[n++] = {"workspace", workspace, L.total, true};
  for (int k = 0; k < pa.n; ++k) arrs[n++] = {pa.name[k], pa.ptr[k], pa.bytes[k], false};
  struct { const char* name; float* ptr; uint64_t bytes; } outs[] = {
      {"dWa", grads->Wa, dproj}, {"dWb", grads->Wb, dproj}, {"dWo", grads->Wo, dproj},
      {"dW1", grads->W1, dmlp}, {"dW2", grads->W2, dmlp}, {"dln_gamma", grads->ln_gamma, dln},
      {"dln_beta", grads->ln_beta, dln}, {"dW_gate", grads->W_gate, dmlp},
      {"dW_up", grads->W_up, dmlp}, {"dW_down", grads->W_down, dmlp}};
  const int first = swiglu ? 5 : 3, count = swiglu ? 5 : 2;
  for (int k = 0; k < 3; ++k) {
    NT_TRY(check_array(outs[k].name, outs[k].ptr, outs[k].bytes));
    arrs[n++] = {outs[k].name, outs[k].ptr, outs[k].bytes, true};
  }
  for (int k = first; k < first + count; ++k) {
    NT_TRY(check_array(outs[k].name, outs[k].ptr, outs[k].bytes));
    arrs[n++] = {outs[k].name, outs[k].ptr, outs[k].bytes, true};
  }
  NT_TRY(check_workspace(workspace, workspace_bytes, L.total));
  const int same[][2] = {{2, 4}};
  NT_TRY(check_disjoint(arrs, n, same, 1));

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  float* a = reinterpret_cast<float*>(base + L.a);
  float* b = reinterpret_cast<float*>(base + L.b);
  void* z = base + L.z;
  float* m = reinterpret_cast<float*>(base + L.m);
  float* g_m = reinterpret_cast<float*>(base + L.g_m);
  float* G = reinterpret_cast<float*>(base + L.G);
  float* g_a = reinterpret_cast<float*>(base + L.g_a);
  float* g_b = reinterpret_cast<float*>(base + L.g_b);
  void* WoT = base + L.WoT;
  void* WaT = base + L.WaT;
  void* WbT = base + L.WbT;
  float* ppart = reinterpret_cast<float*>(base + L.ppart);
  const int64_t T = p->T * S;  // single rows of c_s values
  const int W = S * c_z;       // pair and single row width of the pair-side arrays

  // recompute the forward's a, b, z and m
  NT_TRY(hip_status(nt::launch_linear2(s_in, dtype, w->Wa, w->Wb, a, b, T, c_z, c_s, s),
                    "projections a, b"));
  const bool swiglu_fused = swiglu && nt::swiglu_bwd32_supported(c_z, hidden, dtype);
  if (!swiglu_fused)
    NT_TRY(hip_status(nt::launch_broadcast(*p, a, b, z, W, swiglu ? NT_F32 : dtype, s, true),
                      "broadcast"));
  NT_TRY(hip_status(nt::launch_reduce(*p, z_out, m, W, dtype, s), "column mean"));
  NT_TRY(hip_status(nt::launch_transpose(w->Wo, WoT, c_s, c_z, dtype, s), "transpose Wo"));
  NT_TRY(hip_status(nt::launch_transpose(w->Wa, WaT, c_z, c_s, dtype, s), "transpose Wa"));
  NT_TRY(hip_status(nt::launch_transpose(w->Wb, WbT, c_z, c_s, dtype, s), "transpose Wb"));
  // s~ = s + m Wo^T
  NT_TRY(hip_status(nt::launch_linear(g_s_out, NT_F32, WoT, dtype, nullptr, g_m, NT_F32, T, c_z,
                                      c_s, s),
                    "g_m = g_s Wo"));
  NT_TRY(hip_status(nt::launch_gemm_tn(g_s_out, NT_F32, m, NT_F32, grads->Wo, ppart, T, c_s, c_z,
                                       L.psplits, s),
                    "dWo"));
  // mean (formed inside the transition's gradient), transition, broadcast
  if (swiglu) {
    NT_TRY(hip_status(nt::launch_mean_backward(*p, g_m, g_z_out, G, W, s), "mean backward"));
    if (swiglu_fused)
      NT_TRY(swiglu_transition_backward32(p, a, b, G, *w, *grads, c_z, hidden, base + L.trans,
                                          s));
    else
      NT_TRY(swiglu_transition_backward(p->cells, static_cast<const float*>(z), G, *w, *grads,
                                        c_z, hidden, base + L.trans, s));
  } else if (S == 1) {
    NT_TRY(transition_backward(p, z, nullptr, w->W1, w->W2, G, grads->W1, grads->W2, c_z, hidden,
                               dtype, base + L.trans, s, g_m, g_z_out));
  } else {
    // the mean's adjoint over rows of S slices, then the cell-local gradient
    // over cells * S rows of c_z
    NT_TRY(hip_status(nt::launch_mean_backward(*p, g_m, g_z_out, G, W, s), "mean backward"));
    const nt_partition v = rows_view(*p, S);
    NT_TRY(transition_backward(&v, z, G, w->W1, w->W2, G, grads->W1, grads->W2, c_z, hidden,
                               dtype, base + L.trans, s));
  }
  NT_TRY(hip_status(nt::launch_bcast_adj(*p, G, g_a, g_b, W,
                                         reinterpret_cast<float*>(base + L.adj), s),
                    "row and column sums"));
  // a = s Wa^T, b = s Wb^T
  NT_TRY(hip_status(nt::launch_linear(g_a, NT_F32, WaT, dtype, g_s_out, g_s_in, NT_F32, T, c_s,
                                      c_z, s),
                    "g_s += g_a Wa"));
  NT_TRY(hip_status(nt::launch_linear(g_b, NT_F32, WbT, dtype, g_s_in, g_s_in, NT_F32, T, c_s,
                                      c_z, s),
                    "g_s += g_b Wb"));
  NT_TRY(hip_status(nt::launch_gemm_tn(g_a, NT_F32, s_in, dtype, grads->Wa, ppart, T, c_z, c_s,
                                       L.psplits, s),
                    "dWa"));
  return hip_status(nt::launch_gemm_tn(g_b, NT_F32, s_in, dtype, grads->Wb, ppart, T, c_z, c_s,
                                       L.psplits, s),
                    "dWb");
}

nt_status nt_pair_block_backward(const nt_partition* p, const void* s_in, const void* z_out,
                                 const nt_block_weights* w, const float* g_s_out,
                                 const float* g_z_out, float* g_s_in, const nt_block_grads* grads,
                                 int32_t c_s, int32_t c_z, int32_t hidden, nt_dtype dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  if (!grads) return fail(NT_ERR_NULL, "grads is NULL");
  const nt_block_params q = relu_params(*w);
  const nt_block_param_grads g = relu_grads(*grads);
  return block_backward_s(p, s_in, z_out, &q, g_s_out, g_z_out, g_s_in, &g, c_s, c_z, hidden,
                          dtype, workspace, workspace_bytes, stream, 1);
}

nt_status nt_block_backward_ex_workspace_bytes(const nt_partition* p, int32_t kind, int32_t c_s,
                                               int32_t c_z, int32_t hidden, nt_dtype dtype,
                                               size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_widths(c_s, c_z, hidden));
  if (kind != NT_TRANSITION_RELU_MLP && kind != NT_TRANSITION_LN_SWIGLU)
    return fail(NT_ERR_INVALID, "unknown transition kind %d", (int)kind);
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = block_backward_ws(p, c_s, c_z, hidden, dtype, 1, kind).total;
  return ok();
}

nt_status nt_pair_block_backward_ex(const nt_partition* p, const void* s_in, const void* z_out,
                                    const nt_block_params* w, const float* g_s_out,
                                    const float* g_z_out, float* g_s_in,
                                    const nt_block_param_grads* grads, int32_t c_s, int32_t c_z,
                                    int32_t hidden, nt_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return block_backward_s(p, s_in, z_out, w, g_s_out, g_z_out, g_s_in, grads, c_s, c_z, hidden,
                          dtype, workspace, workspace_bytes, stream, 1);
}

nt_status nt_block_nl_workspace_bytes(const nt_partition* p, int32_t S, int32_t c_s, int32_t c_z,
                                      int32_t hidden, nt_dtype dtype, size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_widths(c_s, c_z, hidden));
  NT_TRY(check_static_axis(S, c_z));
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = block_workspace(p->T, p->T_cols, c_z, dtype, S).total;
  return ok();
}

nt_status nt_pair_block_nl(const nt_partition* p, const void* s_in, void* s_out, void* z_out,
                           const nt_block_weights* w, int32_t S, int32_t c_s, int32_t c_z,
                           int32_t hidden, nt_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  NT_TRY(check_partition(p));
  if (p->col_offsets != p->single_offsets)
    return fail(NT_ERR_INVALID, "the non-leading block takes square partitions");
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  const nt_block_params q = relu_params(*w);
  return pair_block(p, s_in, s_in, s_out, z_out, &q, c_s, c_z, hidden, dtype, workspace,
                    workspace_bytes, stream, S);
}

nt_status nt_block_backward_nl_workspace_bytes(const nt_partition* p, int32_t S, int32_t c_s,
                                               int32_t c_z, int32_t hidden, nt_dtype dtype,
                                               size_t* bytes) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_widths(c_s, c_z, hidden));
  NT_TRY(check_static_axis(S, c_z));
  if (!bytes) return fail(NT_ERR_NULL, "bytes is NULL");
  *bytes = block_backward_ws(p, c_s, c_z, hidden, dtype, S).total;
  return ok();
}

nt_status nt_pair_block_backward_nl(const nt_partition* p, const void* s_in, const void* z_out,
                                    const nt_block_weights* w, const float* g_s_out,
                                    const float* g_z_out, float* g_s_in,
                                    const nt_block_grads* grads, int32_t S, int32_t c_s,
                                    int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  if (!grads) return fail(NT_ERR_NULL, "grads is NULL");
  const nt_block_params q = relu_params(*w);
  const nt_block_param_grads g = relu_grads(*grads);
  return block_backward_s(p, s_in, z_out, &q, g_s_out, g_z_out, g_s_in, &g, c_s, c_z, hidden,
                          dtype, workspace, workspace_bytes, stream, S);
}

}  // extern "C"
