// C-ABI entry points: host-side validation, partition sizing, launch order.
// Every check runs before anything is enqueued, so a non-OK status leaves
// the stream and all outputs untouched.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

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
// b has one row per column single (T_cols, which is T for square pairs).
BlockWorkspace block_workspace(int64_t T, int64_t T_cols, int c_z, nt_dtype) {
  BlockWorkspace w;
  const uint64_t a = nt::align256((size_t)T * c_z * sizeof(float));
  const uint64_t b = nt::align256((size_t)T_cols * c_z * sizeof(float));
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

// One block; s_cols is s_rows for square partitions.
nt_status pair_block(const nt_partition* p, const void* s_rows, const void* s_cols, void* s_out,
                     void* z_out, const nt_block_weights* w, int32_t c_s, int32_t c_z,
                     int32_t hidden, nt_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  NT_TRY(check_partition(p));
  NT_TRY(check_dtype(dtype));
  NT_TRY(check_width("c_s", c_s, nt::kMaxCs));
  NT_TRY(check_width("c_z", c_z, nt::kMaxCz));
  NT_TRY(check_width("hidden", hidden, nt::kMaxHidden));
  if (!w) return fail(NT_ERR_NULL, "weights is NULL");
  const size_t es = esize(dtype);
  const uint64_t sbytes = (uint64_t)p->T * c_s * es;
  const uint64_t cbytes = (uint64_t)p->T_cols * c_s * es;
  const uint64_t pair = (uint64_t)p->cells * c_z * es;
  const uint64_t proj = (uint64_t)c_z * c_s * es;
  const uint64_t mlp = (uint64_t)c_z * hidden * es;
  NT_TRY(check_array("s_rows", s_rows, sbytes));
  NT_TRY(check_array("s_cols", s_cols, cbytes));
  NT_TRY(check_array("s_out", s_out, sbytes));
  NT_TRY(check_array("z_out", z_out, pair));
  NT_TRY(check_array("Wa", w->Wa, proj));
  NT_TRY(check_array("Wb", w->Wb, proj));
  NT_TRY(check_array("W1", w->W1, mlp));
  NT_TRY(check_array("W2", w->W2, mlp));
  NT_TRY(check_array("Wo", w->Wo, proj));
  const BlockWorkspace ws = block_workspace(p->T, p->T_cols, c_z, dtype);
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
  const void* ins[] = {s_rows, w->Wa, w->Wb, w->W1, w->W2, w->Wo, workspace, s_cols};
  const uint64_t insz[] = {sbytes, proj, proj, mlp, mlp, proj, ws.total, cbytes};
  for (int k = 0; k < 8; ++k) {
    if (overlaps(z_out, pair, ins[k], insz[k]) ||
        (k > 0 && k < 7 && overlaps(s_out, sbytes, ins[k], insz[k])))
      return fail(NT_ERR_INVALID, "an output overlaps an input or the workspace");
  }
  if (overlaps(z_out, pair, s_out, sbytes))
    return fail(NT_ERR_INVALID, "z_out overlaps s_out");
  if (p->T == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  void* a = base + ws.a;
  void* b = base + ws.b;
  float* m = reinterpret_cast<float*>(base + ws.m);
  if (s_cols == s_rows && p->T_cols == p->T) {
    NT_TRY(hip_status(nt::launch_linear2(s_rows, dtype, w->Wa, w->Wb, a, b, p->T, c_z, c_s, s),
                      "projections a, b"));
  } else {
    NT_TRY(hip_status(nt::launch_linear(s_rows, dtype, w->Wa, dtype, nullptr, a, NT_F32, p->T,
                                        c_z, c_s, s),
                      "projection a"));
    NT_TRY(hip_status(nt::launch_linear(s_cols, dtype, w->Wb, dtype, nullptr, b, NT_F32,
                                        p->T_cols, c_z, c_s, s),
                      "projection b"));
  }
  NT_TRY(hip_status(nt::launch_transition(*p, nullptr, a, b, z_out, w->W1, w->W2, c_z, hidden,
                                          dtype, s),
                    "fused broadcast + transition"));
  NT_TRY(hip_status(nt::launch_reduce(*p, z_out, m, c_z, dtype, s), "column mean"));
  return hip_status(nt::launch_linear(m, NT_F32, w->Wo, dtype, s_rows, s_out, dtype, p->T, c_s,
                                      c_z, s),
                    "output projection");
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
  return hip_status(nt::launch_transition_swiglu(*p, z_in, z_out, ln_gamma, ln_beta, W_gate, W_up,
                                                 W_down, c_z, hidden, ln_eps,
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
  return pair_block(p, s_in, s_in, s_out, z_out, w, c_s, c_z, hidden, dtype, workspace,
                    workspace_bytes, stream);
}

nt_status nt_pair_block_rect(const nt_partition* p, const void* s_rows, const void* s_cols,
                             void* s_out, void* z_out, const nt_block_weights* w, int32_t c_s,
                             int32_t c_z, int32_t hidden, nt_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return pair_block(p, s_rows, s_cols, s_out, z_out, w, c_s, c_z, hidden, dtype, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"
