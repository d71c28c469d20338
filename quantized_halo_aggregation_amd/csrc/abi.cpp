// C ABI of libqha: host-side argument checks, set-up helpers and kernel launches.
// Every check runs before anything is enqueued, so bad arguments never reach the GPU.
#include "../../include/qha.h"
#include "qha_internal.hpp"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace qha {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return QHA_OK;
}

}  // namespace qha

using qha::fail;
using qha::ok;

namespace {

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool width_supported(int32_t d) {
  return d == 16 || d == 32 || d == 64 || d == 128 || d == 256 || d == 512;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

constexpr int64_t kMaxIndex = 2147483647LL;

int check_rows(const char* name, const float* p, int64_t ld, int32_t d) {
  if (!p) return fail(QHA_ERR_INVALID_ARG, "%s is NULL", name);
  if (ld < d || (ld & 3) != 0) return fail(QHA_ERR_INVALID_ARG, "%s: leading dimension %lld must be >= d=%d and a multiple of 4", name, (long long)ld, d);
  if (!aligned16(p)) return fail(QHA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return QHA_OK;
}

// ws_given: the caller passes the workspace (checked here); otherwise the library's scratch is used.
int check_plan(const qha_agg_plan* plan, int64_t n_rows, int32_t beta, int32_t d, const void* ws, size_t ws_bytes,
               bool ws_given = true) {
  if (!plan) return QHA_OK;
  if (plan->n_rows != n_rows) return fail(QHA_ERR_INVALID_ARG, "plan was built for %lld rows, call has %lld", (long long)plan->n_rows, (long long)n_rows);
  if (plan->chunk <= 0 || plan->group_edges <= 0) return fail(QHA_ERR_INVALID_ARG, "plan budgets must be positive");
  if (plan->n_items < 0 || plan->n_split_items < 0 || plan->n_split_rows < 0 || plan->n_split_items > plan->n_items)
    return fail(QHA_ERR_INVALID_ARG, "plan counts are inconsistent");
  if (plan->n_items > 0 && !plan->items) return fail(QHA_ERR_INVALID_ARG, "plan items is NULL");
  if (plan->n_split_rows > 0 && (!plan->split_row || !plan->split_ptr))
    return fail(QHA_ERR_INVALID_ARG, "plan split arrays are NULL");
  if (plan->skip_empty && beta != 1) return fail(QHA_ERR_INVALID_ARG, "a plan that skips empty rows needs beta = 1");
  const size_t need = qha_agg_workspace_bytes(plan, d);
  if (!ws_given) {
    if (need > QHA_NOALLOC_SCRATCH_BYTES)
      return fail(QHA_ERR_WORKSPACE, "the plan's split-row partials need %zu bytes, the static scratch holds %zu", need, (size_t)QHA_NOALLOC_SCRATCH_BYTES);
  } else if (need > 0) {
    if (!ws || ws_bytes < need) return fail(QHA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(QHA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  }
  return QHA_OK;
}

void fill_plan_args(qha::GatherArgs& g, const qha_agg_plan* plan, int64_t n_rows, void* ws) {
  if (plan) {
    g.n_items = plan->n_items;
    g.n_split_items = plan->n_split_items;
    g.items = plan->items;
    g.n_split_rows = plan->n_split_rows;
    g.split_row = plan->split_row;
    g.split_ptr = plan->split_ptr;
  } else {
    g.n_items = n_rows;
    g.n_split_items = 0;
    g.items = nullptr;
    g.n_split_rows = 0;
    g.split_row = nullptr;
    g.split_ptr = nullptr;
  }
  g.partial = static_cast<double*>(ws);
}

uint64_t row_words(int32_t d, uint32_t b) { return b == 32 ? static_cast<uint64_t>(d) : (static_cast<uint64_t>(d) * b + 31) / 32; }

// Checks a host class table against the row count and copies it into kernel arguments.
int take_classes(const qha_width_classes* cls, int64_t n_rows, int32_t d, qha::Classes* out) {
  std::memset(out, 0, sizeof(*out));
  if (!cls) return QHA_OK;
  if (cls->n < 1 || cls->n > QHA_MAX_CLASSES) return fail(QHA_ERR_INVALID_ARG, "classes: n = %d out of range", cls->n);
  if (cls->start[0] != 0 || cls->start[cls->n] != n_rows)
    return fail(QHA_ERR_INVALID_ARG, "classes must cover rows 0 .. %lld exactly", (long long)n_rows);
  uint64_t expect = cls->base[0];
  for (int i = 0; i < cls->n; ++i) {
    const int32_t b = cls->bits[i];
    if (!(b == 1 || b == 2 || b == 4 || b == 8 || b == 32)) return fail(QHA_ERR_INVALID_ARG, "classes: width %d", b);
    if (cls->start[i + 1] < cls->start[i]) return fail(QHA_ERR_INVALID_ARG, "classes: starts decrease");
    if (cls->base[i] != expect) return fail(QHA_ERR_INVALID_ARG, "classes: class %d does not follow the previous one", i);
    expect += static_cast<uint64_t>(cls->start[i + 1] - cls->start[i]) * row_words(d, static_cast<uint32_t>(b));
    if (expect > 0xFFFFFFFFull) return fail(QHA_ERR_INVALID_ARG, "classes: buffer exceeds 2^32-1 words");
  }
  out->n = cls->n;
  for (int i = 0; i < cls->n; ++i) {
    out->bits[i] = cls->bits[i];
    out->start[i] = cls->start[i];
    out->base[i] = cls->base[i];
  }
  out->start[cls->n] = cls->start[cls->n];
  return QHA_OK;
}

// Walks the rows once and either counts (cap == nullptr) or writes the plan's arrays, which hold
// cap->items items and cap->split_rows split rows: a walk that would write more (a rowptr other than
// the one the plan was sized for) stops writing and fails.
struct PlanWalk {
  int64_t items = 0, split_items = 0, split_rows = 0;
};

int walk_plan(const int32_t* rowptr, int64_t n_rows, int32_t chunk, int32_t group_edges, int32_t skip_empty,
              PlanWalk* cnt, const PlanWalk* cap, int32_t* items, int32_t* split_row, int32_t* split_ptr) {
  PlanWalk w;
  bool over = false;
  auto emit = [&](int64_t r0, int64_t nr, int64_t e0, int64_t e1) {
    if (cap && w.items >= cap->items) over = true;
    if (items && !over) {
      int32_t* it = items + 4 * w.items;
      it[0] = static_cast<int32_t>(r0);
      it[1] = static_cast<int32_t>(nr);
      it[2] = static_cast<int32_t>(e0);
      it[3] = static_cast<int32_t>(e1);
    }
    ++w.items;
  };
  // chunks of split rows first: their items carry the longest work
  if (split_ptr) split_ptr[0] = 0;
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t b = rowptr[r], e = rowptr[r + 1];
    if (e < b) return fail(QHA_ERR_INVALID_ARG, "rowptr decreases at row %lld", (long long)r);
    if (e - b > chunk) {
      for (int64_t c = b; c < e; c += chunk) emit(r, 1, c, c + chunk < e ? c + chunk : e);
      if (cap && w.split_rows >= cap->split_rows) over = true;
      if (split_row && !over) split_row[w.split_rows] = static_cast<int32_t>(r);
      ++w.split_rows;
      if (split_ptr && !over) split_ptr[w.split_rows] = static_cast<int32_t>(w.items);
    }
    if (over) return fail(QHA_ERR_INVALID_ARG, "plan does not match rowptr (more split rows or items)");
  }
  w.split_items = w.items;
  // groups of consecutive rows
  int64_t g0 = -1, gn = 0, ge = 0;
  auto close = [&]() {
    if (gn > 0) emit(g0, gn, rowptr[g0], rowptr[g0 + gn]);
    g0 = -1;
    gn = 0;
    ge = 0;
  };
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t len = static_cast<int64_t>(rowptr[r + 1]) - rowptr[r];
    if (len > chunk) {
      close();
      continue;
    }
    if (len == 0) {            // never inside a group: each edge then closes at most one row
      close();
      if (!skip_empty) emit(r, 1, rowptr[r], rowptr[r]);
      continue;
    }
    if (gn > 0 && (gn >= QHA_GROUP_ROWS || ge + len > group_edges)) close();
    if (gn == 0) g0 = r;
    ++gn;
    ge += len;
  }
  close();
  if (over) return fail(QHA_ERR_INVALID_ARG, "plan does not match rowptr (more work items)");
  if (w.items > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "too many work items");
  *cnt = w;
  return QHA_OK;
}

}  // namespace

extern "C" {

int qha_abi_version(void) { return QHA_ABI_VERSION; }

const char* qha_status_string(int status) {
  switch (status) {
    case QHA_OK: return "ok";
    case QHA_ERR_INVALID_ARG: return "invalid argument";
    case QHA_ERR_UNSUPPORTED: return "unsupported";
    case QHA_ERR_HIP: return "HIP runtime error";
    case QHA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* qha_last_error(void) { return g_err; }

int qha_pack_layout(const uint8_t* bits, int64_t n_rows, int32_t d, uint32_t* word_offset, uint64_t* total_words) {
  if (n_rows < 0) return fail(QHA_ERR_INVALID_ARG, "n_rows < 0");
  if (!word_offset || !total_words || (n_rows > 0 && !bits)) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  if (!width_supported(d)) return fail(QHA_ERR_UNSUPPORTED, "d=%d not supported", d);
  uint64_t acc = 0;
  word_offset[0] = 0;
  for (int64_t r = 0; r < n_rows; ++r) {
    const uint32_t b = bits[r];
    uint64_t w;
    if (b == 32) w = static_cast<uint64_t>(d);
    else if (b == 1 || b == 2 || b == 4 || b == 8) w = (static_cast<uint64_t>(d) * b + 31) / 32;
    else return fail(QHA_ERR_INVALID_ARG, "bits[%lld] = %u is not in {1,2,4,8,32}", (long long)r, b);
    acc += w;
    if (acc > 0xFFFFFFFFull) return fail(QHA_ERR_INVALID_ARG, "packed buffer exceeds 2^32-1 words");
    word_offset[r + 1] = static_cast<uint32_t>(acc);
  }
  *total_words = acc;
  return ok();
}

int qha_pack_classes(const uint8_t* bits, int64_t n_rows, int32_t d, qha_width_classes* classes) {
  if (n_rows < 0 || n_rows > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad n_rows");
  if (!classes || (n_rows > 0 && !bits)) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  if (!width_supported(d)) return fail(QHA_ERR_UNSUPPORTED, "d=%d not supported", d);
  std::memset(classes, 0, sizeof(*classes));
  uint64_t words = 0;
  int n = 0;
  for (int64_t r = 0; r < n_rows; ++r) {
    const uint32_t b = bits[r];
    if (!(b == 1 || b == 2 || b == 4 || b == 8 || b == 32))
      return fail(QHA_ERR_INVALID_ARG, "bits[%lld] = %u is not in {1,2,4,8,32}", (long long)r, b);
    if (n == 0 || static_cast<uint32_t>(classes->bits[n - 1]) != b) {
      if (n == QHA_MAX_CLASSES) return fail(QHA_ERR_UNSUPPORTED, "rows form more than %d runs of equal width", QHA_MAX_CLASSES);
      classes->bits[n] = static_cast<int32_t>(b);
      classes->start[n] = static_cast<int32_t>(r);
      classes->base[n] = static_cast<uint32_t>(words);
      ++n;
    }
    words += row_words(d, b);
    if (words > 0xFFFFFFFFull) return fail(QHA_ERR_INVALID_ARG, "packed buffer exceeds 2^32-1 words");
  }
  if (n == 0) {                       // no rows: one empty class keeps the table well formed
    classes->bits[0] = 32;
    n = 1;
  }
  classes->n = n;
  classes->start[n] = static_cast<int32_t>(n_rows);
  return ok();
}

int qha_validate_csr(int64_t n_rows, int64_t n_cols, const int32_t* rowptr, const int32_t* colidx, int32_t require_sorted) {
  if (n_rows < 0 || n_cols < 0 || n_rows > kMaxIndex || n_cols > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if (!rowptr) return fail(QHA_ERR_INVALID_ARG, "rowptr is NULL");
  if (rowptr[0] != 0) return fail(QHA_ERR_INVALID_ARG, "rowptr[0] != 0");
  for (int64_t r = 0; r < n_rows; ++r) {
    const int32_t b = rowptr[r], e = rowptr[r + 1];
    if (e < b) return fail(QHA_ERR_INVALID_ARG, "rowptr decreases at row %lld", (long long)r);
    if (e > b && !colidx) return fail(QHA_ERR_INVALID_ARG, "colidx is NULL");
    for (int32_t i = b; i < e; ++i) {
      if (colidx[i] < 0 || colidx[i] >= n_cols) return fail(QHA_ERR_INVALID_ARG, "row %lld has column %d outside [0, %lld)", (long long)r, colidx[i], (long long)n_cols);
      if (require_sorted && i > b && colidx[i] <= colidx[i - 1]) return fail(QHA_ERR_INVALID_ARG, "row %lld is not strictly ascending", (long long)r);
    }
  }
  return ok();
}

int qha_csr_transpose(int64_t n_rows, int64_t n_cols, const int32_t* rowptr, const int32_t* colidx, int32_t* colptr, int32_t* rowidx) {
  if (n_rows < 0 || n_cols < 0 || n_rows > kMaxIndex || n_cols > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if (!rowptr || !colptr) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  const int64_t nnz = rowptr[n_rows];
  if (nnz > 0 && (!colidx || !rowidx)) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  std::vector<int64_t> cnt(static_cast<size_t>(n_cols) + 1, 0);
  for (int64_t e = 0; e < nnz; ++e) {
    const int32_t c = colidx[e];
    if (c < 0 || c >= n_cols) return fail(QHA_ERR_INVALID_ARG, "column %d outside [0, %lld)", c, (long long)n_cols);
    ++cnt[static_cast<size_t>(c) + 1];
  }
  for (int64_t c = 0; c < n_cols; ++c) cnt[c + 1] += cnt[c];
  for (int64_t c = 0; c <= n_cols; ++c) colptr[c] = static_cast<int32_t>(cnt[c]);
  for (int64_t r = 0; r < n_rows; ++r)
    for (int32_t e = rowptr[r]; e < rowptr[r + 1]; ++e) rowidx[cnt[colidx[e]]++] = static_cast<int32_t>(r);
  return ok();
}

int qha_agg_plan_size(int64_t n_rows, const int32_t* rowptr, int32_t chunk, int32_t group_edges, int32_t skip_empty,
                      qha_agg_plan* plan) {
  if (n_rows < 0 || n_rows > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad n_rows");
  if (!rowptr || !plan) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  if (chunk <= 0 || group_edges <= 0) return fail(QHA_ERR_INVALID_ARG, "chunk and group_edges must be positive");
  PlanWalk w;
  int st = walk_plan(rowptr, n_rows, chunk, group_edges, skip_empty, &w, nullptr, nullptr, nullptr, nullptr);
  if (st) return st;
  std::memset(plan, 0, sizeof(*plan));
  plan->n_rows = n_rows;
  plan->chunk = chunk;
  plan->group_edges = group_edges;
  plan->skip_empty = skip_empty ? 1 : 0;
  plan->n_items = w.items;
  plan->n_split_items = w.split_items;
  plan->n_split_rows = w.split_rows;
  return ok();
}

int qha_agg_plan_fill(const int32_t* rowptr, const qha_agg_plan* plan, int32_t* items, int32_t* split_row,
                      int32_t* split_ptr) {
  if (!rowptr || !plan) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  if ((plan->n_items > 0 && !items) || !split_ptr || (plan->n_split_rows > 0 && !split_row))
    return fail(QHA_ERR_INVALID_ARG, "NULL output array");
  if (plan->n_rows < 0 || plan->n_rows > kMaxIndex || plan->chunk <= 0 || plan->group_edges <= 0 ||
      plan->n_items < 0 || plan->n_split_rows < 0)
    return fail(QHA_ERR_INVALID_ARG, "malformed plan");
  PlanWalk w, cap;
  cap.items = plan->n_items;
  cap.split_rows = plan->n_split_rows;
  int st = walk_plan(rowptr, plan->n_rows, plan->chunk, plan->group_edges, plan->skip_empty, &w, &cap, items,
                     split_row, split_ptr);
  if (st) return st;
  if (w.items != plan->n_items || w.split_items != plan->n_split_items || w.split_rows != plan->n_split_rows)
    return fail(QHA_ERR_INVALID_ARG, "plan does not match rowptr");
  return ok();
}

size_t qha_agg_workspace_bytes(const qha_agg_plan* plan, int32_t d) {
  if (!plan || d <= 0) return 0;
  return static_cast<size_t>(plan->n_split_items) * static_cast<size_t>(d) * sizeof(double);
}

int qha_degree_norm(const int32_t* deg, int64_t n, int32_t kind, float* out, void* stream) {
  if (n < 0) return fail(QHA_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (!deg || !out)) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  if (kind != QHA_NORM_GCN && kind != QHA_NORM_MEAN) return fail(QHA_ERR_INVALID_ARG, "unknown normalisation %d", kind);
  return hip_status(qha::launch_degree_norm(deg, n, kind, out, static_cast<hipStream_t>(stream)), "degree_norm");
}

int qha_edge_weights(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* r, const float* c,
                     float* w, void* stream) {
  if (n_rows < 0 || n_rows > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad n_rows");
  if (n_rows == 0) return ok();
  if (!rowptr || !colidx || !w) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  return hip_status(qha::launch_edge_weights(n_rows, rowptr, colidx, r, c, w, static_cast<hipStream_t>(stream)),
                    "edge_weights");
}

int qha_quantize_pack(const float* x, int64_t ldx, const int32_t* row_index, int64_t n_rows, int32_t d,
                      const uint8_t* bits, const uint32_t* word_offset, const qha_width_classes* classes,
                      uint64_t seed, uint32_t epoch, uint32_t stream_id, uint32_t node_base, uint32_t* codes,
                      float* meta, void* stream) {
  if (n_rows < 0 || n_rows > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad n_rows");
  if (!width_supported(d)) return fail(QHA_ERR_UNSUPPORTED, "d=%d not supported", d);
  if (n_rows == 0) return ok();
  int st = check_rows("x", x, ldx, d);
  if (st) return st;
  if (!codes || !meta || (!classes && (!bits || !word_offset))) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned4(codes) || !aligned8(meta) || (word_offset && !aligned4(word_offset)) || (row_index && !aligned4(row_index)))
    return fail(QHA_ERR_INVALID_ARG, "misaligned array");
  if (static_cast<uint64_t>(node_base) + static_cast<uint64_t>(n_rows) - 1 > 0xFFFFFFFFull)
    return fail(QHA_ERR_INVALID_ARG, "node ids node_base + r overflow 32 bits");
  qha::QuantArgs a;
  st = take_classes(classes, n_rows, d, &a.cls);
  if (st) return st;
  a.x = x;
  a.ldx = ldx;
  a.row_index = row_index;
  a.n_rows = n_rows;
  a.bits = bits;
  a.word_offset = word_offset;
  a.seed_lo = static_cast<uint32_t>(seed);
  a.seed_hi = static_cast<uint32_t>(seed >> 32);
  a.epoch = epoch;
  a.stream_id = stream_id;
  a.node_base = node_base;
  a.codes = codes;
  a.meta = meta;
  return hip_status(qha::launch_quantize(a, d, static_cast<hipStream_t>(stream)), "quantize_pack");
}

// qha_dequant_aggregate_fwd, with the caller's workspace (ws_given) or the library's scratch.
static int dequant_aggregate(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* w,
                             const int32_t* row_ids, const qha_agg_plan* plan, const float* x_inner, int64_t ldx,
                             int64_t n_inner, const uint32_t* codes, const uint32_t* word_offset,
                             const uint8_t* bits, const qha_width_classes* classes, const float* meta,
                             int64_t n_halo, int32_t d, int32_t beta, float* out, int64_t ldo, void* workspace,
                             size_t workspace_bytes, bool ws_given, void* stream) {
  if (n_rows < 0 || n_rows > kMaxIndex || n_inner < 0 || n_halo < 0 || n_inner + n_halo > kMaxIndex)
    return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if (!width_supported(d)) return fail(QHA_ERR_UNSUPPORTED, "d=%d not supported", d);
  if (beta != 0 && beta != 1) return fail(QHA_ERR_INVALID_ARG, "beta must be 0 or 1");
  if (n_rows == 0) return ok();
  if (!rowptr || !colidx) return fail(QHA_ERR_INVALID_ARG, "rowptr/colidx is NULL");
  int st = check_rows("out", out, ldo, d);
  if (st) return st;
  if (n_inner > 0) {
    st = check_rows("x_inner", x_inner, ldx, d);
    if (st) return st;
  }
  qha::GatherArgs g;
  std::memset(&g, 0, sizeof(g));
  if (n_halo > 0) {
    if (!codes || !meta || (!classes && (!word_offset || !bits)))
      return fail(QHA_ERR_INVALID_ARG, "halo message arrays are NULL");
    if (!aligned8(meta) || !aligned4(codes) || (word_offset && !aligned4(word_offset)))
      return fail(QHA_ERR_INVALID_ARG, "misaligned halo message arrays");
    st = take_classes(classes, n_halo, d, &g.cls);
    if (st) return st;
  }
  st = check_plan(plan, n_rows, beta, d, workspace, workspace_bytes, ws_given);
  if (st) return st;
  if (!ws_given) {
    hipError_t e = hipSuccess;
    workspace = qha::noalloc_scratch(&e);
    if (!workspace) return hip_status(e, "dequant_aggregate_fwd_noalloc: scratch address");
  }
  g.n_rows = n_rows;
  g.rowptr = rowptr;
  g.colidx = colidx;
  g.row_ids = row_ids;
  fill_plan_args(g, plan, n_rows, workspace);
  g.w = w;
  g.x = x_inner;
  g.ldx = ldx;
  g.n_inner = n_inner;
  g.codes = codes;
  g.word_offset = word_offset;
  g.bits = bits;
  g.meta = meta;
  g.n_halo = n_halo;
  g.beta = beta;
  g.out = out;
  g.ldo = ldo;
  return hip_status(qha::launch_gather(g, d, n_halo > 0, static_cast<hipStream_t>(stream)), "dequant_aggregate_fwd");
}

int qha_dequant_aggregate_fwd(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* w,
                              const int32_t* row_ids, const qha_agg_plan* plan, const float* x_inner, int64_t ldx,
                              int64_t n_inner, const uint32_t* codes, const uint32_t* word_offset,
                              const uint8_t* bits, const qha_width_classes* classes, const float* meta,
                              int64_t n_halo, int32_t d, int32_t beta, float* out, int64_t ldo, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return dequant_aggregate(n_rows, rowptr, colidx, w, row_ids, plan, x_inner, ldx, n_inner, codes, word_offset, bits,
                           classes, meta, n_halo, d, beta, out, ldo, workspace, workspace_bytes, true, stream);
}

int qha_dequant_aggregate_fwd_noalloc(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* w,
                                      const int32_t* row_ids, const qha_agg_plan* plan, const float* x_inner,
                                      int64_t ldx, int64_t n_inner, const uint32_t* codes,
                                      const uint32_t* word_offset, const uint8_t* bits,
                                      const qha_width_classes* classes, const float* meta, int64_t n_halo, int32_t d,
                                      int32_t beta, float* out, int64_t ldo, void* stream) {
  return dequant_aggregate(n_rows, rowptr, colidx, w, row_ids, plan, x_inner, ldx, n_inner, codes, word_offset, bits,
                           classes, meta, n_halo, d, beta, out, ldo, nullptr, 0, false, stream);
}

int qha_aggregate_bwd(int64_t n_rows, const int32_t* colptr, const int32_t* rowidx, const float* w,
                      const qha_agg_plan* plan, const float* grad_out, int64_t ldg, int64_t n_grad_rows, int32_t d,
                      int32_t beta, float* grad_in, int64_t ldi, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (n_rows < 0 || n_rows > kMaxIndex || n_grad_rows < 0 || n_grad_rows > kMaxIndex)
    return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if (!width_supported(d)) return fail(QHA_ERR_UNSUPPORTED, "d=%d not supported", d);
  if (beta != 0 && beta != 1) return fail(QHA_ERR_INVALID_ARG, "beta must be 0 or 1");
  if (n_rows == 0) return ok();
  if (!colptr || !rowidx) return fail(QHA_ERR_INVALID_ARG, "colptr/rowidx is NULL");
  int st = check_rows("grad_in", grad_in, ldi, d);
  if (st) return st;
  if (n_grad_rows > 0) {
    st = check_rows("grad_out", grad_out, ldg, d);
    if (st) return st;
  }
  st = check_plan(plan, n_rows, beta, d, workspace, workspace_bytes);
  if (st) return st;
  qha::GatherArgs g;
  std::memset(&g, 0, sizeof(g));
  g.n_rows = n_rows;
  g.rowptr = colptr;
  g.colidx = rowidx;
  fill_plan_args(g, plan, n_rows, workspace);
  g.w = w;
  g.x = grad_out;
  g.ldx = ldg;
  g.n_inner = n_grad_rows;
  g.beta = beta;
  g.out = grad_in;
  g.ldo = ldi;
  return hip_status(qha::launch_gather(g, d, false, static_cast<hipStream_t>(stream)), "aggregate_bwd");
}

int qha_aggregate_bwd_quantize(int64_t n_rows, const int32_t* colptr, const int32_t* rowidx, const float* w,
                               const qha_agg_plan* plan, const float* grad_out, int64_t ldg, int64_t n_grad_rows,
                               int32_t d, int64_t n_stored, int32_t beta, float* grad_in, int64_t ldi,
                               const uint8_t* bits, const uint32_t* word_offset, const qha_width_classes* classes,
                               uint64_t seed, uint32_t epoch, uint32_t stream_id, uint32_t node_base, uint32_t* codes,
                               float* meta, const qha_received* received, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (n_rows < 0 || n_rows > kMaxIndex || n_grad_rows < 0 || n_grad_rows > kMaxIndex || n_stored < 0 ||
      n_stored > n_rows)
    return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if (!width_supported(d)) return fail(QHA_ERR_UNSUPPORTED, "d=%d not supported", d);
  if (beta != 0 && beta != 1) return fail(QHA_ERR_INVALID_ARG, "beta must be 0 or 1");
  if (n_rows == 0) return ok();
  if (!colptr || !rowidx) return fail(QHA_ERR_INVALID_ARG, "colptr/rowidx is NULL");
  int st = 0;
  if (n_grad_rows > 0) {
    st = check_rows("grad_out", grad_out, ldg, d);
    if (st) return st;
  }
  if (n_stored > 0) {
    st = check_rows("grad_in", grad_in, ldi, d);
    if (st) return st;
  }
  const int64_t n_msg = n_rows - n_stored;
  if (n_msg > 0) {
    if (!codes || !meta || (!classes && (!bits || !word_offset))) return fail(QHA_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned4(codes) || !aligned8(meta) || (word_offset && !aligned4(word_offset)))
      return fail(QHA_ERR_INVALID_ARG, "misaligned array");
    if (static_cast<uint64_t>(node_base) + static_cast<uint64_t>(n_msg) - 1 > 0xFFFFFFFFull)
      return fail(QHA_ERR_INVALID_ARG, "node ids node_base + r overflow 32 bits");
  }
  const bool recv = received != nullptr && n_stored > 0;
  if (recv) {
    const qha_received& r = *received;
    if (r.n_rows < 0 || r.n_rows > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "received: bad row count");
    if (!r.copy_ptr || !r.copy_idx) return fail(QHA_ERR_INVALID_ARG, "received: copy_ptr/copy_idx is NULL");
    if (r.n_rows > 0) {
      if (!r.codes || !r.meta || (!r.classes && (!r.bits || !r.word_offset)))
        return fail(QHA_ERR_INVALID_ARG, "received: NULL pointer");
      if (!aligned4(r.codes) || !aligned8(r.meta) || (r.word_offset && !aligned4(r.word_offset)))
        return fail(QHA_ERR_INVALID_ARG, "received: misaligned array");
      if (n_msg > 0 && (r.codes == codes || r.meta == meta))
        return fail(QHA_ERR_INVALID_ARG, "received: the buffer is the one this call writes");
    }
  }
  st = check_plan(plan, n_rows, beta, d, workspace, workspace_bytes);
  if (st) return st;
  if (plan && plan->skip_empty) return fail(QHA_ERR_INVALID_ARG, "every row is written or coded: the plan may not skip empty rows");
  qha::GatherArgs g;
  std::memset(&g, 0, sizeof(g));
  if (n_msg > 0) {
    st = take_classes(classes, n_msg, d, &g.q.cls);
    if (st) return st;
  }
  if (recv) {
    const qha_received& r = *received;
    if (r.n_rows > 0) {
      st = take_classes(r.classes, r.n_rows, d, &g.r.cls);
      if (st) return st;
    }
    g.r.ptr = r.copy_ptr;
    g.r.idx = r.copy_idx;
    g.r.codes = r.codes;
    g.r.meta = r.meta;
    g.r.bits = r.bits;
    g.r.word_offset = r.word_offset;
  }
  g.n_rows = n_rows;
  g.rowptr = colptr;
  g.colidx = rowidx;
  fill_plan_args(g, plan, n_rows, workspace);
  g.w = w;
  g.x = grad_out;
  g.ldx = ldg;
  g.n_inner = n_grad_rows;
  g.beta = beta;
  g.out = grad_in;
  g.ldo = ldi;
  g.q.first = n_stored;
  g.q.codes = codes;
  g.q.meta = meta;
  g.q.bits = bits;
  g.q.word_offset = word_offset;
  g.q.seed_lo = static_cast<uint32_t>(seed);
  g.q.seed_hi = static_cast<uint32_t>(seed >> 32);
  g.q.epoch = epoch;
  g.q.stream_id = stream_id;
  g.q.node_base = node_base;
  return hip_status(qha::launch_gather(g, d, false, static_cast<hipStream_t>(stream), true),
                    "aggregate_bwd_quantize");
}

// Workspace a tiled product cannot run without: its split-k partials.
static size_t gemm_required_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  int32_t s;
  int64_t kps;
  qha::gemm_split_rule(m, n, k, &s, &kps);
  return s > 1 ? static_cast<size_t>(s) * static_cast<size_t>(m) * static_cast<size_t>(n) * sizeof(double) : 0;
}

size_t qha_dense_project_workspace(int32_t trans_a, int32_t trans_b, int64_t m, int64_t n, int64_t k) {
  (void)trans_b;
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  const size_t req = gemm_required_bytes(m, n, k), pre = qha::gemm_bsplit_bytes(trans_a, m, n, k);
  return req > pre ? req : pre;
}

int qha_dense_project(int32_t trans_a, int32_t trans_b, int64_t m, int64_t n, int64_t k, const float* a, int64_t lda,
                      const float* b, int64_t ldb, int32_t beta, float* c, int64_t ldc, int32_t prologue,
                      const float* aux, int64_t ld_aux, int32_t epilogue, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (m < 0 || n < 0 || k < 0 || m > kMaxIndex || n > kMaxIndex || k > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return fail(QHA_ERR_INVALID_ARG, "trans flags must be 0 or 1");
  if (beta != 0 && beta != 1) return fail(QHA_ERR_INVALID_ARG, "beta must be 0 or 1");
  if (prologue != QHA_PRO_NONE && prologue != QHA_PRO_RELU_MASK) return fail(QHA_ERR_INVALID_ARG, "unknown prologue");
  if (epilogue != QHA_EPI_NONE && epilogue != QHA_EPI_RELU) return fail(QHA_ERR_INVALID_ARG, "unknown epilogue");
  if (m == 0 || n == 0) return ok();
  // storage shapes: A is [m x k] or [k x m]; B is [k x n] or [n x k]; the contiguous extent of each
  // must be a multiple of 4 (16-byte loads)
  const int64_t a_cols = trans_a ? m : k, b_cols = trans_b ? k : n;
  if (k > 0) {
    if (!a || !b) return fail(QHA_ERR_INVALID_ARG, "A or B is NULL");
    if ((a_cols & 3) || (b_cols & 3)) return fail(QHA_ERR_INVALID_ARG, "the contiguous extent of A (%lld) and B (%lld) must be multiples of 4", (long long)a_cols, (long long)b_cols);
    if (lda < a_cols || (lda & 3) || !aligned16(a)) return fail(QHA_ERR_INVALID_ARG, "lda / A alignment out of contract");
    if (ldb < b_cols || (ldb & 3) || !aligned16(b)) return fail(QHA_ERR_INVALID_ARG, "ldb / B alignment out of contract");
    if (prologue == QHA_PRO_RELU_MASK && (!aux || ld_aux < a_cols || (ld_aux & 3) || !aligned16(aux)))
      return fail(QHA_ERR_INVALID_ARG, "aux out of contract");
  }
  if (!c || ldc < n || !aligned4(c)) return fail(QHA_ERR_INVALID_ARG, "C / ldc out of contract");
  qha::GemmArgs g;
  g.ta = trans_a;
  g.tb = trans_b;
  g.m = m;
  g.n = n;
  g.k = k;
  g.a = a;
  g.lda = lda;
  g.b = b;
  g.ldb = ldb;
  g.beta = beta;
  g.c = c;
  g.ldc = ldc;
  g.pro = prologue;
  g.aux = aux;
  g.ld_aux = ld_aux;
  g.epi = epilogue;
  if (!trans_a && trans_b && prologue == QHA_PRO_NONE && beta == 0 && m > 0 && qha::panel_fits(n, k)) {
    qha::PanelArgs p;
    std::memset(&p, 0, sizeof(p));
    p.m = m;
    p.a = a;
    p.lda = lda;
    p.w = b;
    p.ldw = ldb;
    p.out = c;
    p.ldo = ldc;
    p.relu = epilogue == QHA_EPI_RELU;
    return hip_status(qha::launch_panel_fwd(p, static_cast<hipStream_t>(stream)), "dense_project");
  }
  qha::gemm_split_rule(m, n, k, &g.splits, &g.k_per_split);
  g.ws = static_cast<double*>(workspace);
  if (g.splits > 1) {
    const size_t need = gemm_required_bytes(m, n, k);
    if (!workspace || workspace_bytes < need) return fail(QHA_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
    if (!aligned16(workspace)) return fail(QHA_ERR_INVALID_ARG, "workspace misaligned");
  }
  // B split once per call when the workspace has room for its parts (the same bits either way)
  const size_t pre = qha::gemm_bsplit_bytes(trans_a, m, n, k);
  g.bsplit = (pre > 0 && workspace && aligned16(workspace) && workspace_bytes >= pre) ? static_cast<uint32_t*>(workspace)
                                                                                       : nullptr;
  return hip_status(qha::launch_gemm(g, static_cast<hipStream_t>(stream)), "dense_project");
}

// Workspace the backward cannot run without: the panel path's dW partials, or the split-k
// partials of dW = dZ^T A.
static size_t dense_bwd_required_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  if (qha::panel_fits(n, k)) return qha::panel_bwd_workspace(m);
  if (qha::dw_panel_fits(m, n, k)) return qha::dw_panel_workspace(m, n, k);
  return gemm_required_bytes(n, k, m);
}

size_t qha_dense_backward_workspace(int64_t m, int64_t n, int64_t k) {
  const size_t req = dense_bwd_required_bytes(m, n, k);
  if (m <= 0 || n <= 0 || k <= 0 || qha::panel_fits(n, k)) return req;
  // dA = dZ W may split W once into the same workspace (dW's partials are written after dA has
  // read W's parts, on the same stream)
  const size_t pre = qha::gemm_bsplit_bytes(0, m, k, n);
  return req > pre ? req : pre;
}

int qha_dense_backward(int64_t m, int64_t n, int64_t k, const float* dh, int64_t ldg, const float* h, int64_t ldh,
                       const float* a, int64_t lda, const float* w, int64_t ldw, float* da, int64_t ldda,
                       float* dw, int64_t lddw, void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0 || k < 0 || m > kMaxIndex || n > kMaxIndex || k > kMaxIndex) return fail(QHA_ERR_INVALID_ARG, "bad sizes");
  if (n == 0 || k == 0) return ok();
  if ((n & 3) || (k & 3)) return fail(QHA_ERR_INVALID_ARG, "n (%lld) and k (%lld) must be multiples of 4", (long long)n, (long long)k);
  if (!w || ldw < k || (ldw & 3) || !aligned16(w)) return fail(QHA_ERR_INVALID_ARG, "W / ldw out of contract");
  if (!dw || lddw < k || !aligned4(dw)) return fail(QHA_ERR_INVALID_ARG, "dW / lddw out of contract");
  if (m > 0) {
    if (!dh || ldg < n || (ldg & 3) || !aligned16(dh)) return fail(QHA_ERR_INVALID_ARG, "dH / ldg out of contract");
    if (!h || ldh < n || (ldh & 3) || !aligned16(h)) return fail(QHA_ERR_INVALID_ARG, "H / ldh out of contract");
    if (!a || lda < k || (lda & 3) || !aligned16(a)) return fail(QHA_ERR_INVALID_ARG, "A / lda out of contract");
    if (!da || ldda < k || !aligned4(da)) return fail(QHA_ERR_INVALID_ARG, "dA / ldda out of contract");
  }
  const size_t need = dense_bwd_required_bytes(m, n, k);
  if (need) {
    if (!workspace || workspace_bytes < need) return fail(QHA_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
    if (!aligned16(workspace)) return fail(QHA_ERR_INVALID_ARG, "workspace misaligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m > 0 && qha::panel_fits(n, k)) {
    qha::PanelArgs p;
    std::memset(&p, 0, sizeof(p));
    p.m = m;
    p.a = a;
    p.lda = lda;
    p.w = w;
    p.ldw = ldw;
    p.dh = dh;
    p.lddh = ldg;
    p.h = h;
    p.ldh = ldh;
    p.da = da;
    p.ldda = ldda;
    p.dw = dw;
    p.lddw = lddw;
    p.ws = static_cast<float*>(workspace);
    return hip_status(qha::launch_panel_bwd(p, s), "dense_backward");
  }
  // general widths: dA = dZ W (masked A operand), then dW = dZ^T A
  qha::GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  if (m > 0) {
    g.ta = 0; g.tb = 0; g.m = m; g.n = k; g.k = n;
    g.a = dh; g.lda = ldg; g.b = w; g.ldb = ldw; g.beta = 0; g.c = da; g.ldc = ldda;
    g.pro = QHA_PRO_RELU_MASK; g.aux = h; g.ld_aux = ldh; g.epi = QHA_EPI_NONE;
    qha::gemm_split_rule(g.m, g.n, g.k, &g.splits, &g.k_per_split);
    if (g.splits > 1) return fail(QHA_ERR_INVALID_ARG, "unexpected split of dA");
    const size_t pre = qha::gemm_bsplit_bytes(0, g.m, g.n, g.k);
    g.bsplit = (pre > 0 && workspace && aligned16(workspace) && workspace_bytes >= pre)
                   ? static_cast<uint32_t*>(workspace) : nullptr;
    const int st = hip_status(qha::launch_gemm(g, s), "dense_backward");
    if (st) return st;
  }
  if (qha::dw_panel_fits(m, n, k)) {
    // dW by row panels (dA has read W's parts from the workspace by now: same stream)
    qha::DwArgs d;
    std::memset(&d, 0, sizeof(d));
    d.m = m;
    d.n = static_cast<int32_t>(n);
    d.k = static_cast<int32_t>(k);
    d.dh = dh;
    d.lddh = ldg;
    d.h = h;
    d.ldh = ldh;
    d.a = a;
    d.lda = lda;
    d.ws = static_cast<float*>(workspace);
    d.ranges = qha::dw_panel_ranges(m, n, k);
    d.groups_z = static_cast<int32_t>(n / 128);
    d.groups_a = static_cast<int32_t>(k / 256);
    return hip_status(qha::launch_dw_panel(d, dw, lddw, s), "dense_backward");
  }
  g.bsplit = nullptr;
  g.ta = 1; g.tb = 0; g.m = n; g.n = k; g.k = m;
  g.a = dh; g.lda = m > 0 ? ldg : n; g.b = a; g.ldb = m > 0 ? lda : k; g.beta = 0; g.c = dw; g.ldc = lddw;
  g.pro = m > 0 ? QHA_PRO_RELU_MASK : QHA_PRO_NONE; g.aux = h; g.ld_aux = m > 0 ? ldh : n; g.epi = QHA_EPI_NONE;
  qha::gemm_split_rule(g.m, g.n, g.k, &g.splits, &g.k_per_split);
  g.ws = static_cast<double*>(workspace);
  return hip_status(qha::launch_gemm(g, s), "dense_backward");
}

}  // extern "C"
