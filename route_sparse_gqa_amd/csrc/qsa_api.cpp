// C-ABI entry points of libqsa: host-side argument checks, workspace layout
// and kernel launches.  No entry point allocates, synchronises the host or
// reads device memory; every failure is reported before anything is
// enqueued.  Argument rules follow the route-sparse GQA pages: nonempty
// dimensions, a positive kv_length, Hq a positive multiple of Hkv, a finite
// positive scale (fa4_qsa page, `fa4_sparse_gqa_attention` and `_preprocess`
// parameters), int32/int64 routes (flex_qsa page, `flex_sparse_gqa_attention`),
// an output independent of the inputs (fa4_qsa page, return value), and no
// silent fallback to another path (qsa page, `qsa_gqa_attention`).
#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>

#include "qsa.h"
#include "qsa_internal.h"

#define QSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxKv = int64_t{1} << 31;  // IDs are stored as int32
constexpr int64_t kMaxGrid = qsa::kMaxBlocks;  // 256-thread workgroups per launch; also the largest B * S_q
constexpr int64_t kMaxIndex = (int64_t{1} << 31) - 1;  // counts and positions stored as int32

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi) bytes; empty when lo == hi
};

// Byte range touched by a strided tensor (shape/strides in elements, shape >= 1); false when an
// offset does not fit in 64 bits (such strides are rejected as a size limit).
bool extent(const void* p, const int64_t* shape, const int64_t* strides, int rank, int64_t elem, Range* out) {
  int64_t lo = 0, hi = 0;
  for (int d = 0; d < rank; ++d) {
    int64_t span = 0;
    if (__builtin_mul_overflow(shape[d] - 1, strides[d], &span)) return false;
    if (__builtin_add_overflow(span < 0 ? lo : hi, span, span < 0 ? &lo : &hi)) return false;
  }
  int64_t lo_b = 0, hi_b = 0;
  if (__builtin_mul_overflow(lo, elem, &lo_b) || __builtin_mul_overflow(hi + 1, elem, &hi_b)) return false;
  const uintptr_t base = reinterpret_cast<uintptr_t>(p);
  *out = Range{base + static_cast<uintptr_t>(lo_b), base + static_cast<uintptr_t>(hi_b)};
  return true;
}

Range dense(const void* p, int64_t bytes) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(p);
  return Range{base, base + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b with overflow detection (both >= 0).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

int check_bf16_tensor(const void* p, const int64_t* strides) {
  if (strides[3] != 1) return QSA_ERR_LAYOUT;
  if (!aligned(p, 16)) return QSA_ERR_LAYOUT;
  for (int d = 0; d < 3; ++d)
    if (strides[d] % 8 != 0) return QSA_ERR_LAYOUT;
  return QSA_OK;
}

struct Sizes {
  int64_t rows = 0;      // B * S_q
  int64_t list = 0;      // B * S_q * K
  int64_t list_bytes = 0;
  int64_t count_bytes = 0;
};

// The route normalisation launch for rows of K slots over kv_length keys fits one grid.
bool route_launch_fits(int64_t rows, int64_t K, int64_t kv_length) {
  return (rows + 3) * qsa::route_normalize_items_per_row(K, kv_length) <= qsa::kMaxLaunchItems;  // 4-row groups
}

int check_route_dims(int64_t B, int64_t S_q, int64_t K, Sizes* s) {
  if (B < 1 || S_q < 1 || K < 1) return QSA_ERR_EMPTY_DIM;
  if (K > QSA_MAX_ROUTES) return QSA_ERR_LIMIT;
  if (!mul_ok(B, S_q, &s->rows) || s->rows > kMaxGrid) return QSA_ERR_LIMIT;
  if (!mul_ok(s->rows, K, &s->list) || s->list > (INT64_MAX >> 3)) return QSA_ERR_LIMIT;
  s->list_bytes = 4 * s->list;
  s->count_bytes = 4 * s->rows;
  return QSA_OK;
}

constexpr size_t kWorkspaceAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_HIP; }

}  // namespace

QSA_EXPORT const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case QSA_ERR_EMPTY_DIM: return "dimensions must be nonempty (B, S_q, S_kv, Hq, Hkv, D, K >= 1)";
    case QSA_ERR_KV_LENGTH: return "kv_length must be in [1, 2^31]";
    case QSA_ERR_HEADS: return "query_heads must be a positive multiple of kv_heads";
    case QSA_ERR_HEAD_DIM: return "head dimension must be 64, 128 or 256";
    case QSA_ERR_ROUTE_DTYPE: return "routes must be int32 or int64";
    case QSA_ERR_SCALE: return "softmax scale must be finite and positive";
    case QSA_ERR_LAYOUT: return "tensor layout unsupported (last stride 1, 16-byte aligned rows required)";
    case QSA_ERR_ALIAS: return "an output overlaps an input or another output";
    case QSA_ERR_WORKSPACE: return "workspace missing or too small";
    case QSA_ERR_LIMIT:
      return "size beyond a library limit (K <= 16384, G <= 16, index heads <= 64, kept blocks <= 4096, "
             "visible blocks <= 65536, grid size)";
    case QSA_ERR_HIP: return "HIP launch error";
    case QSA_ERR_SELECTION:
      return "selection arguments out of range (token_budget >= 1, compress_ratio >= 1, "
             "0 <= q_offset, q_offset + S_q <= S_global)";
    case QSA_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than qsa_forward_noalloc's fixed device array holds "
             "(QSA_NOALLOC_SCRATCH_BYTES); use qsa_forward with a workspace";
    default: return "unknown status";
  }
}

namespace {

constexpr int64_t kPassRowsDefault = 8192;  // rows per pass of the key-range split at the recommended size

// The attention's key-range split for these shapes; false when a size is out of range.
bool attention_plan(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K,
                    qsa::SplitPlan* plan) {
  int64_t rows = 0, tmp = 0;
  if (B < 1 || S_q < 1 || S_kv < 1 || Hq < 1 || Hkv < 1 || K < 1) return false;
  if (D != 64 && D != 128 && D != 256) return false;
  if (!mul_ok(B, S_q, &rows) || rows > kMaxGrid || S_kv > kMaxKv || Hq % Hkv != 0 || Hq / Hkv > QSA_MAX_GROUP)
    return false;
  *plan = qsa::split_plan(rows, S_kv, Hq, D);
  if (plan->use && (!mul_ok(rows, plan->P + 1, &tmp) || !mul_ok(Hq, plan->P * 2 * D, &tmp))) return false;
  return true;
}

// Rows per pass that fit `bytes` of split workspace (every row when they all fit in one pass, whose
// partials need one buffer; else two buffers of a pass), or 0 when fewer than min(rows, kMinPassRows) fit.
int64_t split_pass_rows(const qsa::SplitPlan& plan, int64_t rows, int64_t Hkv, size_t bytes) {
  if (bytes < static_cast<size_t>(plan.offs_bytes)) return 0;
  // split launch: pass * P * Hkv one-wavefront workgroups, plus previous pass * Hkv merging the previous pass
  const int64_t grid_rows = qsa::kMaxWaveBlocks / ((plan.P + 1) * Hkv);
  auto fits = [&](int64_t pass) {
    return static_cast<size_t>(qsa::split_workspace_bytes(plan, pass, rows)) <= bytes;
  };
  if (rows <= grid_rows && fits(rows)) return rows;
  const int64_t per_row = plan.part_o_row_bytes + plan.part_lse_row_bytes;
  int64_t pass =
      std::min({static_cast<int64_t>((bytes - plan.offs_bytes) / (2 * per_row)), grid_rows, rows - 1}) / 4 * 4;
  while (pass > 0 && !fits(pass)) pass -= 4;  // the 256-byte rounding of each part takes a few rows at most
  return pass >= std::min(rows, qsa::kMinPassRows) ? pass : 0;
}

// The smallest split workspace a call can run in: one pass of every row (one partial buffer), or two
// buffers of the smallest pass, whichever is smaller.
size_t split_min_bytes(const qsa::SplitPlan& plan, int64_t rows) {
  const int64_t one_pass = qsa::split_workspace_bytes(plan, rows, rows);
  if (rows <= qsa::kMinPassRows) return static_cast<size_t>(one_pass);
  return static_cast<size_t>(std::min(one_pass, qsa::split_workspace_bytes(plan, qsa::kMinPassRows, rows)));
}

size_t attention_ws(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K) {
  qsa::SplitPlan plan;
  if (!attention_plan(B, S_q, S_kv, Hq, Hkv, D, K, &plan) || !plan.use) return 0;
  const int64_t rows = B * S_q;
  return static_cast<size_t>(qsa::split_workspace_bytes(plan, std::min(rows, kPassRowsDefault), rows));
}

}  // namespace

QSA_EXPORT size_t qsa_attention_workspace_size(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                                               int64_t D, int64_t K) {
  return attention_ws(B, S_q, S_kv, Hq, Hkv, D, K);
}

QSA_EXPORT size_t qsa_forward_workspace_size(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                                             int64_t D, int64_t K) {
  Sizes s;
  qsa::SplitPlan plan;
  if (!attention_plan(B, S_q, S_kv, Hq, Hkv, D, K, &plan)) return 0;
  if (!mul_ok(B, S_q, &s.rows) || !mul_ok(s.rows, K, &s.list) || s.list > (INT64_MAX >> 3)) return 0;
  return round_up(static_cast<size_t>(4 * s.list), kWorkspaceAlign) +
         round_up(static_cast<size_t>(4 * s.rows), kWorkspaceAlign) + attention_ws(B, S_q, S_kv, Hq, Hkv, D, K);
}

QSA_EXPORT int qsa_preprocess(const void* routes, int routes_dtype, int64_t B, int64_t S_q, int64_t K,
                              const int64_t route_strides[3], int64_t kv_length, int32_t* route_list,
                              int32_t* route_count, uint8_t* membership, int32_t* tile_class, void* stream) {
  Sizes s;
  if (int st = check_route_dims(B, S_q, K, &s)) return st;
  if (routes == nullptr || route_strides == nullptr || route_list == nullptr || route_count == nullptr)
    return QSA_ERR_NULL_POINTER;
  if (kv_length < 1 || kv_length > kMaxKv) return QSA_ERR_KV_LENGTH;
  if (!route_launch_fits(s.rows, K, kv_length)) return QSA_ERR_LIMIT;
  if (routes_dtype != QSA_INT32 && routes_dtype != QSA_INT64) return QSA_ERR_ROUTE_DTYPE;
  const int64_t relem = routes_dtype == QSA_INT64 ? 8 : 4;
  if (!aligned(routes, relem) || !aligned(route_list, 4) || !aligned(route_count, 4)) return QSA_ERR_LAYOUT;
  if (membership != nullptr && !aligned(membership, 16)) return QSA_ERR_LAYOUT;
  if (tile_class != nullptr && !aligned(tile_class, 4)) return QSA_ERR_LAYOUT;

  const int64_t ldm = (kv_length + QSA_TILE - 1) / QSA_TILE * QSA_TILE;
  const int64_t n_ti = (S_q + QSA_TILE - 1) / QSA_TILE, n_tj = (kv_length + QSA_TILE - 1) / QSA_TILE;
  int64_t mem_bytes = 0, tiles = 0;
  if (membership != nullptr && !mul_ok(s.rows, ldm, &mem_bytes)) return QSA_ERR_LIMIT;
  if (!mul_ok(B * n_ti, n_tj, &tiles) || tiles > (INT64_MAX >> 3)) return QSA_ERR_LIMIT;
  if ((membership != nullptr || tile_class != nullptr) &&
      (B * n_ti * ((ldm + qsa::kMemSegCols - 1) / qsa::kMemSegCols) * qsa::kMemGroups > kMaxGrid ||
       (tiles + 255) / 256 > kMaxGrid))
    return QSA_ERR_LIMIT;

  const int64_t rshape[3] = {B, S_q, K};
  Range r_in;
  if (!extent(routes, rshape, route_strides, 3, relem, &r_in)) return QSA_ERR_LIMIT;
  const Range outs[4] = {dense(route_list, s.list_bytes), dense(route_count, s.count_bytes),
                         membership ? dense(membership, mem_bytes) : Range{},
                         tile_class ? dense(tile_class, 4 * tiles) : Range{}};
  for (int a = 0; a < 4; ++a) {
    if (overlap(outs[a], r_in)) return QSA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return QSA_ERR_ALIAS;
  }

  (void)hipGetLastError();  // clear a stale error so the checks below see only ours
  hipStream_t st = as_stream(stream);
  int rc = hip_status(qsa::launch_route_normalize(routes, routes_dtype == QSA_INT64, B, S_q, K, route_strides,
                                                  kv_length, route_list, route_count, tile_class,
                                                  tile_class ? tiles : 0, st));
  if (rc != QSA_OK) return rc;
  return hip_status(
      qsa::launch_membership_tiles(route_list, route_count, B, S_q, K, kv_length, membership, tile_class, st));
}

QSA_EXPORT int qsa_tile_lists(const int32_t* tile_class, int64_t B, int64_t n_rows, int64_t n_cols,
                              int32_t* partial_count, int32_t* partial_idx, int32_t* full_count, int32_t* full_idx,
                              int32_t* rev_partial_count, int32_t* rev_partial_idx, int32_t* rev_full_count,
                              int32_t* rev_full_idx, void* stream) {
  if (B < 1 || n_rows < 1 || n_cols < 1) return QSA_ERR_EMPTY_DIM;
  if (tile_class == nullptr) return QSA_ERR_NULL_POINTER;
  int64_t tiles = 0, rows = 0, cols = 0;
  if (n_rows > kMaxIndex || n_cols > kMaxIndex || !mul_ok(B, n_rows, &rows) || !mul_ok(B, n_cols, &cols) ||
      !mul_ok(rows, n_cols, &tiles) || tiles > (INT64_MAX >> 3) || (rows + cols + 3) / 4 > kMaxGrid)
    return QSA_ERR_LIMIT;
  int32_t* const out[8] = {partial_count, partial_idx, full_count, full_idx,
                           rev_partial_count, rev_partial_idx, rev_full_count, rev_full_idx};
  const int64_t elems[8] = {rows, tiles, rows, tiles, cols, tiles, cols, tiles};
  if (!aligned(tile_class, 4)) return QSA_ERR_LAYOUT;
  for (int a = 0; a < 8; ++a)
    if (out[a] != nullptr && !aligned(out[a], 4)) return QSA_ERR_LAYOUT;
  const Range in = dense(tile_class, 4 * tiles);
  for (int a = 0; a < 8; ++a) {
    const Range ra = out[a] ? dense(out[a], 4 * elems[a]) : Range{};
    if (overlap(ra, in)) return QSA_ERR_ALIAS;
    for (int b = a + 1; b < 8; ++b)
      if (overlap(ra, out[b] ? dense(out[b], 4 * elems[b]) : Range{})) return QSA_ERR_ALIAS;
  }
  (void)hipGetLastError();
  return hip_status(qsa::launch_tile_lists(tile_class, B, n_rows, n_cols, out, as_stream(stream)));
}

namespace {

int check_attention(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
                    const void* v, const int64_t v_strides[4], int64_t B, int64_t S_q, int64_t S_kv,
                    int64_t Hq, int64_t Hkv, int64_t D, int64_t K, float scale, void* out, Sizes* s,
                    Range* r_q, Range* r_k, Range* r_v, Range* r_out) {
  if (S_kv < 1 || Hq < 1 || Hkv < 1 || D < 1) return QSA_ERR_EMPTY_DIM;
  if (int st = check_route_dims(B, S_q, K, s)) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || q_strides == nullptr ||
      k_strides == nullptr || v_strides == nullptr)
    return QSA_ERR_NULL_POINTER;
  if (S_kv > kMaxKv) return QSA_ERR_KV_LENGTH;
  if (Hq % Hkv != 0) return QSA_ERR_HEADS;
  if (D != 64 && D != 128 && D != 256) return QSA_ERR_HEAD_DIM;
  if (Hq / Hkv > QSA_MAX_GROUP) return QSA_ERR_LIMIT;
  if (!std::isfinite(scale) || !(scale > 0.f)) return QSA_ERR_SCALE;
  if (int st = check_bf16_tensor(q, q_strides)) return st;
  if (int st = check_bf16_tensor(k, k_strides)) return st;
  if (int st = check_bf16_tensor(v, v_strides)) return st;
  if (!aligned(out, 16)) return QSA_ERR_LAYOUT;
  int64_t units = 0, out_elems = 0;
  if (!mul_ok(s->rows, Hkv, &units) || units > qsa::kMaxWaveBlocks) return QSA_ERR_LIMIT;  // one workgroup per unit
  int64_t row_elems = 0;
  if (!mul_ok(Hq, D, &row_elems) || !mul_ok(s->rows, row_elems, &out_elems) || out_elems > (INT64_MAX >> 2))
    return QSA_ERR_LIMIT;
  const int64_t qshape[4] = {B, S_q, Hq, D}, kshape[4] = {B, S_kv, Hkv, D};
  if (!extent(q, qshape, q_strides, 4, 2, r_q) || !extent(k, kshape, k_strides, 4, 2, r_k) ||
      !extent(v, kshape, v_strides, 4, 2, r_v))
    return QSA_ERR_LIMIT;
  *r_out = dense(out, 2 * out_elems);
  if (overlap(*r_out, *r_q) || overlap(*r_out, *r_k) || overlap(*r_out, *r_v)) return QSA_ERR_ALIAS;
  return QSA_OK;
}

qsa::AttnArgs attn_args(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
                        const void* v, const int64_t v_strides[4], const int32_t* list, const int32_t* count,
                        int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K,
                        float scale, void* out, float* lse = nullptr) {
  qsa::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  std::memcpy(a.qs, q_strides, sizeof a.qs);
  std::memcpy(a.ks, k_strides, sizeof a.ks);
  std::memcpy(a.vs, v_strides, sizeof a.vs);
  a.route_list = list;
  a.route_count = count;
  a.B = B; a.S_q = S_q; a.S_kv = S_kv; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.K = K;
  a.scale = scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return a;
}

// Plans the key-range split, checks the workspace for it and launches the attention.
int run_attention(const qsa::AttnArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  qsa::SplitPlan plan;
  if (!attention_plan(a.B, a.S_q, a.S_kv, a.Hq, a.Hkv, a.D, a.K, &plan)) return QSA_ERR_LIMIT;
  qsa::SplitBuffers w{};
  if (plan.use) {
    const int64_t rows = a.B * a.S_q;
    if (workspace == nullptr || !aligned(workspace, kWorkspaceAlign)) return QSA_ERR_WORKSPACE;
    w.pass_rows = split_pass_rows(plan, rows, a.Hkv, workspace_bytes);
    if (w.pass_rows == 0) return QSA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    w.offs = reinterpret_cast<int32_t*>(ws);
    const size_t o_bytes = round_up(static_cast<size_t>(w.pass_rows * plan.part_o_row_bytes), kWorkspaceAlign);
    const size_t lse_bytes = round_up(static_cast<size_t>(w.pass_rows * plan.part_lse_row_bytes), kWorkspaceAlign);
    for (int j = 0; j < 2; ++j) {  // the second buffer is used only when there is more than one pass
      char* buf = ws + plan.offs_bytes + (w.pass_rows < rows ? j : 0) * (o_bytes + lse_bytes);
      w.part_o[j] = reinterpret_cast<uint16_t*>(buf);
      w.part_lse[j] = reinterpret_cast<float*>(buf + o_bytes);
    }
  }
  return hip_status(qsa::launch_gather_attention(a, plan, w, stream));
}

// Bytes of the attention workspace a call uses (what the aliasing checks cover).
size_t attention_ws_used(const qsa::AttnArgs& a, size_t workspace_bytes) {
  qsa::SplitPlan plan;
  if (!attention_plan(a.B, a.S_q, a.S_kv, a.Hq, a.Hkv, a.D, a.K, &plan) || !plan.use) return 0;
  const int64_t pass = split_pass_rows(plan, a.B * a.S_q, a.Hkv, workspace_bytes);
  return pass > 0 ? static_cast<size_t>(qsa::split_workspace_bytes(plan, pass, a.B * a.S_q)) : 0;
}

}  // namespace

namespace qsa {

int forward_entry(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
                  const void* v, const int64_t v_strides[4], const void* routes, int routes_dtype,
                  const int64_t route_strides[3], int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                  int64_t D, int64_t K, float scale, void* out, void* workspace, size_t workspace_bytes,
                  ScratchFn scratch, void* stream) {
  Sizes s;
  Range r_q, r_k, r_v, r_out;
  if (int st = check_attention(q, q_strides, k, k_strides, v, v_strides, B, S_q, S_kv, Hq, Hkv, D, K, scale,
                               out, &s, &r_q, &r_k, &r_v, &r_out))
    return st;
  if (routes == nullptr || route_strides == nullptr) return QSA_ERR_NULL_POINTER;
  if (routes_dtype != QSA_INT32 && routes_dtype != QSA_INT64) return QSA_ERR_ROUTE_DTYPE;
  if (!route_launch_fits(s.rows, K, S_kv)) return QSA_ERR_LIMIT;
  const int64_t relem = routes_dtype == QSA_INT64 ? 8 : 4;
  if (!aligned(routes, relem)) return QSA_ERR_LAYOUT;
  // the lists and counts first, then the attention's own workspace
  const size_t lists = round_up(static_cast<size_t>(s.list_bytes), kWorkspaceAlign) +
                       round_up(static_cast<size_t>(s.count_bytes), kWorkspaceAlign);
  qsa::SplitPlan plan;
  if (!attention_plan(B, S_q, S_kv, Hq, Hkv, D, K, &plan)) return QSA_ERR_LIMIT;
  if (scratch != nullptr) {  // the caller's fixed scratch replaces the workspace
    const size_t need = lists + (plan.use ? split_min_bytes(plan, s.rows) : 0);
    if (int st = scratch(need, stream, &workspace, &workspace_bytes)) return st;
  }
  if (workspace == nullptr || !aligned(workspace, kWorkspaceAlign)) return QSA_ERR_WORKSPACE;
  if (workspace_bytes < lists) return QSA_ERR_WORKSPACE;
  int32_t* list = static_cast<int32_t*>(workspace);
  int32_t* count = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                              round_up(static_cast<size_t>(s.list_bytes), kWorkspaceAlign));
  const qsa::AttnArgs a =
      attn_args(q, q_strides, k, k_strides, v, v_strides, list, count, B, S_q, S_kv, Hq, Hkv, D, K, scale, out);
  void* att_ws = static_cast<char*>(workspace) + lists;
  const size_t att_bytes = workspace_bytes - lists;
  const int64_t rshape[3] = {B, S_q, K};
  Range r_in;
  if (!extent(routes, rshape, route_strides, 3, relem, &r_in)) return QSA_ERR_LIMIT;
  const Range r_ws = dense(workspace, static_cast<int64_t>(lists + attention_ws_used(a, att_bytes)));
  if (overlap(r_out, r_in) || overlap(r_out, r_ws) || overlap(r_ws, r_q) || overlap(r_ws, r_k) ||
      overlap(r_ws, r_v) || overlap(r_ws, r_in))
    return QSA_ERR_ALIAS;
  // the split's workspace is checked before anything is enqueued
  if (plan.use && split_pass_rows(plan, s.rows, Hkv, att_bytes) == 0) return QSA_ERR_WORKSPACE;

  (void)hipGetLastError();
  hipStream_t st = as_stream(stream);
  int rc = hip_status(qsa::launch_route_normalize(routes, routes_dtype == QSA_INT64, B, S_q, K, route_strides,
                                                  S_kv, list, count, nullptr, 0, st));
  if (rc != QSA_OK) return rc;
  return run_attention(a, att_ws, att_bytes, st);
}

}  // namespace qsa

QSA_EXPORT int qsa_forward(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
                           const void* v, const int64_t v_strides[4], const void* routes, int routes_dtype,
                           const int64_t route_strides[3], int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq,
                           int64_t Hkv, int64_t D, int64_t K, float scale, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return qsa::forward_entry(q, q_strides, k, k_strides, v, v_strides, routes, routes_dtype, route_strides, B, S_q,
                            S_kv, Hq, Hkv, D, K, scale, out, workspace, workspace_bytes, nullptr, stream);
}

QSA_EXPORT int qsa_forward_preprocessed(const void* q, const int64_t q_strides[4], const void* k,
                                        const int64_t k_strides[4], const void* v, const int64_t v_strides[4],
                                        const int32_t* route_list, const int32_t* route_count, int64_t B,
                                        int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K,
                                        float scale, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  Sizes s;
  Range r_q, r_k, r_v, r_out;
  if (int st = check_attention(q, q_strides, k, k_strides, v, v_strides, B, S_q, S_kv, Hq, Hkv, D, K, scale,
                               out, &s, &r_q, &r_k, &r_v, &r_out))
    return st;
  if (route_list == nullptr || route_count == nullptr) return QSA_ERR_NULL_POINTER;
  if (!aligned(route_list, 4) || !aligned(route_count, 4)) return QSA_ERR_LAYOUT;
  const Range r_list = dense(route_list, s.list_bytes), r_count = dense(route_count, s.count_bytes);
  if (overlap(r_out, r_list) || overlap(r_out, r_count)) return QSA_ERR_ALIAS;
  if (lse != nullptr) {
    if (!aligned(lse, 4)) return QSA_ERR_LAYOUT;
    const Range r_lse = dense(lse, 4 * s.rows * Hq);
    if (overlap(r_lse, r_out) || overlap(r_lse, r_q) || overlap(r_lse, r_k) || overlap(r_lse, r_v) ||
        overlap(r_lse, r_list) || overlap(r_lse, r_count))
      return QSA_ERR_ALIAS;
  }
  const qsa::AttnArgs a = attn_args(q, q_strides, k, k_strides, v, v_strides, route_list, route_count, B, S_q,
                                    S_kv, Hq, Hkv, D, K, scale, out, lse);
  const size_t used = workspace != nullptr ? attention_ws_used(a, workspace_bytes) : 0;
  if (used > 0) {
    const Range r_ws = dense(workspace, static_cast<int64_t>(used));
    const Range r_lse = lse != nullptr ? dense(lse, 4 * s.rows * Hq) : Range{};
    if (overlap(r_ws, r_out) || overlap(r_ws, r_q) || overlap(r_ws, r_k) || overlap(r_ws, r_v) ||
        overlap(r_ws, r_list) || overlap(r_ws, r_count) || overlap(r_ws, r_lse))
      return QSA_ERR_ALIAS;
  }
  (void)hipGetLastError();
  return run_attention(a, workspace, workspace_bytes, as_stream(stream));
}

namespace {

// Backward workspace: delta, then the key-segment buffers, then the partial
// sums of split tiles, each 256-B aligned.
struct BwdLayout {
  size_t delta = 0, bits = 0, chunk_prefix = 0, totals = 0, tile_start = 0, segs = 0, part_start = 0,
         slot_start = 0, plan = 0, partial = 0, offs = 0, dq_part = 0, dq_part2 = 0, total = 0;
  int64_t n_kt = 0, capacity = 0, max_parts = 0, dq_pass_rows = 0;
  qsa::SplitPlan split;
};

bool bwd_layout(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K, BwdLayout* l) {
  if (B < 1 || S_q < 1 || S_kv < 1 || Hq < 1 || Hkv < 1 || D < 1 || K < 1) return false;
  int64_t rows = 0, heads = 0, words = 0, chunks = 0, tiles = 0, cap = 0, partial = 0;
  l->n_kt = (S_kv + qsa::kSegKeyTile - 1) / qsa::kSegKeyTile;
  const int64_t W = (S_q + 31) / 32;
  const int64_t C = (S_q + qsa::kSegChunkRows - 1) / qsa::kSegChunkRows;
  if (!mul_ok(B, S_q, &rows) || !mul_ok(rows, Hq, &heads) || !mul_ok(B * W, l->n_kt, &words) ||
      !mul_ok(B * C, l->n_kt, &chunks) || !mul_ok(B, l->n_kt, &tiles) ||
      !mul_ok(rows, K < l->n_kt ? K : l->n_kt, &cap))
    return false;
  // segment positions, chunk prefixes, tile and part starts are int32
  if (cap > kMaxIndex || chunks > kMaxIndex || tiles + 1 > kMaxIndex / 2 || heads > (INT64_MAX >> 3) ||
      words > (INT64_MAX >> 3))
    return false;
  l->capacity = cap;
  l->max_parts = qsa::kSegPartsTotal / Hkv > 1 ? qsa::kSegPartsTotal / Hkv : 1;
  const int64_t slots = qsa::seg_max_slots(l->max_parts, cap);
  if (!mul_ok(slots * Hkv, 512 * D, &partial)) return false;
  size_t off = 0;
  auto take = [&](size_t* at, int64_t bytes) {
    *at = off;
    off += round_up(static_cast<size_t>(bytes), kWorkspaceAlign);
  };
  take(&l->delta, 4 * heads);
  take(&l->bits, 4 * words);
  take(&l->chunk_prefix, 4 * chunks);
  take(&l->totals, 4 * tiles);
  take(&l->tile_start, 4 * (tiles + 1));
  take(&l->segs, 16 * cap);
  take(&l->part_start, 4 * (tiles + 1));
  take(&l->slot_start, 4 * tiles);
  take(&l->plan, 8);
  take(&l->partial, partial);
  // the key-range split of dq (when the forward would split): range starts and one pass of fp32 partial sums
  l->split = qsa::split_plan(rows, S_kv, Hq, D);
  if (l->split.use) {
    int64_t part_bytes = 0;
    l->dq_pass_rows = rows < qsa::kDqPassRows ? rows : qsa::kDqPassRows;
    if (!mul_ok(l->dq_pass_rows * Hq, static_cast<int64_t>(l->split.P) * D * 4, &part_bytes)) return false;
    take(&l->offs, 4 * rows * (l->split.P + 1));
    take(&l->dq_part, part_bytes);
    l->dq_part2 = l->dq_part;
    if (l->dq_pass_rows < rows) take(&l->dq_part2, part_bytes);  // a pass's sums are added during the next
  }
  l->total = off;
  return true;
}

}  // namespace

QSA_EXPORT size_t qsa_backward_workspace_size(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                                              int64_t D, int64_t K) {
  BwdLayout l;
  return bwd_layout(B, S_q, S_kv, Hq, Hkv, D, K, &l) ? l.total : 0;
}

QSA_EXPORT int qsa_backward(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
                            const void* v, const int64_t v_strides[4], const void* out, const void* dout,
                            const int64_t dout_strides[4], const float* lse, const int32_t* route_list,
                            const int32_t* route_count, int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq,
                            int64_t Hkv, int64_t D, int64_t K, float scale, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Sizes s;
  Range r_q, r_k, r_v, r_dq;
  if (int st = check_attention(q, q_strides, k, k_strides, v, v_strides, B, S_q, S_kv, Hq, Hkv, D, K, scale, dq,
                               &s, &r_q, &r_k, &r_v, &r_dq))
    return st;
  if (out == nullptr || dout == nullptr || dout_strides == nullptr || lse == nullptr || route_list == nullptr ||
      route_count == nullptr || dk == nullptr || dv == nullptr)
    return QSA_ERR_NULL_POINTER;
  if (int st = check_bf16_tensor(dout, dout_strides)) return st;
  if (!aligned(out, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(route_list, 4) ||
      !aligned(route_count, 4))
    return QSA_ERR_LAYOUT;
  BwdLayout l;
  if (!bwd_layout(B, S_q, S_kv, Hq, Hkv, D, K, &l)) return QSA_ERR_LIMIT;
  int64_t kv_elems = 0;
  if (!mul_ok(B * S_kv, Hkv * D, &kv_elems) || kv_elems > (INT64_MAX >> 2)) return QSA_ERR_LIMIT;
  // grids: dk/dv and its reduction, dq per (row, KV head) in one-wavefront workgroups (delta and the
  // combine per four of them), the split dq per (range, KV head, row of a pass) plus the previous pass's
  // (row, KV head) units, the segment counts
  if ((l.n_kt * B + l.max_parts) * Hkv > kMaxGrid || l.n_kt * B * 4 * Hkv > kMaxGrid ||
      s.rows * Hkv > qsa::kMaxWaveBlocks ||
      (l.split.use && l.dq_pass_rows * (l.split.P + 1) * Hkv > qsa::kMaxWaveBlocks) ||
      (B * ((S_q + qsa::kSegChunkRows - 1) / qsa::kSegChunkRows) * l.n_kt + 255) / 256 > kMaxGrid)
    return QSA_ERR_LIMIT;
  if (workspace == nullptr || workspace_bytes < l.total || !aligned(workspace, kWorkspaceAlign))
    return QSA_ERR_WORKSPACE;

  const int64_t qshape[4] = {B, S_q, Hq, D};
  const Range r_o = dense(out, 2 * s.rows * Hq * D);
  Range r_g;
  if (!extent(dout, qshape, dout_strides, 4, 2, &r_g)) return QSA_ERR_LIMIT;
  const Range r_lse = dense(lse, 4 * s.rows * Hq);
  const Range r_list = dense(route_list, s.list_bytes), r_count = dense(route_count, s.count_bytes);
  const Range r_dk = dense(dk, 2 * kv_elems), r_dv = dense(dv, 2 * kv_elems);
  const Range r_ws = dense(workspace, static_cast<int64_t>(l.total));
  const Range ins[8] = {r_q, r_k, r_v, r_o, r_g, r_lse, r_list, r_count};
  const Range outs[4] = {r_dq, r_dk, r_dv, r_ws};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 8; ++b)
      if (overlap(outs[a], ins[b])) return QSA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return QSA_ERR_ALIAS;
  }

  char* ws = static_cast<char*>(workspace);
  qsa::SegmentBuffers w;
  w.bits = reinterpret_cast<uint32_t*>(ws + l.bits);
  w.chunk_prefix = reinterpret_cast<int32_t*>(ws + l.chunk_prefix);
  w.totals = reinterpret_cast<int32_t*>(ws + l.totals);
  w.tile_start = reinterpret_cast<int32_t*>(ws + l.tile_start);
  w.segs = reinterpret_cast<int4*>(ws + l.segs);
  w.capacity = l.capacity;
  w.part_start = reinterpret_cast<int32_t*>(ws + l.part_start);
  w.slot_start = reinterpret_cast<int32_t*>(ws + l.slot_start);
  w.plan = reinterpret_cast<int32_t*>(ws + l.plan);
  w.max_parts = l.max_parts;

  qsa::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  std::memcpy(a.qs, q_strides, sizeof a.qs);
  std::memcpy(a.ks, k_strides, sizeof a.ks);
  std::memcpy(a.vs, v_strides, sizeof a.vs);
  std::memcpy(a.gs, dout_strides, sizeof a.gs);
  a.lse = lse;
  a.delta = reinterpret_cast<float*>(ws + l.delta);
  a.route_list = route_list;
  a.route_count = route_count;
  a.seg_start = w.tile_start;
  a.segs = w.segs;
  a.part_start = w.part_start;
  a.slot_start = w.slot_start;
  a.plan = w.plan;
  a.partial = reinterpret_cast<float*>(ws + l.partial);
  a.max_parts = l.max_parts;
  a.B = B; a.S_q = S_q; a.S_kv = S_kv; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.K = K;
  a.scale = scale;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.split = l.split;
  a.offs = l.split.use ? reinterpret_cast<int32_t*>(ws + l.offs) : nullptr;
  a.dq_part[0] = l.split.use ? reinterpret_cast<float*>(ws + l.dq_part) : nullptr;
  a.dq_part[1] = l.split.use ? reinterpret_cast<float*>(ws + l.dq_part2) : nullptr;
  a.dq_pass_rows = l.dq_pass_rows;

  (void)hipGetLastError();
  hipStream_t st = as_stream(stream);
  int rc = hip_status(qsa::launch_attention_dq(a, st));
  if (rc != QSA_OK) return rc;
  rc = hip_status(qsa::launch_key_segments(route_list, route_count, B, S_q, K, S_kv, w, st));
  if (rc != QSA_OK) return rc;
  return hip_status(qsa::launch_attention_dkdv(a, st));
}

namespace {

// Shape checks of route selection; fills the derived sizes.
struct SelectSizes {
  int64_t width = 0, rows = 0, tile_rows = 0, ld = 0, tiles = 0, full_bytes = 0, tile_bytes = 0;
};

int check_select_dims(int64_t B, int64_t S_q, int64_t H, int64_t D, int64_t S_global, int64_t q_offset,
                      int64_t token_budget, int64_t c, SelectSizes* z) {
  if (B < 1 || S_q < 1 || H < 1 || D < 1 || S_global < 1) return QSA_ERR_EMPTY_DIM;
  if (token_budget < 1 || c < 1 || q_offset < 0 || q_offset > S_global || S_q > S_global - q_offset)
    return QSA_ERR_SELECTION;
  if (D != 64 && D != 128 && D != 256) return QSA_ERR_HEAD_DIM;
  if (H > QSA_MAX_INDEX_HEADS || S_global > kMaxIndex || token_budget / c > QSA_MAX_SELECT_BLOCKS ||
      S_global / c > QSA_MAX_VISIBLE_BLOCKS || token_budget > kMaxIndex - c)
    return QSA_ERR_LIMIT;
  z->width = token_budget + c - 1;
  if (!mul_ok(B, S_q, &z->rows) || z->rows > kMaxGrid) return QSA_ERR_LIMIT;
  // the top-k takes one workgroup per row: 1024 threads when a row can see more than 256 * 64 blocks
  if ((q_offset + S_q) / c > 256 * 64 && z->rows > qsa::kMaxLaunchItems / 1024) return QSA_ERR_LIMIT;
  int64_t outs = 0;
  if (!mul_ok(z->rows, z->width, &outs) || outs > (INT64_MAX >> 3)) return QSA_ERR_LIMIT;
  z->tile_rows = qsa::select_rows_per_tile(H);
  z->ld = qsa::select_score_ld(S_q, q_offset, c);
  z->tiles = B * ((S_q + z->tile_rows - 1) / z->tile_rows);
  const int64_t n_chunks = (z->ld + 127) / 128;
  if ((z->tiles + 7) / 8 * 8 > kMaxGrid / n_chunks) return QSA_ERR_LIMIT;
  z->tile_bytes = 4 * z->tile_rows * z->ld;
  if (!mul_ok(z->tiles, z->tile_bytes, &z->full_bytes) || z->full_bytes > (INT64_MAX >> 2)) return QSA_ERR_LIMIT;
  return QSA_OK;
}

}  // namespace

QSA_EXPORT size_t qsa_select_workspace_size(int64_t B, int64_t S_q, int64_t H, int64_t q_offset,
                                            int64_t compress_ratio) {
  SelectSizes z;
  if (q_offset < 0 || compress_ratio < 1 || S_q < 1 || q_offset > INT64_MAX - S_q) return 0;
  // the smallest S_global and budget these sizes allow: the workspace does not depend on them
  if (check_select_dims(B, S_q, H, 64, q_offset + S_q, q_offset, 1, compress_ratio, &z) != QSA_OK &&
      check_select_dims(B, S_q, H, 64, q_offset + S_q, q_offset, compress_ratio, compress_ratio, &z) != QSA_OK)
    return 0;
  return round_up(static_cast<size_t>(z.full_bytes), kWorkspaceAlign);
}

QSA_EXPORT size_t qsa_select_chunk_workspace_size(int64_t B, int64_t S_q, int64_t H, int64_t q_offset,
                                                  int64_t compress_ratio, int64_t query_chunk_size) {
  SelectSizes z;
  if (query_chunk_size < 1 || q_offset < 0 || compress_ratio < 1 || S_q < 1 || q_offset > INT64_MAX - S_q) return 0;
  if (check_select_dims(B, S_q, H, 64, q_offset + S_q, q_offset, 1, compress_ratio, &z) != QSA_OK &&
      check_select_dims(B, S_q, H, 64, q_offset + S_q, q_offset, compress_ratio, compress_ratio, &z) != QSA_OK)
    return 0;
  const int64_t tiles = (query_chunk_size + z.tile_rows - 1) / z.tile_rows;  // whole row tiles per pass
  const int64_t bytes = tiles < z.tiles ? tiles * z.tile_bytes : z.full_bytes;
  return round_up(static_cast<size_t>(bytes), kWorkspaceAlign);
}

QSA_EXPORT int qsa_select_token_ids(const void* index_q, const int64_t q_strides[4], const void* block_k,
                                    const int64_t k_strides[4], const int64_t* seq_lens, int64_t B, int64_t S_q,
                                    int64_t H, int64_t D, int64_t S_global, int64_t q_offset, int64_t token_budget,
                                    int64_t compress_ratio, int32_t* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  SelectSizes z;
  if (int st = check_select_dims(B, S_q, H, D, S_global, q_offset, token_budget, compress_ratio, &z)) return st;
  if (index_q == nullptr || q_strides == nullptr || block_k == nullptr || k_strides == nullptr ||
      seq_lens == nullptr || out == nullptr)
    return QSA_ERR_NULL_POINTER;
  if (int st = check_bf16_tensor(index_q, q_strides)) return st;
  const int64_t ks[4] = {k_strides[0], k_strides[1], 0, k_strides[3]};  // the size-1 head dim is not walked
  if (int st = check_bf16_tensor(block_k, ks)) return st;
  if (!aligned(seq_lens, 8) || !aligned(out, 4)) return QSA_ERR_LAYOUT;
  const int64_t c = compress_ratio;
  const int64_t nv_all = (q_offset + S_q) / c;
  const bool scoring = token_budget / c > 0 && nv_all > token_budget / c;
  if (scoring && (workspace == nullptr || workspace_bytes < static_cast<size_t>(z.tile_bytes) ||
                  !aligned(workspace, kWorkspaceAlign)))
    return QSA_ERR_WORKSPACE;

  const int64_t n_blocks = S_global / c;
  const int64_t qshape[4] = {B, S_q, H, D}, kshape[4] = {B, n_blocks > 0 ? n_blocks : 1, 1, D};
  Range r_q, r_k;
  if (!extent(index_q, qshape, q_strides, 4, 2, &r_q) || !extent(block_k, kshape, ks, 4, 2, &r_k))
    return QSA_ERR_LIMIT;
  const Range r_len = dense(seq_lens, 8 * B);
  const Range r_out = dense(out, 4 * z.rows * z.width);
  const size_t used = std::min(workspace_bytes, static_cast<size_t>(z.full_bytes));
  const Range r_ws = scoring ? dense(workspace, static_cast<int64_t>(used)) : Range{};
  if (overlap(r_out, r_q) || overlap(r_out, r_k) || overlap(r_out, r_len) || overlap(r_out, r_ws) ||
      overlap(r_ws, r_q) || overlap(r_ws, r_k) || overlap(r_ws, r_len))
    return QSA_ERR_ALIAS;

  qsa::SelectArgs a;
  a.iq = static_cast<const uint16_t*>(index_q);
  a.ck = static_cast<const uint16_t*>(block_k);
  std::memcpy(a.qs, q_strides, sizeof a.qs);
  std::memcpy(a.cs, ks, sizeof a.cs);
  a.seq_lens = seq_lens;
  a.B = B; a.S_q = S_q; a.H = H; a.D = D; a.q_offset = q_offset;
  a.token_budget = token_budget; a.compress_ratio = c;
  a.out = out;
  a.scores = static_cast<float*>(workspace);
  a.workspace_bytes = scoring ? used : 0;
  (void)hipGetLastError();
  return hip_status(qsa::launch_select(a, as_stream(stream)));
}
