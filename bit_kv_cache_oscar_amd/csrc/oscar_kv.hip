// C-ABI entry points of liboscar_kv: host-side validation, workspace views and launches.
// No allocation, no synchronisation, no state beyond a per-thread error message.

#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "launch.h"
#include "oscar_kv.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_last_error[0] = '\0';
  return OSCAR_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(OSCAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int32_t check_desc_impl(const oscar_layer_desc* d) {
  if (!d) return fail(OSCAR_ERR_INVALID_ARG, "desc is null");
  if (d->head_dim != 128) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (d->group_size != 128) return fail(OSCAR_ERR_UNSUPPORTED, "group_size %d != 128", d->group_size);
  if (d->page_tokens != 64) return fail(OSCAR_ERR_UNSUPPORTED, "page_tokens %d != 64", d->page_tokens);
  if (d->sink_tokens != 64) return fail(OSCAR_ERR_UNSUPPORTED, "sink_tokens %d != 64", d->sink_tokens);
  if (d->recent_tokens != 256) return fail(OSCAR_ERR_UNSUPPORTED, "recent_tokens %d != 256", d->recent_tokens);
  if (d->n_q_heads <= 0 || d->n_kv_heads <= 0)
    return fail(OSCAR_ERR_INVALID_ARG, "head counts must be positive (%d, %d)", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(OSCAR_ERR_INVALID_ARG, "n_q_heads %d not a multiple of n_kv_heads %d", d->n_q_heads, d->n_kv_heads);
  const int gq = d->n_q_heads / d->n_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
    return fail(OSCAR_ERR_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8,16}", gq);
  if (d->n_kv_heads > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "n_kv_heads %d too large", d->n_kv_heads);
  return OSCAR_OK;
}

// As check_desc_impl, with groups of 64 or 32 dims allowed as well (the entry points that
// read or write grouped pages, and those that do not depend on the group size).
int32_t check_desc_grouped(const oscar_layer_desc* d) {
  if (!d) return fail(OSCAR_ERR_INVALID_ARG, "desc is null");
  if (d->group_size != 32 && d->group_size != 64 && d->group_size != 128)
    return fail(OSCAR_ERR_UNSUPPORTED, "group_size %d not in {32, 64, 128}", d->group_size);
  oscar_layer_desc one = *d;
  one.group_size = 128;
  return check_desc_impl(&one);
}

oscar::LayerShape shape_of(const oscar_layer_desc* d) {
  oscar::LayerShape s;
  s.n_q = d->n_q_heads;
  s.n_kv = d->n_kv_heads;
  s.gq = d->n_q_heads / d->n_kv_heads;
  s.window = d->sink_tokens + d->recent_tokens;
  return s;
}

// The INT2 pass keeps each wave's pending value sums in int32 between the (data-driven)
// moves of its reference maximum; a page adds at most 255 x 48 x 64 to one of them, so a
// wave may walk at most 2048 pages, and with four waves per workgroup a split at most
// 8192 (a request's pages are bounded by its block-table row).
constexpr long long kMaxSplitPages = 8192;

int32_t check_pages(int32_t max_pages, int32_t n_splits) {
  if (max_pages <= 0) return fail(OSCAR_ERR_INVALID_ARG, "max_pages %d <= 0", max_pages);
  if (n_splits > 0 && (static_cast<long long>(max_pages) + n_splits - 1) / n_splits > kMaxSplitPages)
    return fail(OSCAR_ERR_UNSUPPORTED, "max_pages %d over %d splits: more than %lld pages per split", max_pages,
                n_splits, kMaxSplitPages);
  return OSCAR_OK;
}

constexpr int kBulkMinRows = 64;  // oscar_demote takes the matrix-core kernel from this many tokens

int window_splits_of(const oscar_layer_desc* d) { return (d->sink_tokens + d->recent_tokens + 63) / 64; }

}  // namespace

namespace oscar {

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

// [m | l | pad | acc | query limbs | query scalars]
size_t partials_bytes(int batch, int n_q, int n_splits) {
  const size_t n = static_cast<size_t>(batch) * n_q * n_splits;
  const size_t heads = static_cast<size_t>(batch) * n_q;
  const size_t acc_off = align256(8 * n);
  const size_t ql_off = align256(acc_off + n * 128 * sizeof(float));
  const size_t qs_off = align256(ql_off + heads * 512);
  return qs_off + heads * sizeof(QueryScal);
}

// [INT2 partials + query tail | window partials | arrival counters]
size_t step_workspace_bytes(int batch, int n_q, int n_kv, int n_splits, int n_wsplits) {
  return align256(partials_bytes(batch, n_q, n_splits)) + align256(partials_bytes(batch, n_q, n_wsplits)) +
         align256(static_cast<size_t>(batch) * n_kv * 4 * kCounterStride);
}

PartialsView partials_view(void* base, int batch, int n_q, int n_splits) {
  const size_t n = static_cast<size_t>(batch) * n_q * n_splits;
  const size_t heads = static_cast<size_t>(batch) * n_q;
  const size_t acc_off = align256(8 * n);
  const size_t ql_off = align256(acc_off + n * 128 * sizeof(float));
  const size_t qs_off = align256(ql_off + heads * 512);
  char* p = static_cast<char*>(base);
  PartialsView v;
  v.m = reinterpret_cast<float*>(p);
  v.l = reinterpret_cast<float*>(p + 4 * n);
  v.acc = reinterpret_cast<float*>(p + acc_off);
  v.qlimb = p + ql_off;
  v.qscal = reinterpret_cast<QueryScal*>(p + qs_off);
  return v;
}

}  // namespace oscar

namespace oscar {
// grouped.hip: groups of 64 or 32 rotated dims (128 is the one-group format)
size_t grouped_page_bytes(int n_kv, int group);
hipError_t launch_demote_grouped(int n_kv, int group, const void* k_src, const void* v_src, int n,
                                 const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                                 const float* clip_k, const float* clip_v, void* pool, hipStream_t stream);
hipError_t launch_decode_grouped(const LayerShape& L, int group, const void* q, const void* rot_k, const void* pool,
                                 const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch,
                                 float sm_scale, int n_splits, const PartialsView& out, hipStream_t stream);
}  // namespace oscar

extern "C" {

int32_t oscar_version(void) { return 100; }

const char* oscar_status_string(int32_t status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_ERR_INVALID_ARG: return "invalid argument";
    case OSCAR_ERR_UNSUPPORTED: return "unsupported shape";
    case OSCAR_ERR_WORKSPACE: return "workspace too small";
    case OSCAR_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* oscar_last_error(void) { return g_last_error; }

int32_t oscar_check_desc(const oscar_layer_desc* desc) {
  const int32_t st = check_desc_grouped(desc);
  return st == OSCAR_OK ? ok() : st;
}

size_t oscar_page_bytes(const oscar_layer_desc* desc) {
  if (check_desc_grouped(desc) != OSCAR_OK) return 0;
  return oscar::grouped_page_bytes(desc->n_kv_heads, desc->group_size);
}

int32_t oscar_window_tokens(const oscar_layer_desc* desc) {
  if (check_desc_grouped(desc) != OSCAR_OK) return 0;
  return desc->sink_tokens + desc->recent_tokens;
}

int32_t oscar_window_splits(const oscar_layer_desc* desc) {
  if (check_desc_grouped(desc) != OSCAR_OK) return 0;
  return window_splits_of(desc);
}

size_t oscar_partials_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits) {
  if (check_desc_grouped(desc) != OSCAR_OK || batch < 0 || n_splits < 0) return 0;
  return oscar::partials_bytes(batch, desc->n_q_heads, n_splits);
}

int32_t oscar_default_splits(const oscar_layer_desc* desc, int32_t batch, int32_t max_hist_len) {
  if (check_desc_grouped(desc) != OSCAR_OK || batch <= 0) return 1;
  const long long pages = (static_cast<long long>(max_hist_len > 0 ? max_hist_len : 0) + 63) / 64;
  const int gq = desc->n_q_heads / desc->n_kv_heads;
  // query heads per INT2 workgroup: 8, or 4 over grouped pages
  const int tile = desc->group_size == 128 ? 8 : 4;
  const long long groups = static_cast<long long>(batch) * desc->n_kv_heads * (gq > tile ? gq / tile : 1);
  // small grids: one 8-wave workgroup per compute unit (at most 256 workgroups, which the
  // fused decode runs with 8 waves); larger ones: about two 4-wave workgroups per unit
  long long s, by_pages;
  if (groups <= 128) {
    s = 256 / groups;
    by_pages = (pages + 7) / 8;  // at least one page per wave
  } else {
    s = (512 + groups / 2) / groups;
    by_pages = (pages + 3) / 4;
  }
  if (s > by_pages) s = by_pages;
  // no split may hold more pages than the INT2 pass accepts
  const long long need = (pages + kMaxSplitPages - 1) / kMaxSplitPages;
  if (s < need) s = need;
  if (s < 1) s = 1;
  if (s > 65535) s = 65535;
  return static_cast<int32_t>(s);
}

}  // extern "C"

namespace {

// The codebook argument of the Lloyd-Max entry points: non-null and 4-byte aligned.
int32_t check_codebook(const void* codebook) {
  if (!codebook) return fail(OSCAR_ERR_INVALID_ARG, "null codebook");
  if (reinterpret_cast<uintptr_t>(codebook) % 4 != 0) return fail(OSCAR_ERR_INVALID_ARG, "codebook not 4-byte aligned");
  return OSCAR_OK;
}

int32_t demote_impl(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                    const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                    const float* clip_k, const float* clip_v, const uint32_t* codebook, void* pool, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (n < 0) return fail(OSCAR_ERR_INVALID_ARG, "n %d < 0", n);
  if (n == 0) return ok();
  if (!k_src || !v_src || !dst_page || !dst_slot || !rot_k || !rot_v || !clip_k || !clip_v || !pool)
    return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (2LL * n * desc->n_kv_heads > 0x7FFFFFFFLL)
    return fail(OSCAR_ERR_UNSUPPORTED, "2 * n * n_kv_heads exceeds the grid limit");
  const oscar::LayerShape L = shape_of(desc);
  // many rows: the matrix-core kernel (whole 16-token tiles); a few: one workgroup per row
  if (n >= kBulkMinRows)
    return hip_status(oscar::launch_demote_bulk(L, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v,
                                                pool, static_cast<hipStream_t>(stream), codebook),
                      "demote launch");
  return hip_status(oscar::launch_demote_rows(L, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v,
                                              pool, static_cast<hipStream_t>(stream), codebook),
                    "demote launch");
}

}  // namespace

extern "C" {

int32_t oscar_demote(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                     const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                     const float* clip_k, const float* clip_v, void* pool, void* stream) {
  return demote_impl(desc, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, nullptr, pool, stream);
}

int32_t oscar_demote_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                              const float* clip_k, const float* clip_v, const uint8_t* codebook, void* pool,
                              void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return demote_impl(desc, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v,
                     reinterpret_cast<const uint32_t*>(codebook), pool, stream);
}

int32_t oscar_decode_int2(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* pool,
                          const int32_t* block_table, int32_t max_pages, const int32_t* hist_len, int32_t batch,
                          float sm_scale, int32_t n_splits, void* partials, size_t partials_bytes, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (n_splits <= 0 || n_splits > 65535) return fail(OSCAR_ERR_INVALID_ARG, "n_splits %d out of [1, 65535]", n_splits);
  if (int32_t e = check_pages(max_pages, n_splits)) return e;
  if (!q || !rot_k || !pool || !block_table || !hist_len || !partials)
    return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const size_t need = oscar::partials_bytes(batch, desc->n_q_heads, n_splits);
  if (partials_bytes < need)
    return fail(OSCAR_ERR_WORKSPACE, "partials workspace %zu < %zu bytes", partials_bytes, need);
  const oscar::LayerShape L = shape_of(desc);
  const oscar::PartialsView v = oscar::partials_view(partials, batch, desc->n_q_heads, n_splits);
  return hip_status(oscar::launch_decode_int2(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale,
                                              n_splits, v, static_cast<hipStream_t>(stream)),
                    "decode_int2 launch");
}

int32_t oscar_decode_bf16(const oscar_layer_desc* desc, const void* q, const void* k_win, const void* v_win,
                          const int32_t* win_len, int32_t batch, float sm_scale, void* win_partials,
                          size_t win_partials_bytes, void* stream) {
  int32_t st = check_desc_grouped(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (!q || !k_win || !v_win || !win_len || !win_partials) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const int ws = window_splits_of(desc);
  const size_t need = oscar::partials_bytes(batch, desc->n_q_heads, ws);
  if (win_partials_bytes < need)
    return fail(OSCAR_ERR_WORKSPACE, "window partials workspace %zu < %zu bytes", win_partials_bytes, need);
  const oscar::LayerShape L = shape_of(desc);
  const oscar::PartialsView v = oscar::partials_view(win_partials, batch, desc->n_q_heads, ws);
  return hip_status(oscar::launch_decode_bf16(L, q, k_win, v_win, win_len, batch, sm_scale, ws, v,
                                              static_cast<hipStream_t>(stream)),
                    "decode_bf16 launch");
}

size_t oscar_dense_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t capacity) {
  if (check_desc_impl(desc) != OSCAR_OK || batch < 0 || capacity < 0 || capacity % 64 != 0) return 0;
  return oscar::partials_bytes(batch, desc->n_q_heads, capacity / 64);
}

int32_t oscar_decode_dense_bf16(const oscar_layer_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* len, int32_t capacity, int32_t batch, float sm_scale, void* workspace,
                                size_t workspace_bytes, float* out, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (capacity <= 0 || capacity % 64 != 0) return fail(OSCAR_ERR_INVALID_ARG, "capacity %d not a positive multiple of 64", capacity);
  if (capacity / 64 > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "capacity %d > 64 * 65535", capacity);
  if (!q || !k || !v || !len || !workspace || !out) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const int splits = capacity / 64;
  const size_t need = oscar::partials_bytes(batch, desc->n_q_heads, splits);
  if (workspace_bytes < need) return fail(OSCAR_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  oscar::LayerShape L = shape_of(desc);
  L.window = capacity;  // the window pass's buffer layout, over the whole dense context
  const oscar::PartialsView pv = oscar::partials_view(workspace, batch, desc->n_q_heads, splits);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(oscar::launch_decode_bf16(L, q, k, v, len, batch, sm_scale, splits, pv, s), "dense pass launch");
  if (st != OSCAR_OK) return st;
  // no INT2 partials: the merge reduces the dense splits and normalises
  return hip_status(oscar::launch_merge(L, pv, 0, pv, splits, nullptr, out, batch, s), "dense merge launch");
}

size_t oscar_decode_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits) {
  if (check_desc_grouped(desc) != OSCAR_OK || batch < 0 || n_splits < 0) return 0;
  return oscar::step_workspace_bytes(batch, desc->n_q_heads, desc->n_kv_heads, n_splits, window_splits_of(desc));
}

}  // extern "C"

namespace {

// Checks shared by the two halves of the decode step; fills the workspace views. With nqt
// query tokens per request the heads are virtual (token, head) pairs: nqt n_q of them.
int32_t check_step_common(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits, void* workspace,
                          size_t workspace_bytes, oscar::StepArgs& a, int nqt = 1, bool grouped = false) {
  int32_t st = grouped ? check_desc_grouped(desc) : check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (n_splits <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_splits %d <= 0", n_splits);
  if (n_splits > 256) return fail(OSCAR_ERR_UNSUPPORTED, "n_splits %d > 256 (the two-launch decode)", n_splits);
  if (!workspace) return fail(OSCAR_ERR_INVALID_ARG, "null workspace");
  const int ws = window_splits_of(desc);
  const int n_qv = desc->n_q_heads * nqt;
  // the documented size: oscar_decode_workspace_bytes of batch x nqt requests (the same
  // partials as batch requests of nqt x n_q virtual heads, and more counter lines)
  const size_t need = oscar::step_workspace_bytes(batch * nqt, desc->n_q_heads, desc->n_kv_heads, n_splits, ws);
  if (workspace_bytes < need) return fail(OSCAR_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  const oscar::LayerShape L = shape_of(desc);
  char* base = static_cast<char*>(workspace);
  const size_t hist_bytes = (oscar::partials_bytes(batch, n_qv, n_splits) + 255) / 256 * 256;
  const size_t win_bytes = (oscar::partials_bytes(batch, n_qv, ws) + 255) / 256 * 256;
  a = oscar::StepArgs{};
  a.batch = batch;
  a.n_q = n_qv;
  a.n_kv = L.n_kv;
  a.gq = L.gq * nqt;
  a.nqt = nqt;
  a.window = L.window;
  a.n_splits = n_splits;
  a.n_wsplits = ws;
  a.n_groups = 1;
  a.n_qgroups = 128 / desc->group_size;
  a.hist = oscar::partials_view(base, batch, n_qv, n_splits);
  a.win = oscar::partials_view(base + hist_bytes, batch, n_qv, ws);
  a.counters = reinterpret_cast<int*>(base + hist_bytes + win_bytes);
  return OSCAR_OK;
}

int32_t prepare_impl(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                     const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k, const float* clip_v,
                     const void* q, const void* rot_k, const void* rot_v, const uint32_t* codebook, void* pool,
                     const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale,
                     int32_t n_splits, void* workspace, size_t workspace_bytes, void* stream, bool grouped = false) {
  oscar::StepArgs a;
  int32_t st = check_step_common(desc, batch, n_splits, workspace, workspace_bytes, a, 1, grouped);
  if (st != OSCAR_OK) return st;
  if (n < 0) return fail(OSCAR_ERR_INVALID_ARG, "n %d < 0", n);
  if (n > 0 && (!k_src || !v_src || !dst_page || !dst_slot || !clip_k || !clip_v || !rot_v || !pool))
    return fail(OSCAR_ERR_INVALID_ARG, "null demotion argument");
  if (!q || !rot_k || !k_win || !v_win || !win_len) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const long long grid = 2LL * n * desc->n_kv_heads +
                         static_cast<long long>(window_splits_of(desc)) * desc->n_kv_heads * batch +
                         static_cast<long long>(desc->n_q_heads) * batch;
  if (grid > 0x7FFFFFFFLL) return fail(OSCAR_ERR_UNSUPPORTED, "demotion rows exceed the grid limit");
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.n_dem_items = 2 * n * desc->n_kv_heads;
  a.dst_page = dst_page;
  a.dst_slot = dst_slot;
  a.clip_k = clip_k;
  a.clip_v = clip_v;
  a.pool = static_cast<uint8_t*>(pool);
  a.q = static_cast<const uint16_t*>(q);
  a.rot_k = static_cast<const uint16_t*>(rot_k);
  a.rot_v = static_cast<const uint16_t*>(rot_v);
  a.k_win = static_cast<const uint16_t*>(k_win);
  a.v_win = static_cast<const uint16_t*>(v_win);
  a.win_len = win_len;
  a.scale_log2 = static_cast<double>(sm_scale) * 1.4426950408889634;
  a.codebook = codebook;
  return hip_status(oscar::launch_prepare(a, static_cast<hipStream_t>(stream)), "prepare launch");
}

int32_t attend_impl(const oscar_layer_desc* desc, const void* rot_v, const uint32_t* codebook, const void* pool,
                    const int32_t* block_table, int32_t max_pages, const int32_t* hist_len, int32_t batch,
                    int32_t n_splits, void* workspace, size_t workspace_bytes, float* out, void* stream,
                    bool grouped = false) {
  oscar::StepArgs a;
  int32_t st = check_step_common(desc, batch, n_splits, workspace, workspace_bytes, a, 1, grouped);
  if (st != OSCAR_OK) return st;
  if (int32_t e = check_pages(max_pages, n_splits)) return e;
  if (!rot_v || !pool || !block_table || !hist_len || !out) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  a.rot_v = static_cast<const uint16_t*>(rot_v);
  a.pool = static_cast<uint8_t*>(const_cast<void*>(pool));  // only read by the attend launch
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.hist_len = hist_len;
  a.out = out;
  a.codebook = codebook;
  return hip_status(oscar::launch_attend(a, static_cast<hipStream_t>(stream)), "attend launch");
}

int32_t step_impl(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                  const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k, const float* clip_v,
                  const void* q, const void* rot_k, const void* rot_v, const uint32_t* codebook, void* pool,
                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len, const void* k_win,
                  const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                  void* workspace, size_t workspace_bytes, float* out, void* stream, bool grouped = false) {
  // the attend half's arguments are checked before anything is enqueued
  oscar::StepArgs a;
  int32_t st = check_step_common(desc, batch, n_splits, workspace, workspace_bytes, a, 1, grouped);
  if (st != OSCAR_OK) return st;
  if (int32_t e = check_pages(max_pages, n_splits)) return e;
  if (!rot_v || !pool || !block_table || !hist_len || !out) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  st = prepare_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, codebook, pool, k_win,
                    v_win, win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, stream, grouped);
  if (st != OSCAR_OK) return st;
  return attend_impl(desc, rot_v, codebook, pool, block_table, max_pages, hist_len, batch, n_splits, workspace,
                     workspace_bytes, out, stream, grouped);
}

}  // namespace

extern "C" {

int32_t oscar_prepare(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                      const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k, const float* clip_v,
                      const void* q, const void* rot_k, const void* rot_v, void* pool, const void* k_win,
                      const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return prepare_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, nullptr, pool, k_win,
                      v_win, win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, stream);
}

int32_t oscar_attend(const oscar_layer_desc* desc, const void* rot_v, const void* pool, const int32_t* block_table,
                     int32_t max_pages, const int32_t* hist_len, int32_t batch, int32_t n_splits, void* workspace,
                     size_t workspace_bytes, float* out, void* stream) {
  return attend_impl(desc, rot_v, nullptr, pool, block_table, max_pages, hist_len, batch, n_splits, workspace,
                     workspace_bytes, out, stream);
}

int32_t oscar_decode_step(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                          const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k, const float* clip_v,
                          const void* q, const void* rot_k, const void* rot_v, void* pool,
                          const int32_t* block_table, int32_t max_pages, const int32_t* hist_len, const void* k_win,
                          const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale,
                          int32_t n_splits, void* workspace, size_t workspace_bytes, float* out, void* stream) {
  return step_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, nullptr, pool,
                   block_table, max_pages, hist_len, k_win, v_win, win_len, batch, sm_scale, n_splits, workspace,
                   workspace_bytes, out, stream);
}

int32_t oscar_decode(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* rot_v,
                     const void* pool, const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                     const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale,
                     int32_t n_splits, void* workspace, size_t workspace_bytes, float* out, void* stream) {
  // nothing is demoted, so the pool is only read
  return step_impl(desc, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, q, rot_k, rot_v, nullptr,
                   const_cast<void*>(pool), block_table, max_pages, hist_len, k_win, v_win, win_len, batch, sm_scale,
                   n_splits, workspace, workspace_bytes, out, stream);
}

int32_t oscar_prepare_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                               const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                               const float* clip_v, const void* q, const void* rot_k, const void* rot_v,
                               const uint8_t* codebook, void* pool, const void* k_win, const void* v_win,
                               const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return prepare_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v,
                      reinterpret_cast<const uint32_t*>(codebook), pool, k_win, v_win, win_len, batch, sm_scale,
                      n_splits, workspace, workspace_bytes, stream);
}

int32_t oscar_attend_codebook(const oscar_layer_desc* desc, const void* rot_v, const uint8_t* codebook,
                              const void* pool, const int32_t* block_table, int32_t max_pages,
                              const int32_t* hist_len, int32_t batch, int32_t n_splits, void* workspace,
                              size_t workspace_bytes, float* out, void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return attend_impl(desc, rot_v, reinterpret_cast<const uint32_t*>(codebook), pool, block_table, max_pages, hist_len,
                     batch, n_splits, workspace, workspace_bytes, out, stream);
}

int32_t oscar_decode_step_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                                   const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                                   const float* clip_v, const void* q, const void* rot_k, const void* rot_v,
                                   const uint8_t* codebook, void* pool, const int32_t* block_table,
                                   int32_t max_pages, const int32_t* hist_len, const void* k_win, const void* v_win,
                                   const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                                   void* workspace, size_t workspace_bytes, float* out, void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return step_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v,
                   reinterpret_cast<const uint32_t*>(codebook), pool, block_table, max_pages, hist_len, k_win, v_win,
                   win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, out, stream);
}

int32_t oscar_decode_codebook(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* rot_v,
                              const uint8_t* codebook, const void* pool, const int32_t* block_table,
                              int32_t max_pages, const int32_t* hist_len, const void* k_win, const void* v_win,
                              const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                              void* workspace, size_t workspace_bytes, float* out, void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return step_impl(desc, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, q, rot_k, rot_v,
                   reinterpret_cast<const uint32_t*>(codebook), const_cast<void*>(pool), block_table, max_pages,
                   hist_len, k_win, v_win, win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, out, stream);
}

}  // extern "C"

// ---- the decode step in one launch, each request appending one token --------------------
namespace {

int32_t step_append_impl(const oscar_layer_desc* desc, const void* k_src, const void* v_src, const float* clip_k,
                         const float* clip_v, const void* q, const void* rot_k, const void* rot_v,
                         const uint32_t* codebook, void* pool, const int32_t* block_table, int32_t max_pages,
                         const int32_t* hist_len, const void* k_win, const void* v_win, const int32_t* win_len,
                         int32_t batch, float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                         float* out, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (n_splits <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_splits %d <= 0", n_splits);
  if (n_splits > 255) return fail(OSCAR_ERR_UNSUPPORTED, "n_splits %d > 255 (the one-launch step)", n_splits);
  if (int32_t e = check_pages(max_pages, n_splits)) return e;
  const bool append = k_src != nullptr;
  if (append && (!v_src || !clip_k || !clip_v)) return fail(OSCAR_ERR_INVALID_ARG, "null demotion argument");
  if (!append && v_src) return fail(OSCAR_ERR_INVALID_ARG, "v_src without k_src");
  if (!q || !rot_k || !rot_v || !pool || !block_table || !hist_len || !k_win || !v_win || !win_len || !out)
    return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!workspace) return fail(OSCAR_ERR_INVALID_ARG, "null workspace");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const int ws = window_splits_of(desc);
  const int pstride = n_splits + (append ? 1 : 0);
  const size_t need = oscar::step_workspace_bytes(batch, desc->n_q_heads, desc->n_kv_heads, n_splits + 1, ws);
  if (workspace_bytes < need) return fail(OSCAR_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  const int gq = desc->n_q_heads / desc->n_kv_heads;
  const long long items = static_cast<long long>(ws + 1) * desc->n_kv_heads * batch +
                          static_cast<long long>(n_splits) * desc->n_kv_heads * (gq > 8 ? gq / 8 : 1) * batch;
  if (items > 0x7FFFFFFFLL) return fail(OSCAR_ERR_UNSUPPORTED, "grid of %lld workgroups too large", items);
  const oscar::LayerShape L = shape_of(desc);
  char* base = static_cast<char*>(workspace);
  const size_t hist_bytes = (oscar::partials_bytes(batch, L.n_q, n_splits + 1) + 255) / 256 * 256;
  const size_t win_bytes = (oscar::partials_bytes(batch, L.n_q, ws) + 255) / 256 * 256;
  oscar::StepArgs a{};
  a.batch = batch;
  a.n_q = L.n_q;
  a.n_kv = L.n_kv;
  a.gq = L.gq;
  a.nqt = 1;
  a.n_qgroups = 1;
  a.window = L.window;
  a.n_splits = n_splits;
  a.n_wsplits = ws;
  a.n_groups = 1;
  a.hist = oscar::partials_view(base, batch, L.n_q, pstride);
  a.win = oscar::partials_view(base + hist_bytes, batch, L.n_q, ws);
  a.counters = reinterpret_cast<int*>(base + hist_bytes + win_bytes);
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.append = append ? 1 : 0;
  a.clip_k = clip_k;
  a.clip_v = clip_v;
  a.pool = static_cast<uint8_t*>(pool);
  a.q = static_cast<const uint16_t*>(q);
  a.rot_k = static_cast<const uint16_t*>(rot_k);
  a.rot_v = static_cast<const uint16_t*>(rot_v);
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.hist_len = hist_len;
  a.k_win = static_cast<const uint16_t*>(k_win);
  a.v_win = static_cast<const uint16_t*>(v_win);
  a.win_len = win_len;
  a.scale_log2 = static_cast<double>(sm_scale) * 1.4426950408889634;
  a.out = out;
  a.codebook = codebook;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (oscar::step_append_one_launch(batch, L.n_kv, gq > 8 ? gq / 8 : 1, n_splits, ws))
    return hip_status(oscar::launch_step_append(a, hs), "one-launch step");
  // a larger grid: prepare (the appended tokens demoted to the slots hist_len - 1 gives,
  // the window pass, the query preparation), then attend over the whole history
  a.hist = oscar::partials_view(base, batch, L.n_q, n_splits);
  a.n_dem_items = append ? 2 * batch * L.n_kv : 0;
  st = hip_status(oscar::launch_prepare(a, hs), "prepare launch");
  if (st != OSCAR_OK) return st;
  return hip_status(oscar::launch_attend(a, hs), "attend launch");
}

}  // namespace

extern "C" {

size_t oscar_decode_step_append_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits) {
  if (check_desc_impl(desc) != OSCAR_OK || batch < 0 || n_splits < 0) return 0;
  return oscar::step_workspace_bytes(batch, desc->n_q_heads, desc->n_kv_heads, n_splits + 1, window_splits_of(desc));
}

constexpr long long kOneLaunchItems = 240;  // one-launch grid size the split count aims at

// The split count of a one-launch grid (step or multi-query decode) with gqt query rows per
// KV head: one launch when its window and appended-token items and at least half the
// compute units' worth of history splits fit one 8-wave workgroup per unit; otherwise the
// two-launch default. The grid stays at 240 items: measured at batch 1 with 8 KV heads,
// 24, 26, 27 and 28 splits (224 to 256 items) took 13.70, 13.08, 13.06 and 13.08 us per
// step at 32K tokens and 20.19, 19.88, 20.07 and 20.05 us at 100K.
static int32_t one_launch_splits(const oscar_layer_desc* desc, int32_t batch, int gqt, int32_t max_hist_len) {
  const long long pages = (static_cast<long long>(max_hist_len > 0 ? max_hist_len : 0) + 63) / 64;
  const long long groups = static_cast<long long>(batch) * desc->n_kv_heads * (gqt > 8 ? gqt / 8 : 1);
  // window items (two splits each) and appended-token items
  const long long n_win = static_cast<long long>(oscar::window_items(window_splits_of(desc)) + 1) * batch * desc->n_kv_heads;
  long long s = (kOneLaunchItems - n_win) / groups;
  const long long by_pages = (pages + 7) / 8;
  if (s < 1 || s * groups < 128) {
    const int d = oscar_default_splits(desc, batch, max_hist_len);
    return d > 255 ? 255 : d;
  }
  if (s > by_pages) s = by_pages;
  const long long need = (pages + kMaxSplitPages - 1) / kMaxSplitPages;
  if (s < need) s = need;
  if (s < 1) s = 1;
  if (s > 255) s = 255;
  return static_cast<int32_t>(s);
}

int32_t oscar_decode_step_append_launches(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits) {
  if (check_desc_impl(desc) != OSCAR_OK || batch <= 0 || n_splits <= 0) return 0;
  const int gq = desc->n_q_heads / desc->n_kv_heads;
  return oscar::step_append_one_launch(batch, desc->n_kv_heads, gq > 8 ? gq / 8 : 1, n_splits, window_splits_of(desc))
             ? 1
             : 2;
}

int32_t oscar_decode_step_append_splits(const oscar_layer_desc* desc, int32_t batch, int32_t max_hist_len) {
  if (check_desc_impl(desc) != OSCAR_OK || batch <= 0) return 1;
  return one_launch_splits(desc, batch, desc->n_q_heads / desc->n_kv_heads, max_hist_len);
}

int32_t oscar_decode_multi_splits(const oscar_layer_desc* desc, int32_t batch, int32_t n_tokens, int32_t max_hist_len) {
  if (check_desc_impl(desc) != OSCAR_OK || batch <= 0 || n_tokens <= 0) return 1;
  const long long gqt = static_cast<long long>(desc->n_q_heads / desc->n_kv_heads) * n_tokens;
  if (gqt > 16) return oscar_default_splits(desc, batch, max_hist_len);
  return one_launch_splits(desc, batch, static_cast<int>(gqt), max_hist_len);
}

int32_t oscar_decode_step_append(const oscar_layer_desc* desc, const void* k_src, const void* v_src,
                                 const float* clip_k, const float* clip_v, const void* q, const void* rot_k,
                                 const void* rot_v, void* pool, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* hist_len, const void* k_win, const void* v_win, const int32_t* win_len,
                                 int32_t batch, float sm_scale, int32_t n_splits, void* workspace,
                                 size_t workspace_bytes, float* out, void* stream) {
  return step_append_impl(desc, k_src, v_src, clip_k, clip_v, q, rot_k, rot_v, nullptr, pool, block_table, max_pages,
                          hist_len, k_win, v_win, win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, out,
                          stream);
}

int32_t oscar_decode_step_append_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src,
                                          const float* clip_k, const float* clip_v, const void* q, const void* rot_k,
                                          const void* rot_v, const uint8_t* codebook, void* pool,
                                          const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                          const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                          float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                                          float* out, void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return step_append_impl(desc, k_src, v_src, clip_k, clip_v, q, rot_k, rot_v,
                          reinterpret_cast<const uint32_t*>(codebook), pool, block_table, max_pages, hist_len, k_win,
                          v_win, win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, out, stream);
}

}  // extern "C"

// ---- the decode step without a caller workspace ----------------------------------------
//
// For callers that cannot allocate device memory (code under HIP graph capture, serving
// loops that forbid hipMalloc): the step's workspace (INT2 and window partials, query
// data, arrival counters) is this file-scope device array instead. Every GPU the library
// runs on holds its own copy until the process ends. Its address on the current device is
// taken once, with hipGetSymbolAddress, and kept per device: in host code the array's name
// is not a device address.
namespace {

constexpr size_t kStaticScratchBytes = static_cast<size_t>(16) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the current device (looked up on the first call there).
int32_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(OSCAR_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(OSCAR_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OSCAR_OK;
}

}  // namespace

extern "C" {

size_t oscar_decode_step_noalloc_max_bytes(void) { return kStaticScratchBytes; }

int32_t oscar_decode_step_noalloc(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                                  const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                                  const float* clip_v, const void* q, const void* rot_k, const void* rot_v, void* pool,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                  const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                  float sm_scale, int32_t n_splits, float* out, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (n_splits <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_splits %d <= 0", n_splits);
  if (batch > 65535 || n_splits > 256)
    return fail(OSCAR_ERR_UNSUPPORTED, "batch %d or n_splits %d out of range", batch, n_splits);
  const size_t need = oscar::step_workspace_bytes(batch, desc->n_q_heads, desc->n_kv_heads, n_splits,
                                                  window_splits_of(desc));
  if (need > kStaticScratchBytes)
    return fail(OSCAR_ERR_WORKSPACE, "step needs %zu bytes of workspace; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != OSCAR_OK) return st;
  return step_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, nullptr, pool,
                   block_table, max_pages, hist_len, k_win, v_win, win_len, batch, sm_scale, n_splits, ws,
                   kStaticScratchBytes, out, stream);
}

}  // extern "C"

namespace {

int32_t multi_impl(const oscar_layer_desc* desc, const void* q, int32_t n_tokens, const void* rot_k,
                   const void* rot_v, const uint32_t* codebook, const void* pool, const int32_t* block_table,
                   int32_t max_pages, const int32_t* hist_len, const void* k_win, const void* v_win,
                   const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits, void* workspace,
                   size_t workspace_bytes, float* out, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (n_tokens <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_tokens %d <= 0", n_tokens);
  const int gq = desc->n_q_heads / desc->n_kv_heads;
  if ((n_tokens & (n_tokens - 1)) != 0 || static_cast<long long>(gq) * n_tokens > 16)
    return fail(OSCAR_ERR_UNSUPPORTED, "n_tokens %d: a power of two with n_tokens x %d query heads per KV head <= 16",
                n_tokens, gq);
  if (static_cast<long long>(batch) * n_tokens > 65535)
    return fail(OSCAR_ERR_UNSUPPORTED, "batch x n_tokens %lld > 65535", static_cast<long long>(batch) * n_tokens);
  oscar::StepArgs a;
  st = check_step_common(desc, batch, n_splits, workspace, workspace_bytes, a, n_tokens);
  if (st != OSCAR_OK) return st;
  if (int32_t e = check_pages(max_pages, n_splits)) return e;
  if (!q || !rot_k || !rot_v || !pool || !block_table || !hist_len || !k_win || !v_win || !win_len || !out)
    return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  a.q = static_cast<const uint16_t*>(q);
  a.rot_k = static_cast<const uint16_t*>(rot_k);
  a.rot_v = static_cast<const uint16_t*>(rot_v);
  a.pool = static_cast<uint8_t*>(const_cast<void*>(pool));  // only read: nothing is demoted
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.hist_len = hist_len;
  a.k_win = static_cast<const uint16_t*>(k_win);
  a.v_win = static_cast<const uint16_t*>(v_win);
  a.win_len = win_len;
  a.scale_log2 = static_cast<double>(sm_scale) * 1.4426950408889634;
  a.out = out;
  a.codebook = codebook;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int gqt = gq * n_tokens;
  if (oscar::step_append_one_launch(batch, desc->n_kv_heads, gqt > 8 ? gqt / 8 : 1, n_splits, window_splits_of(desc))) {
    // one launch: window items and INT2 splits that rotate the query rows themselves; the
    // arrival counters are zero from the workspace's fill or the previous call
    a.append = 0;
    return hip_status(oscar::launch_step_append(a, s), "one-launch multi-query decode");
  }
  st = hip_status(oscar::launch_prepare(a, s), "prepare launch");
  if (st != OSCAR_OK) return st;
  return hip_status(oscar::launch_attend(a, s), "attend launch");
}

}  // namespace

extern "C" {

int32_t oscar_decode_multi(const oscar_layer_desc* desc, const void* q, int32_t n_tokens, const void* rot_k,
                           const void* rot_v, const void* pool, const int32_t* block_table, int32_t max_pages,
                           const int32_t* hist_len, const void* k_win, const void* v_win, const int32_t* win_len,
                           int32_t batch, float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                           float* out, void* stream) {
  return multi_impl(desc, q, n_tokens, rot_k, rot_v, nullptr, pool, block_table, max_pages, hist_len, k_win, v_win,
                    win_len, batch, sm_scale, n_splits, workspace, workspace_bytes, out, stream);
}

int32_t oscar_decode_multi_codebook(const oscar_layer_desc* desc, const void* q, int32_t n_tokens, const void* rot_k,
                                    const void* rot_v, const uint8_t* codebook, const void* pool,
                                    const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                    const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                    float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                                    float* out, void* stream) {
  if (int32_t e = check_codebook(codebook)) return e;
  return multi_impl(desc, q, n_tokens, rot_k, rot_v, reinterpret_cast<const uint32_t*>(codebook), pool, block_table,
                    max_pages, hist_len, k_win, v_win, win_len, batch, sm_scale, n_splits, workspace,
                    workspace_bytes, out, stream);
}

}  // extern "C"

namespace oscar {
size_t calib_workspace_bytes(int T, int n_q, int n_kv);  // calib.hip
}

extern "C" {

size_t oscar_calib_workspace_bytes(const oscar_layer_desc* desc, int32_t n_tokens) {
  if (check_desc_impl(desc) != OSCAR_OK || n_tokens < 0) return 0;
  return oscar::calib_workspace_bytes(n_tokens, desc->n_q_heads, desc->n_kv_heads);
}

int32_t oscar_calib_covariances(const oscar_layer_desc* desc, const void* q, const void* k, const void* v,
                                int32_t n_tokens, float sm_scale, void* workspace, size_t workspace_bytes,
                                float* sigma_k, float* sigma_v, void* stream) {
  int32_t st = check_desc_impl(desc);
  if (st != OSCAR_OK) return st;
  if (n_tokens <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_tokens %d <= 0", n_tokens);
  if (n_tokens > 65536) return fail(OSCAR_ERR_UNSUPPORTED, "n_tokens %d > 65536", n_tokens);
  if (!q || !k || !v || !workspace || !sigma_k || !sigma_v) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const size_t need = oscar_calib_workspace_bytes(desc, n_tokens);
  if (workspace_bytes < need) return fail(OSCAR_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(k) % 16 ||
      reinterpret_cast<uintptr_t>(v) % 16 || reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(OSCAR_ERR_INVALID_ARG, "q, k, v and workspace must be 16-byte aligned");
  return hip_status(oscar::launch_calib(shape_of(desc), q, k, v, n_tokens, sm_scale, static_cast<float*>(workspace),
                                        sigma_k, sigma_v, static_cast<hipStream_t>(stream)),
                    "calibration launch");
}

int32_t oscar_read_probe_words(void) { return oscar::read_probe_blocks(); }

int32_t oscar_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(OSCAR_ERR_INVALID_ARG, "buf and bytes must be multiples of 16");
  return hip_status(oscar::launch_read_probe(buf, bytes, out, static_cast<hipStream_t>(stream)), "probe launch");
}

int32_t oscar_merge(const oscar_layer_desc* desc, const void* partials, int32_t n_splits, const void* win_partials,
                    const void* rot_v, float* out, int32_t batch, void* stream) {
  int32_t st = check_desc_grouped(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (n_splits <= 0 || n_splits > 65535) return fail(OSCAR_ERR_INVALID_ARG, "n_splits %d out of [1, 65535]", n_splits);
  if (!partials || !win_partials || !rot_v || !out) return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  const oscar::LayerShape L = shape_of(desc);
  const int ws = window_splits_of(desc);
  // the const casts only build read views; merge never writes a workspace
  const oscar::PartialsView h = oscar::partials_view(const_cast<void*>(partials), batch, desc->n_q_heads, n_splits);
  const oscar::PartialsView w = oscar::partials_view(const_cast<void*>(win_partials), batch, desc->n_q_heads, ws);
  return hip_status(oscar::launch_merge(L, h, n_splits, w, ws, rot_v, out, batch, static_cast<hipStream_t>(stream)),
                    "merge launch");
}

int32_t oscar_demote_grouped(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                             const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                             const float* clip_k, const float* clip_v, void* pool, void* stream) {
  int32_t st = check_desc_grouped(desc);
  if (st != OSCAR_OK) return st;
  if (n < 0) return fail(OSCAR_ERR_INVALID_ARG, "n %d < 0", n);
  if (n == 0) return ok();
  if (!k_src || !v_src || !dst_page || !dst_slot || !rot_k || !rot_v || !clip_k || !clip_v || !pool)
    return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (2LL * n * desc->n_kv_heads > 0x7FFFFFFFLL)
    return fail(OSCAR_ERR_UNSUPPORTED, "2 * n * n_kv_heads exceeds the grid limit");
  return hip_status(oscar::launch_demote_grouped(desc->n_kv_heads, desc->group_size, k_src, v_src, n, dst_page,
                                                 dst_slot, rot_k, rot_v, clip_k, clip_v, pool,
                                                 static_cast<hipStream_t>(stream)),
                    "grouped demote launch");
}

int32_t oscar_decode_int2_grouped(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* pool,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                  int32_t batch, float sm_scale, int32_t n_splits, void* partials,
                                  size_t partials_bytes, void* stream) {
  int32_t st = check_desc_grouped(desc);
  if (st != OSCAR_OK) return st;
  if (batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (n_splits <= 0 || n_splits > 65535) return fail(OSCAR_ERR_INVALID_ARG, "n_splits %d out of [1, 65535]", n_splits);
  if (max_pages <= 0) return fail(OSCAR_ERR_INVALID_ARG, "max_pages %d <= 0", max_pages);
  if (!q || !rot_k || !pool || !block_table || !hist_len || !partials)
    return fail(OSCAR_ERR_INVALID_ARG, "null pointer argument");
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(rot_k) % 16 != 0)
    return fail(OSCAR_ERR_INVALID_ARG, "q and rot_k must be 16-byte aligned");
  if (int32_t e = check_pages(max_pages, n_splits)) return e;
  const size_t need = oscar::partials_bytes(batch, desc->n_q_heads, n_splits);
  if (partials_bytes < need)
    return fail(OSCAR_ERR_WORKSPACE, "partials workspace %zu < %zu bytes", partials_bytes, need);
  const oscar::LayerShape L = shape_of(desc);
  const oscar::PartialsView v = oscar::partials_view(partials, batch, desc->n_q_heads, n_splits);
  return hip_status(oscar::launch_decode_grouped(L, desc->group_size, q, rot_k, pool, block_table, max_pages, hist_len,
                                                 batch, sm_scale, n_splits, v, static_cast<hipStream_t>(stream)),
                    "grouped decode launch");
}


int32_t oscar_decode_step_grouped(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                                  const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                                  const float* clip_v, const void* q, const void* rot_k, const void* rot_v, void* pool,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                  const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                  float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes, float* out,
                                  void* stream) {
  return step_impl(desc, k_src, v_src, n, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, nullptr, pool,
                   block_table, max_pages, hist_len, k_win, v_win, win_len, batch, sm_scale, n_splits, workspace,
                   workspace_bytes, out, stream, true);
}

}  // extern "C"
