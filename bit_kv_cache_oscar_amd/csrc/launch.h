// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oscar {

struct LayerShape {
  int n_q;       // query heads
  int n_kv;      // KV heads
  int gq;        // query heads per KV head
  int window;    // BF16 window slots per request and KV head
};

// Memory row of virtual query head hv of request b. With nqt query tokens per request (a
// multi-query decode), KV head kv has nqt * gq virtual heads, (token t, head g) in
// token-major order, while q and out hold [batch][nqt][n_q][128] with n_q = n_qv / nqt;
// with one token the two numberings coincide.
__host__ __device__ inline size_t query_row(int b, int hv, int n_qv, int gqv, int nqt) {
  if (nqt == 1) return static_cast<size_t>(b) * n_qv + hv;
  const int gq = gqv / nqt;
  const int kv = hv / gqv;
  const int r = hv - kv * gqv;
  const int t = r / gq;
  return (static_cast<size_t>(b) * nqt + t) * (n_qv / nqt) + static_cast<size_t>(kv) * gq + (r - t * gq);
}

// Query token of virtual head hv (0 for a single-token decode).
__host__ __device__ inline int query_token(int hv, int gqv, int nqt) { return (hv % gqv) / (gqv / nqt); }

// Per (request, query head) scalars of the rotated query, written by the INT2 pass's
// query preparation: the score scale 2^-sh sm_scale log2(e), sm_scale log2(e) sum(q_rot)
// and the centring term -2 sum(Q) of the fixed-point query Q.
struct QueryScal {
  float qsc;
  float sig;
  int32_t kcent;
  int32_t pad[5];
};
static_assert(sizeof(QueryScal) == 32, "QueryScal is 32 bytes");

// Views of the m, l and acc arrays of a partial-result workspace.
struct PartialsView {
  float* m;
  float* l;
  float* acc;
  char* qlimb;        // INT2 pass only: fixed-point limbs of the rotated query [B][Hq][4][128]
  QueryScal* qscal;   // INT2 pass only: [B][Hq]
};

size_t partials_bytes(int batch, int n_q, int n_splits);
PartialsView partials_view(void* base, int batch, int n_q, int n_splits);
// Ints between two arrival counters: each (request, KV head) counter has a 256-byte line of
// its own. Packed, the counters share one line that every workgroup of the launch updates
// with an agent-scope atomic: measured at 32K tokens, batch 1, 8 KV heads, the one-launch
// step took 14.36 us per step with packed counters and 13.09 us with a line each.
constexpr int kCounterStride = 64;
size_t step_workspace_bytes(int batch, int n_q, int n_kv, int n_splits, int n_wsplits);

// `codebook`: null for the uniform levels, else the codebook words [n_kv][K, V]
hipError_t launch_demote_rows(const LayerShape& L, const void* k_src, const void* v_src, int n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k,
                              const void* rot_v, const float* clip_k, const float* clip_v, void* pool,
                              hipStream_t stream, const uint32_t* codebook = nullptr);
hipError_t launch_demote_bulk(const LayerShape& L, const void* k_src, const void* v_src, int n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k,
                              const void* rot_v, const float* clip_k, const float* clip_v, void* pool,
                              hipStream_t stream, const uint32_t* codebook = nullptr);

// `group`: rotated dims per quantisation group (128, or 64 and 32 for grouped pages)
hipError_t launch_decode_int2(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                              const int32_t* block_table, int max_pages, const int32_t* hist_len,
                              int batch, float sm_scale, int n_splits, const PartialsView& out,
                              hipStream_t stream, int group = 128);

hipError_t launch_decode_bf16(const LayerShape& L, const void* q, const void* k_win, const void* v_win,
                              const int32_t* win_len, int batch, float sm_scale, int n_win_splits,
                              const PartialsView& out, hipStream_t stream);

// Everything the fused decode step needs (passed to its kernels by value).
struct StepArgs {
  // demotion (n_dem_items = 2 * tokens * n_kv; 0 for decode only)
  const uint16_t* k_src;
  const uint16_t* v_src;
  int n_dem_items;
  const int32_t* dst_page;
  const int32_t* dst_slot;
  const float* clip_k;
  const float* clip_v;
  uint8_t* pool;
  // decode
  const uint16_t* q;
  const uint16_t* rot_k;
  const uint16_t* rot_v;
  const int32_t* block_table;
  int max_pages;
  const int32_t* hist_len;
  const uint16_t* k_win;
  const uint16_t* v_win;
  const int32_t* win_len;
  int batch, n_q, n_kv, gq, window, n_splits, n_wsplits, n_groups;
  int win_groups;  // workgroups per (window split, KV head, request), each for gq / win_groups heads
  int nqt;         // query tokens per request; n_q and gq count virtual heads (token, head)
  int n_qgroups = 1;  // quantisation groups per vector of the pool's pages: 1, 2 or 4
  double scale_log2;
  PartialsView hist;  // INT2 partials and the query tail
  PartialsView win;   // window partials
  int* counters;      // [batch][n_kv] arrival counters, kCounterStride ints apart
  float* out;
  // Lloyd-Max codebook variant: words [n_kv][K, V], byte c = level c in sixteenths of the
  // scale; null for the uniform INT2 levels
  const uint32_t* codebook;
  // one-launch step: 1 when token b of k_src / v_src is appended to request b's history
  // (history token hist_len[b] - 1), 0 for no demotion
  int append;
};

// Demotion + window pass + query preparation (one launch), and the INT2 pass with the merge
// done by the last workgroup of each (request, KV head) (one launch).
hipError_t launch_prepare(StepArgs a, hipStream_t stream);
hipError_t launch_attend(StepArgs a, hipStream_t stream);

// The decode step in one launch: window items, appended-token items (each request's
// appended token demoted, its term written as INT2 partial column n_splits), then INT2
// splits with the query prepared inline; the last arrival per (request, KV head) merges.
// `hist` views n_splits + append columns; the counters must be zero at the start and are
// left at zero. hipErrorInvalidValue if the grid does not fit step_append_one_launch.
hipError_t launch_step_append(StepArgs a, hipStream_t stream);
// Window workgroups of the one-launch grid per (request, KV head): each runs two of the
// window's 64-slot splits, one per half of its 8 waves.
__host__ __device__ inline int window_items(int n_wsplits) { return (n_wsplits + 1) / 2; }
// whether the one-launch grid runs in a single dispatch round of 8-wave workgroups (else the
// step is better run as prepare + attend)
bool step_append_one_launch(int batch, int n_kv, int n_groups, int n_splits, int n_wsplits);

// Calibration covariances: Sigma_K and Sigma_V [n_kv][128][128] fp32 of one calibration
// sequence of T tokens (q [T][n_q][128], k and v [T][n_kv][128] bf16); o_work holds
// T n_q 128 floats (the attention outputs).
hipError_t launch_calib(const LayerShape& L, const void* q, const void* k, const void* v, int T, float sm_scale,
                        float* o_work, float* sigma_k, float* sigma_v, hipStream_t stream);

// Read-bandwidth probe: reads bytes / 16 16-byte words of buf, writes read_probe_blocks()
// words to out.
int read_probe_blocks();
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

hipError_t launch_merge(const LayerShape& L, const PartialsView& hist, int n_splits,
                        const PartialsView& win, int n_win_splits, const void* rot_v, float* out,
                        int batch, hipStream_t stream);

}  // namespace oscar
