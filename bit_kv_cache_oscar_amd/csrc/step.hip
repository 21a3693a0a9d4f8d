// Decode step in two launches: oscar_prepare, then oscar_attend (oscar_decode_step and
// oscar_decode issue both).
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: a decode step demotes the
// oldest recent token into the INT2 history (rotate, clip, quantise, pack), then attends
// over the BF16 sink/recent segment and the INT2 history separately and joins the two by
// an online-softmax merge.
//
// Launch 1 (prep), one 256-thread workgroup per item, the items being independent:
//   demotion rows (token, KV head, K or V); BF16 window splits (split, KV head, request,
//   and for a small pass a group of the KV head's query heads);
//   query preparation per (request, query head), which also zeroes the request's
//   per-KV-head arrival counters.
// Launch 2 (main), grid (history split, KV head x head group, request): the INT2 pass of
// the split, then a ticket: every workgroup writes its partial with agent-scope stores,
// waits for them to complete and adds one to its (request, KV head) counter; the workgroup
// that draws the last ticket merges all INT2 and window partials of that KV head's query
// heads and writes the output, after re-arming the counter (so the main launch may be
// repeated on its own). The INT2 value sums are un-rotated (times R_V^T) by each split
// before it writes them when the grid has one 8-wave workgroup per compute unit at most,
// else by the merge. No workgroup ever waits for another.

#include "demote_pass.h"
#include "grouped_pass.h"
#include "int2_pass.h"
#include "merge_pass.h"
#include "window_pass.h"

namespace oscar {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// NG: quantisation groups per vector of the pool's pages (the demotion rows' format)
template <int GQW, int NG>
__global__ __launch_bounds__(256) void prep_kernel(StepArgs a) {
  __shared__ __align__(16) unsigned char smem[cmax(cmax(cmax(demote::kSmemBytes, demote::kGroupedSmemBytes),
                                                        window::window_smem_bytes<GQW>()),
                                                   int2::kQprepSmem)];
  int id = blockIdx.x;
  if (id < a.n_dem_items) {
    if constexpr (NG == 1)
      demote::demote_row(smem, id, a.k_src, a.v_src, a.n_kv, a.append ? nullptr : a.dst_page, a.dst_slot, a.rot_k,
                         a.rot_v, a.clip_k, a.clip_v, a.pool, a.codebook, a.block_table, a.max_pages, a.hist_len);
    else
      demote::demote_grouped_row<NG>(smem, id, a.k_src, a.v_src, a.n_kv, a.dst_page, a.dst_slot, a.rot_k, a.rot_v,
                                     a.clip_k, a.clip_v, a.pool);
    return;
  }
  id -= a.n_dem_items;
  const int n_win = a.n_wsplits * a.n_kv * a.batch * a.win_groups;
  if (id < n_win) {
    // the head group varies slowest: the groups of one split are n_win / win_groups apart,
    // a multiple of 8 for the workloads that split (5 splits x 8 KV heads), so they run on
    // one XCD and the K and V rows the first reads come from that XCD's L2 for the others
    const int base = n_win / a.win_groups;
    const int grp = id / base;
    const int rest = id - grp * base;
    const int c = rest % a.n_wsplits;
    const int kv = (rest / a.n_wsplits) % a.n_kv;
    const int b = rest / (a.n_wsplits * a.n_kv);
    // win_groups is 1, 2 or 4 and divides GQW (the launch chose it)
    if (a.win_groups == 1) {
      window::window_split<GQW>(smem, c, kv, kv * GQW, b, a.q, a.k_win, a.v_win, a.win_len, a.n_q, a.n_kv, a.window,
                                a.n_wsplits, a.scale_log2, a.win.m, a.win.l, a.win.acc, GQW, a.nqt);
    } else if (a.win_groups == 2) {
      if constexpr (GQW % 2 == 0)
        window::window_split<GQW / 2>(smem, c, kv, kv * GQW + grp * (GQW / 2), b, a.q, a.k_win, a.v_win, a.win_len,
                                      a.n_q, a.n_kv, a.window, a.n_wsplits, a.scale_log2, a.win.m, a.win.l, a.win.acc,
                                      GQW, a.nqt);
    } else {
      if constexpr (GQW % 4 == 0)
        window::window_split<GQW / 4>(smem, c, kv, kv * GQW + grp * (GQW / 4), b, a.q, a.k_win, a.v_win, a.win_len,
                                      a.n_q, a.n_kv, a.window, a.n_wsplits, a.scale_log2, a.win.m, a.win.l, a.win.acc,
                                      GQW, a.nqt);
    }
    return;
  }
  id -= n_win;
  const int h = id % a.n_q;
  const int b = id / a.n_q;
  if (threadIdx.x == 0 && h % a.gq == 0) a.counters[(b * a.n_kv + h / a.gq) * kCounterStride] = 0;
  int2::qprep_head(smem, a.q, a.rot_k, a.n_q, a.gq, a.scale_log2, a.hist.qlimb, a.hist.qscal, h, b, a.nqt,
                   a.codebook);
}

// GQ query heads per workgroup, GQT per KV head (GQT = GQ n_groups), NW waves; CB: the
// codebook variant; NG quantisation groups per vector
template <int GQ, int GQT, int NW, bool CB, int NG = 1>
__global__ __launch_bounds__(64 * NW) void main_kernel(StepArgs a) {
  // the INT2 pass and the merge use the same LDS one after the other
  __shared__ __align__(16) unsigned char smem[cmax(int2::int2_smem_bytes<GQ, NW, NG>(), merge::smem_bytes<GQT, NW>())];
  __shared__ int ticket_s;
  // 8-wave workgroups (a grid of at most one per compute unit) un-rotate their own value
  // sums, so the merge after the last ticket is a weighted sum; 4-wave ones, several to a
  // compute unit, leave that to the merge and keep the R_V fragments out of the page loop
  constexpr bool kUnrot = NW == 8;
  int2::int2_split<GQ, true, NW, CB, kUnrot, NG>(smem, blockIdx.x, blockIdx.y, blockIdx.z, a.pool, a.block_table,
                                                 a.max_pages, a.hist_len, a.n_q, a.n_kv, a.n_groups, a.n_splits,
                                                 a.hist.qlimb, a.hist.qscal, a.hist.m, a.hist.l, a.hist.acc,
                                                 a.codebook, int2::InlineQuery(), a.rot_v);
  const int kv = blockIdx.y / a.n_groups;
  const int b = blockIdx.z;
  // the partials went out as agent-scope stores: once each thread's stores have completed
  // and the barrier has passed, the ticket below is drawn after all of them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* counter = a.counters + (b * a.n_kv + kv) * kCounterStride;
  if (threadIdx.x == 0) ticket_s = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket_s != a.n_splits * a.n_groups - 1) return;
  // last arrival for (b, kv): every workgroup of the group has drawn its ticket, so re-arm the
  // counter for the next launch; the group's partials are read with agent-scope loads
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // R_V fragments of the un-rotation (when the splits left it to the merge): requested
  // first, they travel with the partials' loads (one round trip)
  uint4 rb[8 / NW][4];
  if constexpr (!kUnrot) merge::load_rv<NW>(a.rot_v, kv, rb);
  merge::merge_group<GQT, NW, false, !kUnrot>(smem, b, kv, a.n_q, a.hist, a.n_splits, a.win, a.n_wsplits, rb, a.out,
                                               a.nqt);
}

// A small window pass (fewer than 256 workgroups) spreads each KV head's query heads over up
// to four workgroups: each then has a fraction of the value sums and stores, and the batch-1
// window pass, the longest item of the launch, ends sooner. The K and V rows it reads again
// come from L2.
template <int GQT, int NG>
hipError_t launch_prep(StepArgs a, hipStream_t stream) {
  const long long base = static_cast<long long>(a.n_wsplits) * a.n_kv * a.batch;
  a.win_groups = 1;
  while (a.win_groups < 4 && GQT % (2 * a.win_groups) == 0 && base * 2 * a.win_groups <= 256) a.win_groups *= 2;
  const unsigned n_prep =
      static_cast<unsigned>(a.n_dem_items + base * a.win_groups + static_cast<long long>(a.n_q) * a.batch);
  hipLaunchKernelGGL((prep_kernel<GQT, NG>), dim3(n_prep), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Up to 256 workgroups (one per CU) run with 8 waves each, so few splits still give
// every SIMD two waves; larger grids use 4 waves per workgroup.
template <int GQ, int GQT, bool CB, int NG = 1>
hipError_t launch_main_cb(const StepArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_splits, a.n_kv * a.n_groups, a.batch);
  if (static_cast<long long>(grid.x) * grid.y * grid.z <= 256)
    hipLaunchKernelGGL((main_kernel<GQ, GQT, 8, CB, NG>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((main_kernel<GQ, GQT, 4, CB, NG>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int GQ, int GQT>
hipError_t launch_main(const StepArgs& a, hipStream_t stream) {
  return a.codebook ? launch_main_cb<GQ, GQT, true>(a, stream) : launch_main_cb<GQ, GQT, false>(a, stream);
}

// grouped pages: head tiles of four (the per-group metadata leaves no registers for two)
template <int NG>
hipError_t launch_main_grouped(StepArgs a, hipStream_t stream) {
  switch (a.gq) {
    case 1: a.n_groups = 1; return launch_main_cb<1, 1, false, NG>(a, stream);
    case 2: a.n_groups = 1; return launch_main_cb<2, 2, false, NG>(a, stream);
    case 4: a.n_groups = 1; return launch_main_cb<4, 4, false, NG>(a, stream);
    case 8: a.n_groups = 2; return launch_main_cb<4, 8, false, NG>(a, stream);
    case 16: a.n_groups = 4; return launch_main_cb<4, 16, false, NG>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int NG>
hipError_t launch_prep_ng(const StepArgs& a, hipStream_t stream) {
  switch (a.gq) {
    case 1: return launch_prep<1, NG>(a, stream);
    case 2: return launch_prep<2, NG>(a, stream);
    case 4: return launch_prep<4, NG>(a, stream);
    case 8: return launch_prep<8, NG>(a, stream);
    case 16: return launch_prep<16, NG>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// The one-launch step (and the one-launch multi-query decode: nqt query tokens per request
// as virtual heads, no appended token). Items 0 .. n_win - 1 are window splits (split c, KV head, request);
// when appending, the next B n_kv items each demote the appended token of one (KV head,
// request) and write its own attention term; the rest are INT2 splits (KV head, head group,
// split, request, the first fastest) with the query prepared inline and the appended token
// left out. Every
// item starts at once, writes its partials with agent-scope stores and draws a ticket; the
// last of a (request, KV head) merges.
template <int GQ, int GQT, int NW, bool CB>
__global__ __launch_bounds__(64 * NW) void append_kernel(StepArgs a) {
  constexpr int kSmem = cmax(cmax(int2::int2_smem_bytes<GQ, NW>(), merge::smem_bytes<GQT, NW>()),
                             cmax(2 * window::window_smem_bytes<GQT>(), demote::append_smem_bytes<GQT>()));
  __shared__ __align__(16) unsigned char smem[kSmem];
  __shared__ int ticket_s;
  // each window item runs two 64-slot splits, one per half of its waves
  const int n_witems = window_items(a.n_wsplits);
  const int n_win = n_witems * a.n_kv * a.batch;
  const int pstride = a.n_splits + a.append;
  int id = blockIdx.x;
  int kv, b;
  const int n_app = a.append ? a.n_kv * a.batch : 0;
  if (id < n_win) {
    const int c = 2 * (id % n_witems);
    kv = (id / n_witems) % a.n_kv;
    b = id / (n_witems * a.n_kv);
    window::window_split<GQT, NW, true, NW == 8>(smem, c, kv, kv * GQT, b, a.q, a.k_win, a.v_win, a.win_len, a.n_q,
                                                 a.n_kv, a.window, a.n_wsplits, a.scale_log2, a.win.m, a.win.l,
                                                 a.win.acc, GQT, a.nqt);
  } else if (id < n_win + n_app) {
    id -= n_win;
    kv = id % a.n_kv;
    b = id / a.n_kv;
    demote::append_token<NW, GQT, true>(smem, b, kv, a, a.n_splits, pstride);
  } else {
    // the KV head varies fastest: workgroups go to the 8 XCDs in turn, so with 8 KV heads
    // every INT2 item of a KV head (its splits and head groups) runs on one XCD, whose L2
    // then fetches the head's R_K and R_V once, and a page that two head groups read once
    id -= n_win + n_app;
    kv = id % a.n_kv;
    const int rest = id / a.n_kv;
    const int gy = kv * a.n_groups + rest % a.n_groups;
    const int split = (rest / a.n_groups) % a.n_splits;
    b = rest / (a.n_groups * a.n_splits);
    int2::InlineQuery iq;
    iq.q = a.q;
    iq.rot_k = a.rot_k;
    iq.scale_log2 = a.scale_log2;
    iq.n_excl = a.append;
    iq.pstride = pstride;
    iq.nqt = a.nqt;
    iq.gqv = GQT;
    int2::int2_split<GQ, true, NW, CB, true>(smem, split, gy, b, a.pool, a.block_table, a.max_pages, a.hist_len,
                                             a.n_q, a.n_kv, a.n_groups, a.n_splits, nullptr, nullptr, a.hist.m,
                                             a.hist.l, a.hist.acc, a.codebook, iq, a.rot_v);
  }
  // the partials went out as agent-scope stores: once each thread's stores have completed
  // and the barrier has passed, the ticket below is drawn after all of them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* counter = a.counters + (b * a.n_kv + kv) * kCounterStride;
  if (threadIdx.x == 0) ticket_s = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket_s != a.n_splits * a.n_groups + n_witems + a.append - 1) return;
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // every partial is in the window's basis (the INT2 splits and the appended token
  // un-rotated theirs): the merge is a weighted sum
  uint4 rb[8 / NW][4];
  merge::merge_group<GQT, NW, true, false>(smem, b, kv, a.n_q, a.hist, pstride, a.win, a.n_wsplits, rb, a.out,
                                           a.nqt);
}

constexpr int kStepSlots8 = 256;  // 8-wave workgroups resident at once (one per compute unit)

}  // namespace

bool step_append_one_launch(int batch, int n_kv, int n_groups, int n_splits, int n_wsplits) {
  return static_cast<long long>(window_items(n_wsplits) + 1) * n_kv * batch +
             static_cast<long long>(n_splits) * n_kv * n_groups * batch <=
         kStepSlots8;
}

namespace {

// one 8-wave workgroup per item; the grid must fit one dispatch round (the caller checks
// step_append_one_launch)
template <int GQ, int GQT, bool CB>
hipError_t launch_append_cb(const StepArgs& a, hipStream_t stream) {
  const long long items = static_cast<long long>(window_items(a.n_wsplits) + a.append) * a.n_kv * a.batch +
                          static_cast<long long>(a.n_splits) * a.n_kv * a.n_groups * a.batch;
  if (items > kStepSlots8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((append_kernel<GQ, GQT, 8, CB>), dim3(static_cast<unsigned>(items)), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int GQ, int GQT>
hipError_t launch_append(const StepArgs& a, hipStream_t stream) {
  return a.codebook ? launch_append_cb<GQ, GQT, true>(a, stream) : launch_append_cb<GQ, GQT, false>(a, stream);
}

}  // namespace

hipError_t launch_prepare(StepArgs a, hipStream_t stream) {
  switch (a.n_qgroups) {
    case 1: return launch_prep_ng<1>(a, stream);
    case 2: return launch_prep_ng<2>(a, stream);
    case 4: return launch_prep_ng<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attend(StepArgs a, hipStream_t stream) {
  if (a.n_qgroups == 2) return a.codebook ? hipErrorInvalidValue : launch_main_grouped<2>(a, stream);
  if (a.n_qgroups == 4) return a.codebook ? hipErrorInvalidValue : launch_main_grouped<4>(a, stream);
  if (a.n_qgroups != 1) return hipErrorInvalidValue;
  switch (a.gq) {
    case 1: a.n_groups = 1; return launch_main<1, 1>(a, stream);
    case 2: a.n_groups = 1; return launch_main<2, 2>(a, stream);
    case 4: a.n_groups = 1; return launch_main<4, 4>(a, stream);
    case 8: a.n_groups = 1; return launch_main<8, 8>(a, stream);
    case 16: a.n_groups = 2; return launch_main<8, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar

namespace oscar {

hipError_t launch_step_append(StepArgs a, hipStream_t stream) {
  switch (a.gq) {
    case 1: a.n_groups = 1; return launch_append<1, 1>(a, stream);
    case 2: a.n_groups = 1; return launch_append<2, 2>(a, stream);
    case 4: a.n_groups = 1; return launch_append<4, 4>(a, stream);
    case 8: a.n_groups = 1; return launch_append<8, 8>(a, stream);
    case 16: a.n_groups = 2; return launch_append<8, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
