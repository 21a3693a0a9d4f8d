// Demotion of recent-window tokens into the INT2 history (rotate, clip, quantise, pack):
// device code shared by the standalone demote kernel and the fused decode-step kernel.
//
// Method: OSCAR (Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
// Quantization); QbitAI article on OSCAR, serving-path section: the oldest recent token
// is rotated, clipped, quantised and packed four 2-bit codes per byte into the INT2
// history, with a scale and zero point per group.
//
// One workgroup of 256 threads handles one row (token, KV head, K or V). Every global
// read of the row (the token, the rotation, the destination and the clip ratio) is
// issued before any arithmetic. Wave w sums the terms 32w..32w+31 of the output dims
// 2 lane, 2 lane + 1 in fp64 (bf16 x bf16 products are exact there), with sum |p| beside
// each sum; wave 0 joins the four quarters and bounds the error of each dim by
// 2^-47 sum|p| (at most 36 roundings on any path of the fixed summation order). The
// group extremes, fp16 scale and zero point, and every code are then taken at both ends
// of these intervals: when both ends agree (all but a vanishing fraction of rows), the
// decisions equal those made from the exact dot products. Otherwise wave 0 recomputes
// the row's dot products with compensated (two-sum) fp64 sums and decides from those.
// The scale/zero arithmetic is fp64 exactly as specified. With a codebook (the Lloyd-Max
// variant, QbitAI article on OSCAR, comparison with TurboQuant) the scale and zero point
// are the same and each code is the nearest of the four codebook levels instead.

#pragma once

#include "device_common.h"
#include "merge_pass.h"
#include "launch.h"

namespace oscar {
namespace demote {

// quarter partials of waves 1..3: [3][64 lanes][s0, s1, a0, a1]
constexpr int kSmemBytes = 3 * 64 * 4 * 8;

// Fixed-order fp64 sum of 128 exact products: 32 terms per quarter chain, three joins,
// each sum rounded once, so |error| <= 36 (2^-53 + tiny) sum|p| < 2^-47 sum|p|; the
// remaining 28 2^-53 sum|p| covers the rounding of the interval ends themselves.
constexpr double kBound = 0x1p-47;

__device__ __forceinline__ void two_sum_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  c += (s - (t - bp)) + (p - bp);
  s = t;
}

struct ScaleZero {
  uint16_t s16, z16;
};

// fp16 scale and zero point of a group whose extremes are ymax, ymin (clip ratio cr)
__device__ __forceinline__ ScaleZero scale_zero(double cr, double ymax, double ymin) {
#pragma clang fp contract(off)
  const double hi = cr * ymax;
  const double lo = cr * ymin;
  return {f64_to_f16_rne((hi - lo) / 3.0), f64_to_f16_rne(lo)};
}

// 2-bit code of rotated value y from t = (y - z) / s: round half to even, clamped to
// [0, 3], for the uniform levels (lv == 0); the nearest level of codebook word lv otherwise;
// 0 when the scale is 0 or the scale or zero point is infinite
__device__ __forceinline__ int code_of(double y, double z16d, double s16d, uint32_t lv) {
#pragma clang fp contract(off)
  // a scale of 0, or a scale or zero point that overflowed fp16: every code is 0 (no NaN is
  // ever formed)
  if (s16d == 0.0 || !(fabs(s16d) < INFINITY) || !(fabs(z16d) < INFINITY)) return 0;
  const double t = (y - z16d) / s16d;
  if (lv != 0u) return codebook_code(t, lv);
  const double r = rint(t);
  return r > 3.0 ? 3 : (r >= 0.0 ? static_cast<int>(r) : 0);
}

struct Pair {
  double y0, y1;
};

// Compensated fp64 dot products of dims 2 lane and 2 lane + 1 over all 128 terms (the
// rare path: rows whose interval decisions did not settle).
__device__ __noinline__ Pair exact_pair(const uint16_t* __restrict__ src, const uint16_t* __restrict__ rot,
                                        int lane) {
#pragma clang fp contract(off)
  double s0 = 0.0, c0 = 0.0, s1 = 0.0, c1 = 0.0;
  for (int i = 0; i < kHeadDim; ++i) {
    const double xd = bf16_to_f64(src[i]);
    const uint32_t r = *reinterpret_cast<const uint32_t*>(rot + i * kHeadDim + 2 * lane);
    two_sum_add(s0, c0, xd * static_cast<double>(__uint_as_float(r << 16)));
    two_sum_add(s1, c1, xd * static_cast<double>(__uint_as_float(r & 0xFFFF0000u)));
  }
  return {s0 + c0, s1 + c1};
}

// Bit position of dim d's code in its K word (dim 16w + 4m + jj at bits 8jj + 2m).
__device__ __forceinline__ int k_shift(int d) { return 8 * (d & 3) + 2 * ((d & 15) >> 2); }

// Scale, zero point and the codes of dims 2 lane, 2 lane + 1 of one row.
struct RowDecision {
  ScaleZero sz;
  int c0, c1;
};

// Wave-level decision for one row from the fp64 sums (y0, y1) of dims 2 lane, 2 lane + 1 and
// their sum |p| (a0, a1), each within kBound sum|p| of the exact dot product: the group
// extremes, fp16 scale and zero point, and every code are taken at both ends of these
// intervals; when both ends agree, the decisions equal those of the exact dot products.
// Otherwise the row's dot products are recomputed with compensated (two-sum) fp64 sums
// from `src` (the row) and `rot` and decided from those.
__device__ __forceinline__ RowDecision decide_row(double y0, double y1, double a0, double a1, double cr, uint32_t lv,
                                                  const uint16_t* __restrict__ src, const uint16_t* __restrict__ rot,
                                                  int lane) {
#pragma clang fp contract(off)
  double d0 = kBound * a0, d1 = kBound * a1;
  RowDecision r;
  for (int pass = 0;; ++pass) {
    const double ymax = wave_max_f64(fmax(y0, y1));
    const double ymin = wave_min_f64(fmin(y0, y1));
    const double dm = wave_max_f64(fmax(d0, d1));
    // the scale is monotone in each extreme, so its range over the intervals is spanned
    // by these two corners; the zero point by the two ends of ymin's interval
    r.sz = scale_zero(cr, ymax - dm, ymin + dm);
    const ScaleZero sz2 = scale_zero(cr, ymax + dm, ymin - dm);
    const double s16d = f16_bits_to_f64(r.sz.s16);
    const double z16d = f16_bits_to_f64(r.sz.z16);
    r.c0 = code_of(y0 - d0, z16d, s16d, lv);
    r.c1 = code_of(y1 - d1, z16d, s16d, lv);
    // wave-uniform: both ends of every interval give the same decision (dm finite also
    // rules out overflow and NaN in the products)
    const bool row_ok = (r.sz.s16 == sz2.s16) && (r.sz.z16 == sz2.z16) && dm <= 1e300;
    const bool lane_ok = (r.c0 == code_of(y0 + d0, z16d, s16d, lv)) && (r.c1 == code_of(y1 + d1, z16d, s16d, lv));
    if (pass == 1 || (row_ok && __all(lane_ok))) break;
    const Pair e = exact_pair(src, rot, lane);
    y0 = e.y0;
    y1 = e.y1;
    d0 = d1 = 0.0;
  }
  return r;
}

// Stores of one decided row: the (s, z) pair, then the codes (one wave).
__device__ __forceinline__ void store_row(uint8_t* __restrict__ pool, int page, int slot, int head, int n_kv, int is_v,
                                          const RowDecision& d, int lane) {
  uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * kHeadBlock;
  if (lane == 0) {
    uint32_t* meta = reinterpret_cast<uint32_t*>(blk + (is_v ? kVMeta : kKMeta) + 4 * slot);
    *meta = static_cast<uint32_t>(d.sz.s16) | (static_cast<uint32_t>(d.sz.z16) << 16);
  }
  const int dd = 2 * lane;
  if (is_v) {
    // V codes are dim-major: this dim's word for slots 16u..16u+15 is shared with other
    // tokens, so clear and set only this slot's two bits.
    const int r = slot & 15;
    const int sh = 8 * (r & 3) + 2 * (r >> 2);
    uint32_t* w0 = reinterpret_cast<uint32_t*>(blk + v_word_offset(dd, slot >> 4));
    uint32_t* w1 = reinterpret_cast<uint32_t*>(blk + v_word_offset(dd + 1, slot >> 4));
    atomicAnd(w0, ~(3u << sh));
    atomicAnd(w1, ~(3u << sh));
    atomicOr(w0, static_cast<uint32_t>(d.c0) << sh);
    atomicOr(w1, static_cast<uint32_t>(d.c1) << sh);
    return;
  }
  // K word w (dims 16w..16w+15) gathers lanes 8w..8w+7; their bits are disjoint
  uint32_t bits = (static_cast<uint32_t>(d.c0) << k_shift(dd)) | (static_cast<uint32_t>(d.c1) << k_shift(dd + 1));
  bits |= __shfl_xor(bits, 1, 64);
  bits |= __shfl_xor(bits, 2, 64);
  bits |= __shfl_xor(bits, 4, 64);
  if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(blk + k_word_offset(slot, lane >> 3)) = bits;
}

// `item` = 2 (token n_kv + head) + (1 for V, 0 for K). With dst_page null the token is
// appended: token t goes to request t's history token hist_len[t] - 1, in the slot the
// block table gives it (nothing when that history is empty).
__device__ __forceinline__ void demote_row(unsigned char* __restrict__ smem, int item,
                                           const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
                                           int n_kv, const int32_t* __restrict__ dst_page,
                                           const int32_t* __restrict__ dst_slot, const uint16_t* __restrict__ rot_k,
                                           const uint16_t* __restrict__ rot_v, const float* __restrict__ clip_k,
                                           const float* __restrict__ clip_v, uint8_t* __restrict__ pool,
                                           const uint32_t* __restrict__ codebook = nullptr,
                                           const int32_t* __restrict__ block_table = nullptr, int max_pages = 0,
                                           const int32_t* __restrict__ hist_len = nullptr) {
#pragma clang fp contract(off)
  double(*part)[64][4] = reinterpret_cast<double(*)[64][4]>(smem);
  const int row = item >> 1;  // token * n_kv + head
  const int is_v = item & 1;
  const int tok = row / n_kv;
  const int head = row - tok * n_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const uint16_t* src = (is_v ? v_src : k_src) + static_cast<size_t>(row) * kHeadDim;
  const uint16_t* rot = (is_v ? rot_v : rot_k) + static_cast<size_t>(head) * kHeadDim * kHeadDim;

  // ---- every read of the row, issued before any arithmetic
  uint32_t xw[16], rw[32];
  const uint32_t* xp = reinterpret_cast<const uint32_t*>(src + 32 * wave);
#pragma unroll
  for (int k = 0; k < 16; ++k) xw[k] = xp[k];
  const uint32_t* rp = reinterpret_cast<const uint32_t*>(rot + 32 * wave * kHeadDim + 2 * lane);
#pragma unroll
  for (int i = 0; i < 32; ++i) rw[i] = rp[i * (kHeadDim / 2)];
  int page = 0, slot = 0;
  float crf = 0.f;
  uint32_t lv = 0u;  // codebook word (0: the uniform levels)
  if (!dst_page && hist_len[tok] < 1) return;  // appending to an empty history: nothing (uniform)
  if (wave == 0) {
    if (dst_page) {
      page = dst_page[tok];
      slot = dst_slot[tok];
    } else {
      // appending: token `tok` is request tok's history token hist_len - 1
      const int j = hist_len[tok] - 1;
      page = block_table[static_cast<size_t>(tok) * max_pages + j / kPageTokens];
      slot = j % kPageTokens;
    }
    crf = is_v ? clip_v[head] : clip_k[head];
    if (codebook) lv = codebook[2 * head + is_v];
  }

  // ---- this quarter's 32 terms of dims 2 lane, 2 lane + 1, and sum |p|
  double s0 = 0.0, s1 = 0.0, a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t xb = (i & 1) ? (xw[i >> 1] & 0xFFFF0000u) : (xw[i >> 1] << 16);
    const double xd = static_cast<double>(__uint_as_float(xb));
    const double r0 = static_cast<double>(__uint_as_float(rw[i] << 16));
    const double r1 = static_cast<double>(__uint_as_float(rw[i] & 0xFFFF0000u));
    s0 = fma(xd, r0, s0);
    s1 = fma(xd, r1, s1);
    a0 = fma(fabs(xd), fabs(r0), a0);
    a1 = fma(fabs(xd), fabs(r1), a1);
  }
  if (wave > 0) {
    double* pp = part[wave - 1][lane];
    pp[0] = s0;
    pp[1] = s1;
    pp[2] = a0;
    pp[3] = a1;
  }
  __syncthreads();
  if (wave > 0) return;  // uniform per wave; no barrier follows

  // ---- wave 0: join the quarters, decide on the error intervals
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const double* pp = part[w][lane];
    s0 = s0 + pp[0];
    s1 = s1 + pp[1];
    a0 = a0 + pp[2];
    a1 = a1 + pp[3];
  }
  const RowDecision d = decide_row(s0, s1, a0, a1, static_cast<double>(crf), lv, src, rot, lane);
  store_row(pool, page, slot, head, n_kv, is_v, d, lane);
}

// LDS of append_token: per row group, the quarter sums of waves 1..3 ([3][64][4] doubles),
// and the K group's quarter sums of q R_K for each query head ([3][GQT][64][2] doubles)
// and the packed bf16 high / low parts of the dequantised V row for its un-rotation
template <int GQT>
constexpr int append_smem_bytes() {
  return 2 * 3 * 64 * 4 * 8 + 3 * GQT * 64 * 2 * 8 + 2 * merge::kARow * 4;
}

// Level of code c in the dequantisation: c for the uniform levels, level c of the codebook
// word lv (in sixteenths) otherwise.
__device__ __forceinline__ double level_of(int c, uint32_t lv) {
  return lv ? static_cast<double>((lv >> (8 * c)) & 0xFFu) * 0.0625 : static_cast<double>(c);
}

// The one-launch decode step's appended token of request b and KV head kv: history token
// hist_len[b] - 1 (the slot the block table gives it). Its K and V rows (k_src, v_src
// [B][n_kv][128]) are demoted there exactly as oscar_demote does, and its own term of the
// attention of the KV head's GQT query heads is written as one more INT2 partial, split
// column `col` of `pstride` (rotated V basis: m = its score in log2 units, l = 1, acc = its
// dequantised V). K runs on waves 0..3 with q R_K accumulated beside it in fp64 (bf16
// products are exact); V on waves 4..7, or after K on a 4-wave workgroup. It is the work of
// a workgroup of its own, from the start of the launch. Every wave of the workgroup calls
// this (it holds barriers); the partial goes out with agent-scope stores.
// A request with an empty history gets an empty partial. With kUnrot the partial's value
// is un-rotated (times R_V^T) before it is written, as the INT2 splits' then are.
template <int NW, int GQT, bool kUnrot = false>
__device__ __forceinline__ void append_token(unsigned char* __restrict__ smem, int b, int kv, const StepArgs& a,
                                             int col, int pstride) {
#pragma clang fp contract(off)
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  double(*rpart)[3][64][4] = reinterpret_cast<double(*)[3][64][4]>(smem);
  double(*qpart)[GQT][64][2] = reinterpret_cast<double(*)[GQT][64][2]>(smem + 2 * 3 * 64 * 4 * 8);
  uint32_t* vhi_s = reinterpret_cast<uint32_t*>(smem + 2 * 3 * 64 * 4 * 8 + 3 * GQT * 64 * 2 * 8);
  uint32_t* vlo_s = vhi_s + merge::kARow;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int nh = a.hist_len[b];
  const size_t hrow = static_cast<size_t>(b) * a.n_q + static_cast<size_t>(kv) * GQT;
  auto put = [](float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  if (nh < 1) {
    for (int i = threadIdx.x; i < GQT * kHeadDim; i += 64 * NW) {
      const size_t o = (hrow + i / kHeadDim) * pstride + col;
      put(a.hist.acc + o * kHeadDim + (i % kHeadDim), 0.f);
      if (i % kHeadDim == 0) {
        put(a.hist.m + o, -INFINITY);
        put(a.hist.l + o, 0.f);
      }
    }
    return;
  }
  uint4 rb[8 / NW][4];
  if constexpr (kUnrot) merge::load_rv<NW>(a.rot_v, kv, rb);
  const int j = nh - 1;
  const int page = a.block_table[static_cast<size_t>(b) * a.max_pages + j / kPageTokens];
  const int slot = j % kPageTokens;
  const size_t row = static_cast<size_t>(b) * a.n_kv + kv;
  double qrot[GQT][2];  // K group leader: q R_K of each head at dims 2 lane, 2 lane + 1
  double khat0 = 0.0, khat1 = 0.0;

  for (int pass = 0; pass < (NW == 8 ? 1 : 2); ++pass) {
    // row group of this wave: 0 = K, 1 = V; wave wl of the group sums rows 32 wl .. + 31
    const int grp = NW == 8 ? (wave >> 2) : pass;
    const int wl = wave & 3;
    const int is_v = grp;
    const uint16_t* src = (is_v ? a.v_src : a.k_src) + row * kHeadDim;
    const uint16_t* rot = (is_v ? a.rot_v : a.rot_k) + static_cast<size_t>(kv) * kHeadDim * kHeadDim;
    uint32_t xw[16], rw[32];
    const uint32_t* xp = reinterpret_cast<const uint32_t*>(src + 32 * wl);
#pragma unroll
    for (int k = 0; k < 16; ++k) xw[k] = xp[k];
    const uint32_t* rp = reinterpret_cast<const uint32_t*>(rot + 32 * wl * kHeadDim + 2 * lane);
#pragma unroll
    for (int i = 0; i < 32; ++i) rw[i] = rp[i * (kHeadDim / 2)];
    double s0 = 0.0, s1 = 0.0, a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t xb = (i & 1) ? (xw[i >> 1] & 0xFFFF0000u) : (xw[i >> 1] << 16);
      const double xd = static_cast<double>(__uint_as_float(xb));
      const double r0 = static_cast<double>(__uint_as_float(rw[i] << 16));
      const double r1 = static_cast<double>(__uint_as_float(rw[i] & 0xFFFF0000u));
      s0 = fma(xd, r0, s0);
      s1 = fma(xd, r1, s1);
      a0 = fma(fabs(xd), fabs(r0), a0);
      a1 = fma(fabs(xd), fabs(r1), a1);
    }
    if (!is_v) {
      // q R_K of the KV head's query heads over the same rows
#pragma unroll
      for (int g = 0; g < GQT; ++g) {
        const uint32_t* qp = reinterpret_cast<const uint32_t*>(a.q + (hrow + g) * kHeadDim + 32 * wl);
        double q0 = 0.0, q1 = 0.0;
#pragma unroll
        for (int i = 0; i < 32; i += 2) {
          const uint32_t qq = qp[i / 2];  // wave-uniform
          const double qa = static_cast<double>(__uint_as_float(qq << 16));
          const double qb = static_cast<double>(__uint_as_float(qq & 0xFFFF0000u));
          q0 = fma(qa, static_cast<double>(__uint_as_float(rw[i] << 16)), q0);
          q1 = fma(qa, static_cast<double>(__uint_as_float(rw[i] & 0xFFFF0000u)), q1);
          q0 = fma(qb, static_cast<double>(__uint_as_float(rw[i + 1] << 16)), q0);
          q1 = fma(qb, static_cast<double>(__uint_as_float(rw[i + 1] & 0xFFFF0000u)), q1);
        }
        qrot[g][0] = q0;
        qrot[g][1] = q1;
        if (wl > 0) {
          qpart[wl - 1][g][lane][0] = q0;
          qpart[wl - 1][g][lane][1] = q1;
        }
      }
    }
    if (wl > 0) {
      double* pp = rpart[grp][wl - 1][lane];
      pp[0] = s0;
      pp[1] = s1;
      pp[2] = a0;
      pp[3] = a1;
    }
    __syncthreads();
    if (wl == 0) {
      // the group's leader: join the quarters, decide, store, and its part of the partial
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const double* pp = rpart[grp][w][lane];
        s0 = s0 + pp[0];
        s1 = s1 + pp[1];
        a0 = a0 + pp[2];
        a1 = a1 + pp[3];
      }
      const uint32_t lv = a.codebook ? a.codebook[2 * kv + is_v] : 0u;
      const float crf = is_v ? a.clip_v[kv] : a.clip_k[kv];
      const RowDecision d = decide_row(s0, s1, a0, a1, static_cast<double>(crf), lv, src, rot, lane);
      store_row(a.pool, page, slot, kv, a.n_kv, is_v, d, lane);
      // the dequantised value at dims 2 lane, 2 lane + 1 (rotated basis)
      const double sd = f16_bits_to_f64(d.sz.s16), zd = f16_bits_to_f64(d.sz.z16);
      const double h0 = level_of(d.c0, lv) * sd + zd, h1 = level_of(d.c1, lv) * sd + zd;
      if (!is_v) {
        khat0 = h0;
        khat1 = h1;
#pragma unroll
        for (int g = 0; g < GQT; ++g) {
          double x0 = qrot[g][0], x1 = qrot[g][1];
#pragma unroll
          for (int w = 0; w < 3; ++w) {
            x0 = x0 + qpart[w][g][lane][0];
            x1 = x1 + qpart[w][g][lane][1];
          }
          const double dot = wave_sum_f64(x0 * khat0 + x1 * khat1);
          if (lane == 0) {
            const size_t o = (hrow + g) * pstride + col;
            put(a.hist.m + o, static_cast<float>(dot * a.scale_log2));
            put(a.hist.l + o, 1.f);
          }
        }
      } else if constexpr (kUnrot) {
        merge::split2(static_cast<float>(h0), static_cast<float>(h1), vhi_s[lane], vlo_s[lane]);
      } else {
#pragma unroll
        for (int g = 0; g < GQT; ++g) {
          const size_t o = (hrow + g) * pstride + col;
          put(a.hist.acc + o * kHeadDim + 2 * lane, static_cast<float>(h0));
          put(a.hist.acc + o * kHeadDim + 2 * lane + 1, static_cast<float>(h1));
        }
      }
    }
    if (NW == 4 && pass == 0) __syncthreads();  // the V pass reuses the LDS
  }
  if constexpr (kUnrot) {
    // the V row's A operand is in LDS: every wave un-rotates its output tiles, for all
    // the KV head's query heads (the same vector)
    __syncthreads();
    merge::unrotate_tiles<NW>(vhi_s, vlo_s, 1, rb, [&](int, int d, float v) {
#pragma unroll
      for (int g = 0; g < GQT; ++g) put(a.hist.acc + ((hrow + g) * pstride + col) * kHeadDim + d, v);
    });
  }
}

}  // namespace demote
}  // namespace oscar
