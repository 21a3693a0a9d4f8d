// Demotion of one row into pages with NG quantisation groups per vector (groups of 128 / NG
// rotated dims, one fp16 scale and zero point per group): device code shared by the grouped
// demotion kernel and the grouped decode step's first launch.
//
// Method: OSCAR; QbitAI article on OSCAR, section on aiming the rotation at attention: the
// bit-reversal in R makes the INT2 groups more balanced (the scale and zero point are per
// group); serving-path section: demotion rotates, clips, quantises and packs.
//
// One 256-thread workgroup per (token, KV head, K or V), as the one-group per-row demotion:
// fp64 dot products with an error bound per dim, decisions at both ends of the intervals,
// compensated sums when they do not settle; the extremes, scale and zero point are taken per
// group (a group's dims are held by 64 / NG consecutive lanes of wave 0). The page layout is
// head_block_bytes<NG>'s: the codes as in the one-group layout, then the K (scale, zero)
// pairs, NG per slot, then the V pairs.

#pragma once

#include "demote_pass.h"

namespace oscar {
namespace demote {

constexpr int kGroupedSmemBytes = 3 * 64 * 4 * 8;

// max (SEL 0) or min (SEL 1) over aligned segments of W lanes
template <int W, int SEL>
__device__ __forceinline__ double seg_ext(double v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) {
    const double u = __shfl_xor(v, o, 64);
    v = SEL == 0 ? fmax(v, u) : fmin(v, u);
  }
  return v;
}

// Row `item` / 2 (token, KV head) of k_src or v_src (item odd: V) into its page and slot.
// All 256 threads call it; `smem` holds kGroupedSmemBytes.
template <int NG>
__device__ __forceinline__ void demote_grouped_row(
    unsigned char* __restrict__ smem, int item, const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int n_kv,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ dst_slot, const uint16_t* __restrict__ rot_k,
    const uint16_t* __restrict__ rot_v, const float* __restrict__ clip_k, const float* __restrict__ clip_v,
    uint8_t* __restrict__ pool) {
#pragma clang fp contract(off)
  constexpr int kLanes = 64 / NG;  // lanes of wave 0 holding one group (two dims each)
  double(*part)[64][4] = reinterpret_cast<double(*)[64][4]>(smem);
  const int row = item >> 1;
  const int is_v = item & 1;
  const int tok = row / n_kv;
  const int head = row - tok * n_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* src = (is_v ? v_src : k_src) + static_cast<size_t>(row) * kHeadDim;
  const uint16_t* rot = (is_v ? rot_v : rot_k) + static_cast<size_t>(head) * kHeadDim * kHeadDim;

  uint32_t xw[16], rw[32];
  const uint32_t* xp = reinterpret_cast<const uint32_t*>(src + 32 * wave);
#pragma unroll
  for (int k = 0; k < 16; ++k) xw[k] = xp[k];
  const uint32_t* rp = reinterpret_cast<const uint32_t*>(rot + 32 * wave * kHeadDim + 2 * lane);
#pragma unroll
  for (int i = 0; i < 32; ++i) rw[i] = rp[i * (kHeadDim / 2)];
  int page = 0, slot = 0;
  float crf = 0.f;
  if (wave == 0) {
    page = dst_page[tok];
    slot = dst_slot[tok];
    crf = is_v ? clip_v[head] : clip_k[head];
  }
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
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const double* pp = part[w][lane];
    s0 = s0 + pp[0];
    s1 = s1 + pp[1];
    a0 = a0 + pp[2];
    a1 = a1 + pp[3];
  }
  double y0 = s0, y1 = s1;
  double d0 = kBound * a0, d1 = kBound * a1;
  const double cr = static_cast<double>(crf);
  ScaleZero sz;
  int c0, c1;
  for (int pass = 0;; ++pass) {
    // the extremes of this lane's group (both of its dims lie in it)
    const double ymax = seg_ext<kLanes, 0>(fmax(y0, y1));
    const double ymin = seg_ext<kLanes, 1>(fmin(y0, y1));
    const double dm = seg_ext<kLanes, 0>(fmax(d0, d1));
    sz = scale_zero(cr, ymax - dm, ymin + dm);
    const ScaleZero sz2 = scale_zero(cr, ymax + dm, ymin - dm);
    const double s16d = f16_bits_to_f64(sz.s16);
    const double z16d = f16_bits_to_f64(sz.z16);
    c0 = code_of(y0 - d0, z16d, s16d, 0u);
    c1 = code_of(y1 - d1, z16d, s16d, 0u);
    const bool group_ok = (sz.s16 == sz2.s16) && (sz.z16 == sz2.z16) && dm <= 1e300;
    const bool lane_ok = (c0 == code_of(y0 + d0, z16d, s16d, 0u)) &&
                         (c1 == code_of(y1 + d1, z16d, s16d, 0u));
    if (pass == 1 || __all(group_ok && lane_ok)) break;
    const Pair e = exact_pair(src, rot, lane);
    y0 = e.y0;
    y1 = e.y1;
    d0 = d1 = 0.0;
  }

  uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * head_block_bytes<NG>();
  if (lane % kLanes == 0) {
    const int g = lane / kLanes;
    uint32_t* meta = reinterpret_cast<uint32_t*>(blk + 4096 + (is_v ? 256 * NG : 0) + 4 * (NG * slot + g));
    *meta = static_cast<uint32_t>(sz.s16) | (static_cast<uint32_t>(sz.z16) << 16);
  }
  const int dd = 2 * lane;
  if (is_v) {
    const int r = slot & 15;
    const int sh = 8 * (r & 3) + 2 * (r >> 2);
    uint32_t* w0 = reinterpret_cast<uint32_t*>(blk + v_word_offset(dd, slot >> 4));
    uint32_t* w1 = reinterpret_cast<uint32_t*>(blk + v_word_offset(dd + 1, slot >> 4));
    atomicAnd(w0, ~(3u << sh));
    atomicAnd(w1, ~(3u << sh));
    atomicOr(w0, static_cast<uint32_t>(c0) << sh);
    atomicOr(w1, static_cast<uint32_t>(c1) << sh);
    return;
  }
  uint32_t bits = (static_cast<uint32_t>(c0) << k_shift(dd)) |
                  (static_cast<uint32_t>(c1) << k_shift(dd + 1));
  bits |= __shfl_xor(bits, 1, 64);
  bits |= __shfl_xor(bits, 2, 64);
  bits |= __shfl_xor(bits, 4, 64);
  if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(blk + k_word_offset(slot, lane >> 3)) = bits;
}

}  // namespace demote
}  // namespace oscar
