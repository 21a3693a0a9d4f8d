// Demotion of recent-window tokens into the INT2 history (rotate, clip, quantise, pack):
// device code shared by the standalone demote kernel and the fused decode-step kernel.
//
// Method: OSCAR (Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
// Quantization); QbitAI article on OSCAR, serving-path section: the oldest recent token
// is rotated, clipped, quantised and packed four 2-bit codes per byte into the INT2
// history, with a scale and zero point per group.
//
// One workgroup of 256 threads handles one row (token, KV head, K or V) with its rotation
// staged in LDS; threads j and j + 128 sum the two halves of output dim j. Each half is
// accumulated in fp64 with compensated (two-sum) chains over exact bf16 x bf16 products
// and the halves are joined by the same two-sum, so the group extremes, and from them the
// fp16 scale and zero point, come from the dot product's fp64 value; the scale/zero
// arithmetic is fp64 exactly as specified.

#pragma once

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace demote {

constexpr int kSmemBytes = kHeadDim * kHeadDim * 2 + kHeadDim * 8 + kHeadDim * 16 + 64 + kHeadDim;

__device__ __forceinline__ void two_sum_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  c += (s - (t - bp)) + (p - bp);
  s = t;
}

// `item` = 2 (token n_kv + head) + (1 for V, 0 for K)
__device__ __forceinline__ void demote_row(unsigned char* __restrict__ smem, int item,
                                           const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
                                           int n_kv, const int32_t* __restrict__ dst_page,
                                           const int32_t* __restrict__ dst_slot, const uint16_t* __restrict__ rot_k,
                                           const uint16_t* __restrict__ rot_v, const float* __restrict__ clip_k,
                                           const float* __restrict__ clip_v, uint8_t* __restrict__ pool) {
  // every product and sum below is rounded on its own, as the quantiser specifies
#pragma clang fp contract(off)
  uint16_t* r_s = reinterpret_cast<uint16_t*>(smem);
  double* xs = reinterpret_cast<double*>(smem + kHeadDim * kHeadDim * 2);
  double* half_s = xs + kHeadDim;                 // (s, c) of the upper halves
  double* red_s = half_s + 2 * kHeadDim;          // wave maxima then minima
  uint8_t* codes_s = reinterpret_cast<uint8_t*>(red_s + 8);

  const int row = item >> 1;  // token * n_kv + head
  const int is_v = item & 1;
  const int tok = row / n_kv;
  const int head = row - tok * n_kv;
  const int tid = threadIdx.x;
  const int j = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  const int wave = tid >> 6;

  const uint16_t* src = (is_v ? v_src : k_src) + static_cast<size_t>(row) * kHeadDim;
  stage_rotation(r_s, (is_v ? rot_v : rot_k) + static_cast<size_t>(head) * kHeadDim * kHeadDim, tid, 256);
  if (tid < kHeadDim) xs[tid] = bf16_to_f64(src[tid]);
  __syncthreads();

  // two independent compensated chains per half (for latency), joined by the same two-sum
  double s[2] = {0.0, 0.0}, c[2] = {0.0, 0.0};
  const int i0 = 64 * half;
#pragma unroll 8
  for (int i = i0; i < i0 + 64; i += 2)
#pragma unroll
    for (int u = 0; u < 2; ++u) two_sum_add(s[u], c[u], xs[i + u] * bf16_to_f64(r_s[(i + u) * kHeadDim + j]));
  double st = s[0], ct = c[0] + c[1];
  two_sum_add(st, ct, s[1]);
  if (half) {
    half_s[2 * j] = st;
    half_s[2 * j + 1] = ct;
  }
  __syncthreads();
  double y = 0.0;
  if (!half) {
    ct += half_s[2 * j + 1];
    two_sum_add(st, ct, half_s[2 * j]);
    y = st + ct;
  }
  // extremes over the 128 dims (waves 0 and 1)
  const double wmax = wave_max(y);
  const double wmin = wave_min(y);
  if ((tid & 63) == 0 && wave < 2) {
    red_s[wave] = wmax;
    red_s[4 + wave] = wmin;
  }
  __syncthreads();
  const double ymax = fmax(red_s[0], red_s[1]);
  const double ymin = fmin(red_s[4], red_s[5]);

  const double cr = static_cast<double>(is_v ? clip_v[head] : clip_k[head]);
  const double hi = cr * ymax;
  const double lo = cr * ymin;
  const double sc = (hi - lo) / 3.0;
  const uint16_t s16 = f64_to_f16_rne(sc);
  const uint16_t z16 = f64_to_f16_rne(lo);
  const double s16d = f16_bits_to_f64(s16);
  const double z16d = f16_bits_to_f64(z16);
  int code = 0;
  if (s16d != 0.0) {
    const double t = rint((y - z16d) / s16d);
    code = t < 0.0 ? 0 : (t > 3.0 ? 3 : static_cast<int>(t));
  }

  const int page = dst_page[tok];
  const int slot = dst_slot[tok];
  uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * kHeadBlock;
  if (tid == 0) {
    uint32_t* meta = reinterpret_cast<uint32_t*>(blk + (is_v ? kVMeta : kKMeta) + 4 * slot);
    *meta = static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16);
  }
  if (is_v) {
    // V codes are dim-major: this dim's word for slots 16u..16u+15 is shared with other
    // tokens, so clear and set only this slot's two bits.
    if (!half) {
      const int r = slot & 15;
      const int sh = 8 * (r & 3) + 2 * (r >> 2);
      uint32_t* w = reinterpret_cast<uint32_t*>(blk + v_word_offset(j, slot >> 4));
      atomicAnd(w, ~(3u << sh));
      atomicOr(w, static_cast<uint32_t>(code) << sh);
    }
    return;  // uniform over the workgroup: is_v is per row
  }
  if (!half) codes_s[j] = static_cast<uint8_t>(code);
  __syncthreads();
  if (tid < 8) {
    // K word w holds dims 16w..16w+15, dim 16w+4m+jj at bits 8jj+2m.
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        word |= static_cast<uint32_t>(codes_s[16 * tid + 4 * m + jj]) << (8 * jj + 2 * m);
    *reinterpret_cast<uint32_t*>(blk + k_word_offset(slot, tid)) = word;
  }
}

}  // namespace demote
}  // namespace oscar
