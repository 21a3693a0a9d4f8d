// BF16 sink/recent pass of decode attention: device code shared by the standalone window
// kernel and the fused decode kernels.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the sink (first 64
// tokens) and the recent window (last 256 tokens) stay in BF16 and are handled by a BF16
// kernel, separately from the INT2 history.
//
// A workgroup serves one (window split of 64 slots, KV head, request), 256 threads: four threads per slot
// for the scores (dot products in fp64, so large logits keep their low bits), then
// thread (dim pair, 16-slot group) for the value sum; every load of a phase is issued
// before its arithmetic.

#pragma once

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace window {

template <int GQ>
constexpr int window_smem_bytes() {
  return GQ * kHeadDim * 4 + GQ * kPageTokens * 8 + GQ * kPageTokens * 4 + 2 * GQ * 4 + 4 * GQ * kHeadDim * 4;
}

// One workgroup (256 threads) of the BF16 window pass: slots 64 c .. 64 c + 63 of KV head kv
// of request b for the KV head's GQ query heads. `smem` holds window_smem_bytes<GQ>().
template <int GQ>
__device__ __forceinline__ void window_split(
    unsigned char* __restrict__ smem, int c, int kv, int b, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_win, const uint16_t* __restrict__ v_win,
    const int32_t* __restrict__ win_len, int n_q, int n_kv, int window, int n_wsplits, double scale_log2,
    float* __restrict__ out_m, float* __restrict__ out_l, float* __restrict__ out_acc) {
  double(*sc_s)[kPageTokens] = reinterpret_cast<double(*)[kPageTokens]>(smem);
  float(*q_s)[kHeadDim] = reinterpret_cast<float(*)[kHeadDim]>(smem + GQ * kPageTokens * 8);
  float(*p_s)[kPageTokens] = reinterpret_cast<float(*)[kPageTokens]>(smem + GQ * kPageTokens * 8 + GQ * kHeadDim * 4);
  float* m_s = reinterpret_cast<float*>(smem + GQ * kPageTokens * 12 + GQ * kHeadDim * 4);
  float* l_s = m_s + GQ;
  float(*acc_s)[GQ][kHeadDim] = reinterpret_cast<float(*)[GQ][kHeadDim]>(smem + GQ * kPageTokens * 12 + GQ * kHeadDim * 4 + 2 * GQ * 4);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h0 = kv * GQ;

  for (int i = tid; i < GQ * kHeadDim; i += 256)
    q_s[i >> 7][i & 127] = bf16_to_f32(q[(static_cast<size_t>(b) * n_q + h0) * kHeadDim + i]);

  const int t0 = c * kPageTokens;
  const int ntok = max(0, min(kPageTokens, win_len[b] - t0));
  const size_t base = ((static_cast<size_t>(b) * n_kv + kv) * window + t0) * kHeadDim;

  // scores: four threads per slot, 32 dims each, dot products in fp64 (bf16 products are
  // exact), four heads at a time
  {
    const int slot = tid >> 2;
    const int quarter = tid & 3;
    const bool valid = slot < ntok;
    uint4 kx[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      kx[w] = valid ? reinterpret_cast<const uint4*>(k_win + base + static_cast<size_t>(slot) * kHeadDim + 32 * quarter)[w]
                    : make_uint4(0, 0, 0, 0);
    __syncthreads();
    constexpr int kChunk = GQ < 4 ? GQ : 4;
#pragma unroll 1
    for (int g0 = 0; g0 < GQ; g0 += kChunk) {
      double dot[kChunk];
#pragma unroll
      for (int g = 0; g < kChunk; ++g) dot[g] = 0.0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t xs[4] = {kx[w].x, kx[w].y, kx[w].z, kx[w].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double lo = static_cast<double>(__uint_as_float(xs[e] << 16));
          const double hi = static_cast<double>(__uint_as_float(xs[e] & 0xFFFF0000u));
          const int d = 32 * quarter + 8 * w + 2 * e;
#pragma unroll
          for (int g = 0; g < kChunk; ++g)
            dot[g] = fma(hi, static_cast<double>(q_s[g0 + g][d + 1]),
                         fma(lo, static_cast<double>(q_s[g0 + g][d]), dot[g]));
        }
      }
#pragma unroll
      for (int g = 0; g < kChunk; ++g) {
        double v = dot[g];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        if (quarter == 0) sc_s[g0 + g][slot] = valid ? v * scale_log2 : -INFINITY;
      }
    }
  }
  __syncthreads();
  // per head: reference point = the float nearest the largest score, weights, their sum
  for (int g = wave; g < GQ; g += 4) {
    const double s = sc_s[g][lane];
    const float big = static_cast<float>(wave_max(s));
    const float pt = (lane < ntok) ? exp2f(static_cast<float>(s - static_cast<double>(big))) : 0.f;
    p_s[g][lane] = pt;
    const float l = wave_sum(pt);
    if (lane == 0) {
      m_s[g] = ntok > 0 ? big : -INFINITY;
      l_s[g] = l;
    }
  }
  __syncthreads();

  // value sum: thread (dim pair, slot group of 16)
  const int dp = tid & 63;
  const int sg = tid >> 6;
  uint32_t vv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = 16 * sg + i;
    vv[i] = t < ntok ? *reinterpret_cast<const uint32_t*>(v_win + base + static_cast<size_t>(t) * kHeadDim + 2 * dp) : 0u;
  }
  float a0[GQ], a1[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) a0[g] = a1[g] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v0 = __uint_as_float(vv[i] << 16);
    const float v1 = __uint_as_float(vv[i] & 0xFFFF0000u);
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float pt = p_s[g][16 * sg + i];
      a0[g] = fmaf(pt, v0, a0[g]);
      a1[g] = fmaf(pt, v1, a1[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    acc_s[sg][g][2 * dp] = a0[g];
    acc_s[sg][g][2 * dp + 1] = a1[g];
  }
  __syncthreads();
  for (int idx = tid; idx < GQ * kHeadDim; idx += 256) {
    const int g = idx >> 7;
    const int d = idx & 127;
    const size_t o = (static_cast<size_t>(b) * n_q + h0 + g) * n_wsplits + c;
    out_acc[o * kHeadDim + d] = acc_s[0][g][d] + acc_s[1][g][d] + acc_s[2][g][d] + acc_s[3][g][d];
    if (d == 0) {
      out_m[o] = m_s[g];
      out_l[o] = l_s[g];
    }
  }
}

}  // namespace window
}  // namespace oscar
