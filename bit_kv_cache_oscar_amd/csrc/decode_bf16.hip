// BF16 sink/recent pass of decode attention.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the sink (first 64
// tokens) and the recent window (last 256 tokens) stay in BF16 and are handled by a BF16
// kernel, separately from the INT2 history.
//
// Grid (window split of 64 slots, kv_head, request), one wave each: lane = slot for the
// scores, lane = dims 2*lane and 2*lane + 1 for the value sum.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

template <int GQ>
__global__ __launch_bounds__(64) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_win, const uint16_t* __restrict__ v_win,
    const int32_t* __restrict__ win_len, int n_q, int n_kv, int window, int n_wsplits, float scale_log2,
    float* __restrict__ out_m, float* __restrict__ out_l, float* __restrict__ out_acc) {
  __shared__ float q_s[GQ][kHeadDim];
  const int c = blockIdx.x;
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int h0 = kv * GQ;

  for (int i = lane; i < GQ * kHeadDim; i += 64)
    q_s[i >> 7][i & 127] = bf16_to_f32(q[(static_cast<size_t>(b) * n_q + h0) * kHeadDim + i]);
  __syncthreads();

  const int t0 = c * kPageTokens;
  const int ntok = max(0, min(kPageTokens, win_len[b] - t0));
  const size_t base = ((static_cast<size_t>(b) * n_kv + kv) * window + t0) * kHeadDim;
  const bool valid = lane < ntok;

  float dot[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) dot[g] = 0.f;
  if (valid) {
    const uint4* krow = reinterpret_cast<const uint4*>(k_win + base + static_cast<size_t>(lane) * kHeadDim);
#pragma unroll 4
    for (int w = 0; w < 16; ++w) {
      const uint4 x = krow[w];
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(xs[e] << 16);
        const float hi = __uint_as_float(xs[e] & 0xFFFF0000u);
        const int d = 8 * w + 2 * e;
#pragma unroll
        for (int g = 0; g < GQ; ++g) dot[g] = fmaf(hi, q_s[g][d + 1], fmaf(lo, q_s[g][d], dot[g]));
      }
    }
  }

  float pw[GQ], mx[GQ], ls[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const float sc = valid ? dot[g] * scale_log2 : -INFINITY;
    mx[g] = wave_max(sc);
    pw[g] = valid ? exp2f(sc - mx[g]) : 0.f;
    ls[g] = wave_sum(pw[g]);
  }

  float acc0[GQ], acc1[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) acc0[g] = acc1[g] = 0.f;
  const uint16_t* vbase = v_win + base + 2 * lane;
  for (int t = 0; t < ntok; ++t) {
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(vbase + static_cast<size_t>(t) * kHeadDim);
    const float v0 = __uint_as_float(vv << 16);
    const float v1 = __uint_as_float(vv & 0xFFFF0000u);
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float pt = lane_value(pw[g], t);
      acc0[g] = fmaf(pt, v0, acc0[g]);
      acc1[g] = fmaf(pt, v1, acc1[g]);
    }
  }

#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const size_t o = (static_cast<size_t>(b) * n_q + h0 + g) * n_wsplits + c;
    out_acc[o * kHeadDim + 2 * lane] = acc0[g];
    out_acc[o * kHeadDim + 2 * lane + 1] = acc1[g];
    if (lane == 0) {
      out_m[o] = ntok > 0 ? mx[g] : -INFINITY;
      out_l[o] = ntok > 0 ? ls[g] : 0.f;
    }
  }
}

template <int GQ>
hipError_t launch(const LayerShape& L, const void* q, const void* k_win, const void* v_win,
                  const int32_t* win_len, int batch, float sm_scale, int n_wsplits, const PartialsView& out,
                  hipStream_t stream) {
  hipLaunchKernelGGL(decode_bf16_kernel<GQ>, dim3(n_wsplits, L.n_kv, batch), dim3(64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_win),
                     static_cast<const uint16_t*>(v_win), win_len, L.n_q, L.n_kv, L.window, n_wsplits,
                     sm_scale * kLog2e, out.m, out.l, out.acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const LayerShape& L, const void* q, const void* k_win, const void* v_win,
                              const int32_t* win_len, int batch, float sm_scale, int n_wsplits,
                              const PartialsView& out, hipStream_t stream) {
  switch (L.gq) {
    case 1: return launch<1>(L, q, k_win, v_win, win_len, batch, sm_scale, n_wsplits, out, stream);
    case 2: return launch<2>(L, q, k_win, v_win, win_len, batch, sm_scale, n_wsplits, out, stream);
    case 4: return launch<4>(L, q, k_win, v_win, win_len, batch, sm_scale, n_wsplits, out, stream);
    case 8: return launch<8>(L, q, k_win, v_win, win_len, batch, sm_scale, n_wsplits, out, stream);
    case 16: return launch<16>(L, q, k_win, v_win, win_len, batch, sm_scale, n_wsplits, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
