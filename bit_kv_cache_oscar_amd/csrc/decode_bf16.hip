// BF16 sink/recent pass of decode attention.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the sink (first 64
// tokens) and the recent window (last 256 tokens) stay in BF16 and are handled by a BF16
// kernel, separately from the INT2 history.
//
// Grid (window split of 64 slots, kv_head, request), 256 threads: four threads per slot
// for the scores (dot products in fp64, so large logits keep their low bits), then
// thread (dim pair, 16-slot group) for the value sum; every load of a phase is issued
// before its arithmetic.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

template <int GQ>
__global__ __launch_bounds__(256) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_win, const uint16_t* __restrict__ v_win,
    const int32_t* __restrict__ win_len, int n_q, int n_kv, int window, int n_wsplits, double scale_log2,
    float* __restrict__ out_m, float* __restrict__ out_l, float* __restrict__ out_acc) {
  __shared__ float q_s[GQ][kHeadDim];
  __shared__ double sc_s[GQ][kPageTokens];
  __shared__ float p_s[GQ][kPageTokens];
  __shared__ float m_s[GQ];
  __shared__ float l_s[GQ];
  __shared__ float acc_s[4][GQ][kHeadDim];
  const int c = blockIdx.x;
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
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

template <int GQ>
hipError_t launch(const LayerShape& L, const void* q, const void* k_win, const void* v_win,
                  const int32_t* win_len, int batch, float sm_scale, int n_wsplits, const PartialsView& out,
                  hipStream_t stream) {
  hipLaunchKernelGGL(decode_bf16_kernel<GQ>, dim3(n_wsplits, L.n_kv, batch), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_win),
                     static_cast<const uint16_t*>(v_win), win_len, L.n_q, L.n_kv, L.window, n_wsplits,
                     static_cast<double>(sm_scale) * 1.4426950408889634, out.m, out.l, out.acc);
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
