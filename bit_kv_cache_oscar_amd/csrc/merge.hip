// Online-softmax merge of the INT2 and BF16 segments, with the value un-rotation.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the BF16 and INT2 parts
// of decode are combined by an online-softmax merge. The INT2 value sum lives in the
// rotated basis of R_V (values were rotated before quantisation), so it is multiplied by
// R_V^T before joining the BF16 part; un-rotating after the reduction is exact because
// the un-rotation is linear.
//
// Grid (query head, request), 256 threads: R_V of the head's KV head is staged in LDS,
// the split reductions keep many loads in flight, then one row of R_V per output dim.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

constexpr int kRowPad = 130;  // bf16 elements per LDS row: odd dword stride, no bank conflicts

// Online-softmax reduction of `ns` partials of one (request, head) held at m[o..o+ns),
// l[o..), acc[(o..)*128 + d]: 128 dims x 2 split-halves per pass over 256 threads.
// Returns (max, sum) to every thread and leaves the reduced acc in out_s[128].
__device__ __forceinline__ void reduce_splits(const float* __restrict__ pm, const float* __restrict__ pl,
                                              const float* __restrict__ pa, size_t o, int ns, float* red_s,
                                              float* part_s, float* out_s, float& big_out, float& l_out) {
  const int tid = threadIdx.x;
  float big = -INFINITY;
  for (int s = tid; s < ns; s += 256) big = fmaxf(big, pm[o + s]);
  big = wave_max(big);
  if ((tid & 63) == 0) red_s[tid >> 6] = big;
  __syncthreads();
  big = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  __syncthreads();
  float l = 0.f;
  if (big != -INFINITY)
    for (int s = tid; s < ns; s += 256) l = fmaf(exp2f(pm[o + s] - big), pl[o + s], l);
  l = wave_sum(l);
  if ((tid & 63) == 0) red_s[tid >> 6] = l;
  const int d = tid & 127;
  const int half = tid >> 7;
  float a = 0.f;
  if (big != -INFINITY) {
#pragma unroll 16
    for (int s = half; s < ns; s += 2) a = fmaf(exp2f(pm[o + s] - big), pa[(o + s) * kHeadDim + d], a);
  }
  part_s[tid] = a;
  __syncthreads();
  l_out = red_s[0] + red_s[1] + red_s[2] + red_s[3];
  big_out = big;
  if (tid < 128) out_s[tid] = part_s[tid] + part_s[tid + 128];
  __syncthreads();
}

template <int GQ>
__global__ __launch_bounds__(256) void merge_kernel(
    const float* __restrict__ hm, const float* __restrict__ hl, const float* __restrict__ hacc, int n_splits,
    const float* __restrict__ wm, const float* __restrict__ wl, const float* __restrict__ wacc, int n_wsplits,
    const uint16_t* __restrict__ rot_v, float* __restrict__ out, int n_q) {
  __shared__ uint16_t r_s[kHeadDim * kRowPad];
  __shared__ float accr_s[kHeadDim];
  __shared__ float accw_s[kHeadDim];
  __shared__ float part_s[256];
  __shared__ float red_s[4];

  const int h = blockIdx.x;
  const int kv = h / GQ;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  if (n_splits > 0) {  // (no INT2 partials: no rotated sum to un-rotate, R_V is not read)
    // R_V into LDS rows padded to an odd dword stride (conflict-free row reads below)
    const uint4* src = reinterpret_cast<const uint4*>(rot_v + static_cast<size_t>(kv) * kHeadDim * kHeadDim);
#pragma unroll
    for (int i = tid; i < kHeadDim * kHeadDim / 8; i += 256) {
      const uint4 v = src[i];
      uint32_t* dst = reinterpret_cast<uint32_t*>(r_s + (i >> 4) * kRowPad + (i & 15) * 8);
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
  }
  const size_t row = static_cast<size_t>(b) * n_q + h;
  float mh, lh, mw, lw;
  reduce_splits(hm, hl, hacc, row * n_splits, n_splits, red_s, part_s, accr_s, mh, lh);
  reduce_splits(wm, wl, wacc, row * n_wsplits, n_wsplits, red_s, part_s, accw_s, mw, lw);
  if (tid < 128) {
    float oh = 0.f;
    const uint16_t* r = r_s + tid * kRowPad;
    if (n_splits > 0) {
#pragma unroll 8
      for (int j = 0; j < kHeadDim; ++j) oh = fmaf(accr_s[j], bf16_to_f32(r[j]), oh);
    }
    const float big = fmaxf(mh, mw);
    float res = 0.f;
    if (big != -INFINITY) {
      const float al = exp2f(mh - big);
      const float be = exp2f(mw - big);
      res = fmaf(al, oh, be * accw_s[tid]) / fmaf(al, lh, be * lw);
    }
    out[row * kHeadDim + tid] = res;
  }
}

template <int GQ>
hipError_t launch(const LayerShape& L, const PartialsView& hist, int n_splits, const PartialsView& win,
                  int n_wsplits, const void* rot_v, float* out, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel<GQ>, dim3(L.n_q, batch), dim3(256), 0, stream, hist.m, hist.l, hist.acc,
                     n_splits, win.m, win.l, win.acc, n_wsplits, static_cast<const uint16_t*>(rot_v), out, L.n_q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const LayerShape& L, const PartialsView& hist, int n_splits, const PartialsView& win,
                        int n_wsplits, const void* rot_v, float* out, int batch, hipStream_t stream) {
  switch (L.gq) {
    case 1: return launch<1>(L, hist, n_splits, win, n_wsplits, rot_v, out, batch, stream);
    case 2: return launch<2>(L, hist, n_splits, win, n_wsplits, rot_v, out, batch, stream);
    case 4: return launch<4>(L, hist, n_splits, win, n_wsplits, rot_v, out, batch, stream);
    case 8: return launch<8>(L, hist, n_splits, win, n_wsplits, rot_v, out, batch, stream);
    case 16: return launch<16>(L, hist, n_splits, win, n_wsplits, rot_v, out, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
