// Online-softmax merge of the INT2 and BF16 segments, with the value un-rotation.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the BF16 and INT2 parts
// of decode are combined by an online-softmax merge. The INT2 value sum lives in the
// rotated basis of R_V (values were rotated before quantisation), so it is multiplied by
// R_V^T before joining the BF16 part; un-rotating after the reduction is exact because
// the un-rotation is linear.
//
// Grid (kv_head, request), 256 threads: R_V of the head is staged once in LDS and serves
// every query head of the group.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

constexpr int kRowPad = 130;  // bf16 elements per LDS row: odd dword stride, no bank conflicts

template <int GQ>
__global__ __launch_bounds__(256) void merge_kernel(
    const float* __restrict__ hm, const float* __restrict__ hl, const float* __restrict__ hacc, int n_splits,
    const float* __restrict__ wm, const float* __restrict__ wl, const float* __restrict__ wacc, int n_wsplits,
    const uint16_t* __restrict__ rot_v, float* __restrict__ out, int n_q) {
  __shared__ uint16_t r_s[kHeadDim * kRowPad];
  __shared__ float accr_s[kHeadDim];
  __shared__ float accw_s[kHeadDim];
  __shared__ float scal_s[4];

  const int kv = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const uint16_t* rot = rot_v + static_cast<size_t>(kv) * kHeadDim * kHeadDim;
  for (int i = tid; i < kHeadDim * kHeadDim; i += 256) r_s[(i >> 7) * kRowPad + (i & 127)] = rot[i];

  for (int g = 0; g < GQ; ++g) {
    const int h = kv * GQ + g;
    const int d = tid & 127;
    const bool hist_side = tid < 128;
    const int ns = hist_side ? n_splits : n_wsplits;
    const size_t o = (static_cast<size_t>(b) * n_q + h) * ns;
    const float* pm = hist_side ? hm : wm;
    const float* pl = hist_side ? hl : wl;
    const float* pa = hist_side ? hacc : wacc;
    float big = -INFINITY;
    for (int s = 0; s < ns; ++s) big = fmaxf(big, pm[o + s]);
    float l = 0.f, a = 0.f;
    if (big != -INFINITY) {
      for (int s = 0; s < ns; ++s) {
        const float w = exp2f(pm[o + s] - big);
        l = fmaf(w, pl[o + s], l);
        a = fmaf(w, pa[(o + s) * kHeadDim + d], a);
      }
    }
    (hist_side ? accr_s : accw_s)[d] = a;
    if (d == 0) {
      scal_s[hist_side ? 0 : 2] = big;
      scal_s[hist_side ? 1 : 3] = l;
    }
    __syncthreads();
    if (tid < 128) {
      float oh = 0.f;
      const uint16_t* row = r_s + tid * kRowPad;
#pragma unroll 8
      for (int j = 0; j < kHeadDim; ++j) oh = fmaf(accr_s[j], bf16_to_f32(row[j]), oh);
      const float mh = scal_s[0], lh = scal_s[1], mw = scal_s[2], lw = scal_s[3];
      const float big2 = fmaxf(mh, mw);
      float res = 0.f;
      if (big2 != -INFINITY) {
        const float al = exp2f(mh - big2);
        const float be = exp2f(mw - big2);
        res = fmaf(al, oh, be * accw_s[tid]) / fmaf(al, lh, be * lw);
      }
      out[(static_cast<size_t>(b) * n_q + h) * kHeadDim + tid] = res;
    }
    __syncthreads();
  }
}

template <int GQ>
hipError_t launch(const LayerShape& L, const PartialsView& hist, int n_splits, const PartialsView& win,
                  int n_wsplits, const void* rot_v, float* out, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel<GQ>, dim3(L.n_kv, batch), dim3(256), 0, stream, hist.m, hist.l, hist.acc,
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
