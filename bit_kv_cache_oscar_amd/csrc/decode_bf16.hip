// Standalone BF16 window pass (oscar_decode_bf16): one workgroup per (window split, KV
// head, request). The device code, and the method it follows, is in window_pass.h.

#include "window_pass.h"

namespace oscar {
namespace {

template <int GQ>
__global__ __launch_bounds__(256) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_win, const uint16_t* __restrict__ v_win,
    const int32_t* __restrict__ win_len, int n_q, int n_kv, int window, int n_wsplits, double scale_log2,
    float* __restrict__ out_m, float* __restrict__ out_l, float* __restrict__ out_acc) {
  __shared__ __align__(16) unsigned char smem[window::window_smem_bytes<GQ>()];
  window::window_split<GQ>(smem, blockIdx.x, blockIdx.y, blockIdx.y * GQ, blockIdx.z, q, k_win, v_win, win_len, n_q,
                           n_kv, window, n_wsplits, scale_log2, out_m, out_l, out_acc);
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
