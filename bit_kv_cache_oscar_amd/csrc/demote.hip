// Standalone demotion (oscar_demote): one 256-thread workgroup per (token, KV head, K or
// V). The device code, and the method it follows, is in demote_pass.h.

#include "demote_pass.h"

namespace oscar {
namespace {

__global__ __launch_bounds__(256) void demote_rows_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int n_kv,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ dst_slot,
    const uint16_t* __restrict__ rot_k, const uint16_t* __restrict__ rot_v,
    const float* __restrict__ clip_k, const float* __restrict__ clip_v, uint8_t* __restrict__ pool,
    const uint32_t* __restrict__ codebook) {
  __shared__ __align__(16) unsigned char smem[demote::kSmemBytes];
  demote::demote_row(smem, blockIdx.x, k_src, v_src, n_kv, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool,
                     codebook);
}

}  // namespace

hipError_t launch_demote_rows(const LayerShape& L, const void* k_src, const void* v_src, int n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k,
                              const void* rot_v, const float* clip_k, const float* clip_v, void* pool,
                              hipStream_t stream, const uint32_t* codebook) {
  const long long rows = static_cast<long long>(n) * L.n_kv;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(demote_rows_kernel, dim3(static_cast<unsigned>(2 * rows)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), L.n_kv,
                     dst_page, dst_slot, static_cast<const uint16_t*>(rot_k),
                     static_cast<const uint16_t*>(rot_v), clip_k, clip_v, static_cast<uint8_t*>(pool), codebook);
  return hipGetLastError();
}

}  // namespace oscar
