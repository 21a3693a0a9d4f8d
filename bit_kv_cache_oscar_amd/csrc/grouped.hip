// Quantisation groups shorter than the head dimension (G = 64 or 32 rotated dims, one fp16
// scale and zero point per group): demotion (oscar_demote_grouped) and the INT2 history pass
// (oscar_decode_int2_grouped). The BF16 window pass and the merge are those of the one-group
// path, which take partials in the same format.
//
// Method: OSCAR; QbitAI article on OSCAR, section on aiming the rotation at attention: the
// bit-reversal in R makes the INT2 groups more balanced (the scale and zero point are per
// group); serving-path section: demotion rotates, clips, quantises and packs; the INT2 pass
// unpacks, dequantises with the scale and zero point and accumulates in floating point.
//
// Page layout of a head block (head_block_bytes<n_g>, n_g = 128 / G): the K and V codes as
// in the one-group layout (bytes 0..4095), then the K (s16, z16) of slot t, group g at
// 4096 + 4 (n_g t + g), then the V pairs the same way.
//
// Demotion: grouped_pass.h. INT2 pass: the one-group matrix-core pass of int2_pass.h with
// per-group K products, per-group P' weights and per-group zero-point sums (decode_int2.hip
// launches it).

#include "grouped_pass.h"

namespace oscar {
namespace {

template <int NG>
__global__ __launch_bounds__(256) void demote_grouped_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int n_kv,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ dst_slot, const uint16_t* __restrict__ rot_k,
    const uint16_t* __restrict__ rot_v, const float* __restrict__ clip_k, const float* __restrict__ clip_v,
    uint8_t* __restrict__ pool) {
  __shared__ __align__(16) unsigned char smem[demote::kGroupedSmemBytes];
  demote::demote_grouped_row<NG>(smem, blockIdx.x, k_src, v_src, n_kv, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v,
                                 pool);
}

template <int NG>
hipError_t launch_demote_grouped_ng(int n_kv, const void* k_src, const void* v_src, int n, const int32_t* dst_page,
                                    const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                                    const float* clip_k, const float* clip_v, void* pool, hipStream_t stream) {
  hipLaunchKernelGGL(demote_grouped_kernel<NG>, dim3(static_cast<unsigned>(2LL * n * n_kv)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), n_kv, dst_page,
                     dst_slot, static_cast<const uint16_t*>(rot_k), static_cast<const uint16_t*>(rot_v), clip_k,
                     clip_v, static_cast<uint8_t*>(pool));
  return hipGetLastError();
}

}  // namespace

size_t grouped_page_bytes(int n_kv, int group) { return static_cast<size_t>(n_kv) * (4096 + 512 * (kHeadDim / group)); }

hipError_t launch_demote_grouped(int n_kv, int group, const void* k_src, const void* v_src, int n,
                                 const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                                 const float* clip_k, const float* clip_v, void* pool, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  switch (group) {
    case 128: return launch_demote_grouped_ng<1>(n_kv, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool, stream);
    case 64: return launch_demote_grouped_ng<2>(n_kv, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool, stream);
    case 32: return launch_demote_grouped_ng<4>(n_kv, k_src, v_src, n, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_grouped(const LayerShape& L, int group, const void* q, const void* rot_k, const void* pool,
                                 const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch,
                                 float sm_scale, int n_splits, const PartialsView& out, hipStream_t stream) {
  return launch_decode_int2(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream,
                            group);
}

}  // namespace oscar
