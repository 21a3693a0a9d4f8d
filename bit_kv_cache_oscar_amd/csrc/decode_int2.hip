// Standalone INT2 history pass (oscar_decode_int2, and oscar_decode_int2_grouped over pages
// with two or four quantisation groups per vector): query preparation, then one workgroup
// per (history split, KV head x head group, request). The device code, and the method it
// follows, is in int2_pass.h.

#include "int2_pass.h"

namespace oscar {
namespace {

__global__ __launch_bounds__(256) void qprep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ rot_k,
                                                    int n_q, int gq, double scale_log2, char* __restrict__ qlimb,
                                                    QueryScal* __restrict__ qscal) {
  __shared__ __align__(16) unsigned char smem[int2::kQprepSmem];
  int2::qprep_head(smem, q, rot_k, n_q, gq, scale_log2, qlimb, qscal, blockIdx.x, blockIdx.y);
}

template <int GQ, int NG>
__global__ __launch_bounds__(256) void decode_int2_kernel(
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ hist_len, int n_q, int n_kv, int n_groups, int n_splits,
    const char* __restrict__ qlimb, const QueryScal* __restrict__ qscal, float* __restrict__ out_m,
    float* __restrict__ out_l, float* __restrict__ out_acc) {
  __shared__ __align__(16) unsigned char smem[int2::int2_smem_bytes<GQ, int2::kWaves, NG>()];
  int2::int2_split<GQ, false, int2::kWaves, false, false, NG>(smem, blockIdx.x, blockIdx.y, blockIdx.z, pool,
                                                              block_table, max_pages, hist_len, n_q, n_kv, n_groups,
                                                              n_splits, qlimb, qscal, out_m, out_l, out_acc);
}

template <int GQ, int NG>
hipError_t launch(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                  const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch,
                  float sm_scale, int n_splits, const PartialsView& out, hipStream_t stream) {
  const int n_groups = L.gq / GQ;
  const double scale_log2 = static_cast<double>(sm_scale) * 1.4426950408889634;
  hipLaunchKernelGGL(qprep_kernel, dim3(L.n_q, batch), dim3(256), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(rot_k), L.n_q, L.gq, scale_log2, out.qlimb, out.qscal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_int2_kernel<GQ, NG>), dim3(n_splits, L.n_kv * n_groups, batch), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(pool), block_table, max_pages, hist_len, L.n_q, L.n_kv, n_groups,
                     n_splits, out.qlimb, out.qscal, out.m, out.l, out.acc);
  return hipGetLastError();
}

template <int NG>
hipError_t launch_ng(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                     const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch, float sm_scale,
                     int n_splits, const PartialsView& out, hipStream_t stream) {
  switch (L.gq) {
    case 1: return launch<1, NG>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 2: return launch<2, NG>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 4: return launch<4, NG>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    // with groups, head tiles of four: the per-group metadata leaves no registers for two
    case 8: return launch<NG == 1 ? 8 : 4, NG>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 16: return launch<NG == 1 ? 8 : 4, NG>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_int2(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                              const int32_t* block_table, int max_pages, const int32_t* hist_len,
                              int batch, float sm_scale, int n_splits, const PartialsView& out,
                              hipStream_t stream, int group) {
  switch (group) {
    case 128: return launch_ng<1>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 64: return launch_ng<2>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 32: return launch_ng<4>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
