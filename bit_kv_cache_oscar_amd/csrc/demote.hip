// Demotion of recent-window tokens into the INT2 history (rotate, clip, quantise, pack).
//
// Method: OSCAR (Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
// Quantization); QbitAI article on OSCAR, serving-path section: the oldest recent token
// is rotated, clipped, quantised and packed four 2-bit codes per byte into the INT2
// history, with a scale and zero point per group.
//
// One workgroup of 128 threads handles one row (token, KV head, K or V) with its rotation
// staged in LDS; thread j owns output dim j. The rotation is accumulated in fp64
// with a compensated (two-sum) chain over exact bf16 x bf16 products, so the group
// extremes, and from them the fp16 scale and zero point, come from the dot product's
// fp64 value; the scale/zero arithmetic is fp64 exactly as specified.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

__device__ __forceinline__ void two_sum_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  c += (s - (t - bp)) + (p - bp);
  s = t;
}

__global__ __launch_bounds__(128) void demote_rows_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int n_kv,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ dst_slot,
    const uint16_t* __restrict__ rot_k, const uint16_t* __restrict__ rot_v,
    const float* __restrict__ clip_k, const float* __restrict__ clip_v, uint8_t* __restrict__ pool) {
  // every product and sum below is rounded on its own, as the quantiser specifies
#pragma clang fp contract(off)
  __shared__ __align__(16) uint16_t r_s[kHeadDim * kHeadDim];
  __shared__ double xs[kHeadDim];
  __shared__ double red_max[2];
  __shared__ double red_min[2];
  __shared__ uint8_t codes_s[kHeadDim];

  const int row = blockIdx.x >> 1;  // token * n_kv + head
  const int is_v = blockIdx.x & 1;
  const int tok = row / n_kv;
  const int head = row - tok * n_kv;
  const int j = threadIdx.x;
  const int wave = threadIdx.x >> 6;

  const uint16_t* src = (is_v ? v_src : k_src) + static_cast<size_t>(row) * kHeadDim;
  stage_rotation(r_s, (is_v ? rot_v : rot_k) + static_cast<size_t>(head) * kHeadDim * kHeadDim, j, 128);
  xs[j] = bf16_to_f64(src[j]);
  __syncthreads();

  // four independent compensated chains (for latency), joined by the same two-sum
  double s[4] = {0.0, 0.0, 0.0, 0.0}, c[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
  for (int i = 0; i < kHeadDim; i += 4)
#pragma unroll
    for (int u = 0; u < 4; ++u) two_sum_add(s[u], c[u], xs[i + u] * bf16_to_f64(r_s[(i + u) * kHeadDim + j]));
  double st = s[0], ct = c[0] + c[1] + c[2] + c[3];
  two_sum_add(st, ct, s[1]);
  two_sum_add(st, ct, s[2]);
  two_sum_add(st, ct, s[3]);
  const double y = st + ct;

  const double wmax = wave_max(y);
  const double wmin = wave_min(y);
  if ((threadIdx.x & 63) == 0) {
    red_max[wave] = wmax;
    red_min[wave] = wmin;
  }
  __syncthreads();
  const double ymax = fmax(red_max[0], red_max[1]);
  const double ymin = fmin(red_min[0], red_min[1]);

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
  if (j == 0) {
    uint32_t* meta = reinterpret_cast<uint32_t*>(blk + (is_v ? kVMeta : kKMeta) + 4 * slot);
    *meta = static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16);
  }
  if (is_v) {
    // V codes are dim-major: this dim's word for slots 16u..16u+15 is shared with other
    // tokens, so clear and set only this slot's two bits.
    const int r = slot & 15;
    const int sh = 8 * (r & 3) + 2 * (r >> 2);
    uint32_t* w = reinterpret_cast<uint32_t*>(blk + v_word_offset(j, slot >> 4));
    atomicAnd(w, ~(3u << sh));
    atomicOr(w, static_cast<uint32_t>(code) << sh);
    return;
  }
  codes_s[j] = static_cast<uint8_t>(code);
  __syncthreads();
  if (j < 8) {
    // K word w holds dims 16w..16w+15, dim 16w+4m+jj at bits 8jj+2m.
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        word |= static_cast<uint32_t>(codes_s[16 * j + 4 * m + jj]) << (8 * jj + 2 * m);
    *reinterpret_cast<uint32_t*>(blk + k_word_offset(slot, j)) = word;
  }
}

}  // namespace

hipError_t launch_demote_rows(const LayerShape& L, const void* k_src, const void* v_src, int n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k,
                              const void* rot_v, const float* clip_k, const float* clip_v, void* pool,
                              hipStream_t stream) {
  const long long rows = static_cast<long long>(n) * L.n_kv;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(demote_rows_kernel, dim3(static_cast<unsigned>(2 * rows)), dim3(128), 0, stream,
                     static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), L.n_kv,
                     dst_page, dst_slot, static_cast<const uint16_t*>(rot_k),
                     static_cast<const uint16_t*>(rot_v), clip_k, clip_v, static_cast<uint8_t*>(pool));
  return hipGetLastError();
}

}  // namespace oscar
