// Offline calibration statistics on the GPU (oscar_calib_covariances): the two covariances
// the per-head rotations are built from.
//
// Method: OSCAR; QbitAI article on OSCAR, section on aiming the rotation at attention: the
// key rotation comes from the query covariance Q^T Q and the value rotation from the
// score-weighted value covariance V^T S^T S V (S the attention scores), both estimated
// offline on calibration data; their eigenvectors give U in R = U * Hadamard * bit-reversal.
//
// Two launches per layer:
//  1. attention outputs O_h = S_h V for every query head h, S_h the causal softmax of
//     sm_scale q_h k^T over the calibration sequence, in fp32 on the vector ALU: a workgroup
//     takes 16 query tokens of one head; keys and values pass through LDS in tiles of 64,
//     each thread scoring four keys (bf16 products are exact in fp32), with an online softmax
//     in log2 units whose maximum moves once per tile;
//  2. Gram sums Sigma[kv] = sum over (token t, query head h of the group) of x^T x, with
//     x = q[t, h] for the keys and x = O_h[t] for the values, on v_mfma_f32_16x16x4_f32: one
//     workgroup per 16x16 output tile, its four waves summing quarters of the rows in a fixed
//     order, so the result is deterministic and exactly symmetric.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileTokens = 16;  // query tokens per workgroup of the attention pass
constexpr int kKeyTile = 64;     // keys per LDS tile of the attention pass

__device__ __forceinline__ void bf16x8_to_f32(const uint4& w, float* out) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(a[i] << 16);
    out[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
  }
}

// grid (ceil(T / 16), Hq), 256 threads, for 16 query tokens of head blockIdx.y. Keys and
// values pass through LDS in tiles of 64 (rows padded to 17 16-byte chunks, so the 16 rows a
// score step reads lie in distinct banks); the next tile's loads are issued before the current
// tile is used. Per tile, thread (token, k) = (tid / 16, tid % 16):
//   scores of keys k, k + 16, k + 32, k + 48 (four independent 128-term fp32 dot products);
//   the token's running maximum and sum move once per tile (16-lane reductions);
//   its weights go to LDS, and the thread then adds the tile's weighted values of dims
//   8k .. 8k + 7 to its running sums.
__global__ __launch_bounds__(256) void calib_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int T, int n_q, int n_kv,
                                                         int gq, float scale_log2, float* __restrict__ out) {
  constexpr int kRow = kHeadDim / 8 + 1;  // 16-byte chunks per padded LDS row
  __shared__ uint4 k_s[kKeyTile][kRow];
  __shared__ uint4 v_s[kKeyTile][kRow];
  __shared__ uint4 q_s[kTileTokens][kRow];
  __shared__ float p_s[kTileTokens][kKeyTile];
  const int r = threadIdx.x >> 4;  // token of the tile (score and value steps alike)
  const int c = threadIdx.x & 15;  // key offset (scores), 16-byte chunk of dims (values)
  const int h = blockIdx.y;
  const int kv = h / gq;
  const int t = blockIdx.x * kTileTokens + r;
  const bool valid = t < T;
  q_s[r][c] = valid ? *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(t) * n_q + h) * kHeadDim + 8 * c)
                    : make_uint4(0u, 0u, 0u, 0u);
  // keys 0 .. u_end - 1 cover every token of the tile (causal)
  const int u_end = min(T, static_cast<int>(blockIdx.x) * kTileTokens + kTileTokens);
  const size_t row_stride = static_cast<size_t>(n_kv) * kHeadDim;
  // loader role: thread (r, c) moves chunk c of keys r + 16 i, i < 4, of K and V
  const uint16_t* kbase = k + static_cast<size_t>(kv) * kHeadDim + 8 * c;
  const uint16_t* vbase = v + static_cast<size_t>(kv) * kHeadDim + 8 * c;
  uint4 lk0, lk1, lk2, lk3, lv0, lv1, lv2, lv3;
#define CALIB_FETCH(U0)                                                                           \
  do {                                                                                           \
    const int ub = (U0) + r;                                                                     \
    /* past the end: the last key again, masked below */                                         \
    lk0 = *reinterpret_cast<const uint4*>(kbase + min(ub, u_end - 1) * row_stride);              \
    lk1 = *reinterpret_cast<const uint4*>(kbase + min(ub + 16, u_end - 1) * row_stride);         \
    lk2 = *reinterpret_cast<const uint4*>(kbase + min(ub + 32, u_end - 1) * row_stride);         \
    lk3 = *reinterpret_cast<const uint4*>(kbase + min(ub + 48, u_end - 1) * row_stride);         \
    lv0 = *reinterpret_cast<const uint4*>(vbase + min(ub, u_end - 1) * row_stride);              \
    lv1 = *reinterpret_cast<const uint4*>(vbase + min(ub + 16, u_end - 1) * row_stride);         \
    lv2 = *reinterpret_cast<const uint4*>(vbase + min(ub + 32, u_end - 1) * row_stride);         \
    lv3 = *reinterpret_cast<const uint4*>(vbase + min(ub + 48, u_end - 1) * row_stride);         \
  } while (0)
  static_assert(kKeyTile == 64 && kTileTokens == 16, "four keys per thread and tile, 16 tokens");
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  CALIB_FETCH(0);
  for (int u0 = 0; u0 < u_end; u0 += kKeyTile) {
    __syncthreads();  // the previous tile (and its weights) are no longer read
    k_s[r][c] = lk0;
    k_s[r + 16][c] = lk1;
    k_s[r + 32][c] = lk2;
    k_s[r + 48][c] = lk3;
    v_s[r][c] = lv0;
    v_s[r + 16][c] = lv1;
    v_s[r + 32][c] = lv2;
    v_s[r + 48][c] = lv3;
    __syncthreads();
    if (u0 + kKeyTile < u_end) CALIB_FETCH(u0 + kKeyTile);  // uniform: in flight during this tile
    // scores of keys c + 16 j (bf16 products exact in fp32)
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ch = 0; ch < kHeadDim / 8; ++ch) {
      float qf[8];
      bf16x8_to_f32(q_s[r][ch], qf);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float kf[8];
        bf16x8_to_f32(k_s[c + 16 * j][ch], kf);
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[j] = fmaf(qf[i], kf[i], sc[j]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = u0 + c + 16 * j;
      // causal mask and the end of the keys; tokens past T take key 0 only (never stored)
      const bool keep = u < u_end && (valid ? (u <= t) : (u == 0));
      sc[j] = keep ? sc[j] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sc[j]);
    }
    const float m_new = fmaxf(m, row16_max(tmax));  // finite: every token keeps key 0
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(sc[j] - m_new);
      p_s[r][c + 16 * j] = p;
      ps += p;
    }
    l = fmaf(l, alpha, row16_sum(ps));
    m = m_new;
    __syncthreads();  // the token's weights are in LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    const int n_keys = min(kKeyTile, u_end - u0);
#pragma unroll 4
    for (int j = 0; j < n_keys; ++j) {
      float vf[8];
      bf16x8_to_f32(v_s[j][c], vf);
      const float p = p_s[r][j];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
  }
#undef CALIB_FETCH
  if (!valid) return;
  const float inv = 1.f / l;
  float4* o = reinterpret_cast<float4*>(out + (static_cast<size_t>(t) * n_q + h) * kHeadDim + 8 * c);
  o[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  o[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
}

__device__ __forceinline__ float load_f32(const uint16_t* p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
__device__ __forceinline__ float load_f32(const float* p) { return *p; }

// grid (n_kv, 64), 256 threads: workgroup y owns output tile y of the 8 x 8 tiles of
// 16 x 16, and wave w sums the rows of quarter w of the row range. Row rho = g + gq t
// (token t, head kv gq + g) of x is at x + ((t n_q + kv gq + g) 128). Lane (g4, n) feeds row
// 4 i + g4 of MFMA step i: column i0 + n to A and j0 + n to B, and ends with the partial of
// sigma[i0 + 4 g4 + e][j0 + n] in element e; the four quarters are added in order through
// LDS (deterministic, and exactly symmetric: entry (j, i) sums the same products in the
// same order).
template <typename In>
__global__ __launch_bounds__(256) void calib_gram_kernel(const In* __restrict__ x, int T, int n_q, int gq,
                                                         float* __restrict__ sigma) {
  __shared__ f32x4 part[3][64];
  const int kv = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i0 = 16 * (blockIdx.y >> 3);
  const int j0 = 16 * (blockIdx.y & 7);
  const int g4 = lane >> 4;
  const int n = lane & 15;
  const int rows = T * gq;
  const int quarter = ((rows + 15) / 16) * 4;  // rows per wave, a multiple of 4
  const int r_begin = wave * quarter;
  const int r_end = min(rows, r_begin + quarter);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kUnroll = 8;
  for (int base = r_begin; base < r_end; base += 4 * kUnroll) {
    float a[kUnroll], b[kUnroll];
#pragma unroll
    for (int s = 0; s < kUnroll; ++s) {
      const int rho = base + 4 * s + g4;
      a[s] = b[s] = 0.f;
      if (rho < r_end) {
        const int t = rho / gq;
        const In* row = x + (static_cast<size_t>(t) * n_q + kv * gq + (rho - t * gq)) * kHeadDim;
        a[s] = load_f32(row + i0 + n);
        b[s] = load_f32(row + j0 + n);
      }
    }
#pragma unroll
    for (int s = 0; s < kUnroll; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  }
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += part[w][lane];
  float* out = sigma + (static_cast<size_t>(kv) * kHeadDim + i0 + 4 * g4) * kHeadDim + j0 + n;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e * kHeadDim] = acc[e];
}

}  // namespace

hipError_t launch_calib(const LayerShape& L, const void* q, const void* k, const void* v, int T, float sm_scale,
                        float* o_work, float* sigma_k, float* sigma_v, hipStream_t stream) {
  const float scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  hipLaunchKernelGGL(calib_gram_kernel<uint16_t>, dim3(L.n_kv, 64), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), T, L.n_q, L.gq, sigma_k);
  hipLaunchKernelGGL(calib_attn_kernel, dim3((T + kTileTokens - 1) / kTileTokens, L.n_q), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), T, L.n_q, L.n_kv, L.gq, scale_log2, o_work);
  hipLaunchKernelGGL(calib_gram_kernel<float>, dim3(L.n_kv, 64), dim3(256), 0, stream,
                     static_cast<const float*>(o_work), T, L.n_q, L.gq, sigma_v);
  return hipGetLastError();
}

}  // namespace oscar
