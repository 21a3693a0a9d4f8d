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
//     takes 16 query tokens of one head, 16 lanes per token with 8 dims each (bf16 products
//     are exact in fp32); keys and values pass through LDS in tiles of 64 and are walked in
//     order with an online softmax in log2 units;
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

// grid (ceil(T / 16), Hq), 256 threads: thread (r, c) = (tid / 16, tid % 16) holds dims
// 8c..8c+7 of query token 16 blockIdx.x + r of head blockIdx.y. Keys and values come in
// tiles of 64 tokens staged in LDS (one round of loads per tile, the next tile's loads
// issued before the current tile is used).
__global__ __launch_bounds__(256) void calib_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int T, int n_q, int n_kv,
                                                         int gq, float scale_log2, float* __restrict__ out) {
  __shared__ uint4 kv_s[2][kKeyTile][kHeadDim / 8];  // [K, V][key][16-byte chunk]
  const int r = threadIdx.x >> 4;
  const int c = threadIdx.x & 15;
  const int h = blockIdx.y;
  const int kv = h / gq;
  const int t = blockIdx.x * kTileTokens + r;
  const bool valid = t < T;
  float qd[8];
  {
    uint4 w = {0u, 0u, 0u, 0u};
    if (valid) w = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(t) * n_q + h) * kHeadDim + 8 * c);
    bf16x8_to_f32(w, qd);
#pragma unroll
    for (int i = 0; i < 8; ++i) qd[i] *= scale_log2;  // scores in log2 units
  }
  // keys 0 .. u_end - 1 cover every token of the tile (causal)
  const int u_end = min(T, static_cast<int>(blockIdx.x) * kTileTokens + kTileTokens);
  const size_t row_stride = static_cast<size_t>(n_kv) * kHeadDim;
  // loader role: thread (r, c) moves chunk c of keys r + 16 i, i < 4, of K and V
  const uint16_t* kbase = k + static_cast<size_t>(kv) * kHeadDim + 8 * c;
  const uint16_t* vbase = v + static_cast<size_t>(kv) * kHeadDim + 8 * c;
  uint4 lk0, lk1, lk2, lk3, lv0, lv1, lv2, lv3;  // the next tile's rows r, r + 16, r + 32, r + 48
#define CALIB_FETCH(U0)                                                                           \
  do {                                                                                           \
    const int ub = (U0) + r;                                                                     \
    /* past the end: the last key again, masked in the loop */                                   \
    lk0 = *reinterpret_cast<const uint4*>(kbase + min(ub, u_end - 1) * row_stride);              \
    lk1 = *reinterpret_cast<const uint4*>(kbase + min(ub + 16, u_end - 1) * row_stride);         \
    lk2 = *reinterpret_cast<const uint4*>(kbase + min(ub + 32, u_end - 1) * row_stride);         \
    lk3 = *reinterpret_cast<const uint4*>(kbase + min(ub + 48, u_end - 1) * row_stride);         \
    lv0 = *reinterpret_cast<const uint4*>(vbase + min(ub, u_end - 1) * row_stride);              \
    lv1 = *reinterpret_cast<const uint4*>(vbase + min(ub + 16, u_end - 1) * row_stride);         \
    lv2 = *reinterpret_cast<const uint4*>(vbase + min(ub + 32, u_end - 1) * row_stride);         \
    lv3 = *reinterpret_cast<const uint4*>(vbase + min(ub + 48, u_end - 1) * row_stride);         \
  } while (0)
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  static_assert(kKeyTile == 64, "four rows per thread and tile");
  CALIB_FETCH(0);
  for (int u0 = 0; u0 < u_end; u0 += kKeyTile) {
    __syncthreads();  // the previous tile is no longer read
    kv_s[0][r][c] = lk0;
    kv_s[0][r + 16][c] = lk1;
    kv_s[0][r + 32][c] = lk2;
    kv_s[0][r + 48][c] = lk3;
    kv_s[1][r][c] = lv0;
    kv_s[1][r + 16][c] = lv1;
    kv_s[1][r + 32][c] = lv2;
    kv_s[1][r + 48][c] = lv3;
    __syncthreads();
    if (u0 + kKeyTile < u_end) CALIB_FETCH(u0 + kKeyTile);  // uniform: in flight during this tile
    const int n_keys = min(kKeyTile, u_end - u0);
    // eight keys at a time: their scores are independent, and the running maximum and the
    // rescaling of the sums move once per eight keys
    for (int jb = 0; jb < n_keys; jb += 8) {
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        float kd[8];
        bf16x8_to_f32(kv_s[0][jb + jj][c], kd);
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = fmaf(qd[i], kd[i], d);
        sc[jj] = d;
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sc[jj] = row16_sum(sc[jj]);
      float bm = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int u = u0 + jb + jj;
        // causal mask and the tile's end; tokens past T take key 0 only (never stored)
        const bool keep = (jb + jj < n_keys) && (valid ? (u <= t) : (u == 0));
        sc[jj] = keep ? sc[jj] : -INFINITY;
        bm = fmaxf(bm, sc[jj]);
      }
      const float m_new = fmaxf(m, bm);
      if (m_new == -INFINITY) continue;  // nothing seen yet (uniform per token row)
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        float vd[8];
        bf16x8_to_f32(kv_s[1][jb + jj][c], vd);
        const float p = __builtin_amdgcn_exp2f(sc[jj] - m_new);
        l += p;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(p, vd[i], acc[i]);
      }
      m = m_new;
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
