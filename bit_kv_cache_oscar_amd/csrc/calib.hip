// Offline calibration statistics on the GPU (oscar_calib_covariances): the two covariances
// the per-head rotations are built from.
//
// Method: OSCAR; QbitAI article on OSCAR, section on aiming the rotation at attention: the
// key rotation comes from the query covariance Q^T Q and the value rotation from the
// score-weighted value covariance V^T S^T S V (S the attention scores), both estimated
// offline on calibration data; their eigenvectors give U in R = U * Hadamard * bit-reversal.
//
// Per layer:
//  1. attention outputs O_h = S_h V for every query head h, S_h the causal softmax of
//     sm_scale q_h k^T over the calibration sequence, in fp32 on the vector ALU: a workgroup
//     takes 16 query tokens of one head, flash-attention style on the matrix cores: keys and
//     values pass through LDS in tiles of 64, scores on bf16 MFMA (exact products, fp32 sums),
//     an online softmax in log2 units whose maximum moves once per tile, and the weighted
//     value sums on fp32 MFMA;
//  2. Gram sums Sigma[kv] = sum over (token t, query head h of the group) of x^T x, with
//     x = q[t, h] for the keys (bf16 MFMA) and x = O_h[t] for the values (fp32 MFMA): row
//     chunks staged transposed in LDS, 16 partial sums per KV head added in a fixed order, so
//     the result is deterministic and exactly symmetric.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 wbf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTileTokens = 16;  // query tokens per workgroup of the attention pass
constexpr int kKeyTile = 64;     // keys per LDS tile of the attention pass

// grid (ceil(T / 16), Hq), 256 threads (4 waves), for 16 query tokens of head blockIdx.y,
// flash-attention style on the matrix cores. Keys and values pass through LDS in tiles of 64
// (the next tile's loads issued before the current one is used). Per tile:
//   scores: wave w takes keys 16 w .. 16 w + 15; C[token][key] over the 128 dims in four
//     v_mfma_f32_16x16x32_bf16 (A = the tokens' query rows, B = the key rows; bf16 products
//     exact, fp32 sums); lane (g, n) holds tokens 4 g .. 4 g + 3 of key n;
//   the tokens' running maxima move once per tile (16-lane maxima, joined across the waves
//     through LDS); the weights go to LDS as fp32, their sums likewise;
//   values: wave w owns dims 32 w .. 32 w + 31 (two 16-dim tiles) and adds P V over the tile's
//     keys with v_mfma_f32_16x16x4_f32 (A = weights, B = value rows as fp32), after scaling
//     its running sums by the tokens' rescale factors.
__global__ __launch_bounds__(256) void calib_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int T, int n_q, int n_kv,
                                                         int gq, float scale_log2, float* __restrict__ out) {
  constexpr int kRow = kHeadDim / 8 + 1;  // 16-byte chunks per padded K row
  constexpr int kPRow = kKeyTile + 1;     // floats per padded weight row
  __shared__ uint4 k_s[kKeyTile][kRow];
  __shared__ uint16_t v_s[kKeyTile][kHeadDim + 8];
  __shared__ float p_s[kTileTokens][kPRow];
  __shared__ float wmax_s[4][kTileTokens];
  __shared__ float wsum_s[4][kTileTokens];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;  // MFMA lane group
  const int n = lane & 15;  // MFMA column
  const int h = blockIdx.y;
  const int kv = h / gq;
  const int t0 = blockIdx.x * kTileTokens;
  // query operand: token n, dims 32 s + 8 g .. + 7 for the four k-steps s
  uint4 qa[4];
  {
    const bool qv = t0 + n < T;
    const uint16_t* qrow = q + (static_cast<size_t>(t0 + n) * n_q + h) * kHeadDim + 8 * g;
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qa[st] = qv ? *reinterpret_cast<const uint4*>(qrow + 32 * st) : make_uint4(0u, 0u, 0u, 0u);
  }
  // keys 0 .. u_end - 1 cover every token of the tile (causal)
  const int u_end = min(T, t0 + kTileTokens);
  const size_t row_stride = static_cast<size_t>(n_kv) * kHeadDim;
  // loader role: thread (r, c) = (tid / 16, tid % 16) moves chunk c of keys r + 16 i, i < 4
  const int r = tid >> 4;
  const int c = tid & 15;
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
  static_assert(kKeyTile == 64 && kTileTokens == 16, "16 keys per wave, 16 tokens");
  // running state of tokens 4 g + i (the same in every wave: all compute it alike)
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  f32x4 o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};  // dims 32 wave + 16 dt + n
  CALIB_FETCH(0);
  for (int u0 = 0; u0 < u_end; u0 += kKeyTile) {
    __syncthreads();  // the previous tile, its weights and maxima are no longer read
    k_s[r][c] = lk0;
    k_s[r + 16][c] = lk1;
    k_s[r + 32][c] = lk2;
    k_s[r + 48][c] = lk3;
    *reinterpret_cast<uint4*>(&v_s[r][8 * c]) = lv0;
    *reinterpret_cast<uint4*>(&v_s[r + 16][8 * c]) = lv1;
    *reinterpret_cast<uint4*>(&v_s[r + 32][8 * c]) = lv2;
    *reinterpret_cast<uint4*>(&v_s[r + 48][8 * c]) = lv3;
    __syncthreads();
    if (u0 + kKeyTile < u_end) CALIB_FETCH(u0 + kKeyTile);  // uniform: in flight during this tile
    // scores of keys 16 wave + n for tokens 4 g + i
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(wbf16x8, qa[st]),
                                                  __builtin_bit_cast(wbf16x8, k_s[16 * wave + n][4 * st + g]), sc, 0, 0, 0);
    const int u = u0 + 16 * wave + n;
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      // causal mask and the end of the keys; tokens past T take key 0 only (never stored)
      const bool keep = u < u_end && (t < T ? (u <= t) : (u == 0));
      s[i] = keep ? sc[i] * scale_log2 : -INFINITY;
      const float wm = row16_max(s[i]);
      if (n == 0) wmax_s[wave][4 * g + i] = wm;
    }
    __syncthreads();
    float m_new[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * g + i;
      const float tm = fmaxf(fmaxf(wmax_s[0][tok], wmax_s[1][tok]), fmaxf(wmax_s[2][tok], wmax_s[3][tok]));
      m_new[i] = fmaxf(m[i], tm);  // finite: every token keeps key 0
      alpha[i] = __builtin_amdgcn_exp2f(m[i] - m_new[i]);
      const float p = __builtin_amdgcn_exp2f(s[i] - m_new[i]);
      p_s[tok][16 * wave + n] = p;
      const float ws = row16_sum(p);
      if (n == 0) wsum_s[wave][tok] = ws;
    }
    __syncthreads();  // weights and their sums are in LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * g + i;
      l[i] = fmaf(l[i], alpha[i], (wsum_s[0][tok] + wsum_s[1][tok]) + (wsum_s[2][tok] + wsum_s[3][tok]));
      m[i] = m_new[i];
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      f32x4 acc = o[dt];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha[i];
      const int d = 32 * wave + 16 * dt + n;
#pragma unroll
      for (int ks = 0; ks < kKeyTile / 4; ++ks) {
        const float a = p_s[n][4 * ks + g];
        const float b = __uint_as_float(static_cast<uint32_t>(v_s[4 * ks + g][d]) << 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
      }
      o[dt] = acc;
    }
  }
#undef CALIB_FETCH
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g + i;
    if (t >= T) continue;
    const float inv = 1.f / l[i];
    float* orow = out + (static_cast<size_t>(t) * n_q + h) * kHeadDim + 32 * wave + n;
    orow[0] = o[0][i] * inv;
    orow[16] = o[1][i] * inv;
  }
}

// Gram sums. Row rho = g + gq t (token t, head kv gq + g of the group) of x is at
// x + ((t n_q + kv gq + g) 128). Workgroup (kv, y) of grid (n_kv, kGramParts) takes row chunks
// y, y + kGramParts, ... of kChunk rows, each staged transposed in LDS (column i of the chunk
// as one contiguous LDS row), and sums x^T x of its chunks on the matrix cores: wave w owns
// output tiles 16 w .. 16 w + 15 of the 8 x 8 tiles of 16 x 16 (lane (g, n) ends with
// rows 4 g + e, column n of each tile). Its partial goes to part[y][kv]; calib_gram_reduce
// adds the kGramParts partials in order (deterministic; entry (j, i) sums the same products
// in the same order as (i, j), so the result is exactly symmetric).
constexpr int kGramParts = 32;

template <typename In>
struct GramCfg;
template <>
struct GramCfg<uint16_t> {  // bf16 rows: v_mfma_f32_16x16x32_bf16, 32 rows per step
  static constexpr int kChunk = 256;
  static constexpr int kPad = 8;
};
template <>
struct GramCfg<float> {  // fp32 rows: v_mfma_f32_16x16x4_f32, 4 rows per step
  static constexpr int kChunk = 64;
  static constexpr int kPad = 4;
};

template <typename In>
__global__ __launch_bounds__(256) void calib_gram_kernel(const In* __restrict__ x, int T, int n_q, int gq,
                                                         float* __restrict__ part) {
  constexpr int kChunk = GramCfg<In>::kChunk;
  constexpr int kLd = kChunk + GramCfg<In>::kPad;  // elements per transposed LDS row
  __shared__ __align__(16) In xt[kHeadDim * kLd];  // xt[col * kLd + row]
  const int kv = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int rows = T * gq;
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = blockIdx.y * kChunk; c0 < rows; c0 += kGramParts * kChunk) {
    __syncthreads();  // the previous chunk is no longer read
    // stage: the threads of a row group copy one row's 16-byte pieces each (coalesced), rows
    // past the end as zeros
    constexpr int kPer = 16 / static_cast<int>(sizeof(In));  // elements per 16-byte piece
    constexpr int kTpr = kHeadDim / kPer;                      // threads per row
    const int piece = tid % kTpr;
#pragma unroll 4
    for (int rr = tid / kTpr; rr < kChunk; rr += 256 / kTpr) {
      const int rho = c0 + rr;
      const bool in = rho < rows;
      const int t = in ? rho / gq : 0;
      const In* row = x + (static_cast<size_t>(t) * n_q + kv * gq + (in ? rho - t * gq : 0)) * kHeadDim;
      const uint4 w = in ? *reinterpret_cast<const uint4*>(row + kPer * piece) : make_uint4(0u, 0u, 0u, 0u);
      const In* e = reinterpret_cast<const In*>(&w);
#pragma unroll
      for (int i = 0; i < kPer; ++i) xt[(kPer * piece + i) * kLd + rr] = e[i];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int tile = 16 * wave + j;
      const In* ar = xt + (16 * (tile >> 3) + n) * kLd;
      const In* br = xt + (16 * (tile & 7) + n) * kLd;
      if constexpr (sizeof(In) == 2) {
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks) {
          const uint4 a = *reinterpret_cast<const uint4*>(ar + 32 * ks + 8 * g);
          const uint4 b = *reinterpret_cast<const uint4*>(br + 32 * ks + 8 * g);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(wbf16x8, a), __builtin_bit_cast(wbf16x8, b),
                                                          acc[j], 0, 0, 0);
        }
      } else {
#pragma unroll 8
        for (int ks = 0; ks < kChunk / 4; ++ks)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[4 * ks + g], br[4 * ks + g], acc[j], 0, 0, 0);
      }
    }
  }
  float* out = part + (static_cast<size_t>(blockIdx.y) * gridDim.x + kv) * kHeadDim * kHeadDim;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int tile = 16 * wave + j;
    float* o = out + (16 * (tile >> 3) + 4 * g) * kHeadDim + 16 * (tile & 7) + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e * kHeadDim] = acc[j][e];
  }
}

// sigma[kv] = sum over p of part[p][kv], p in order; grid (n_kv, 64), 256 threads
__global__ __launch_bounds__(256) void calib_gram_reduce(const float* __restrict__ part, int n_kv,
                                                         float* __restrict__ sigma) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kHeadDim * kHeadDim + blockIdx.y * 256 + threadIdx.x;
  const size_t stride = static_cast<size_t>(n_kv) * kHeadDim * kHeadDim;
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < kGramParts; ++p) s += part[p * stride + i];
  sigma[i] = s;
}

}  // namespace

size_t calib_workspace_bytes(int T, int n_q, int n_kv) {
  // attention outputs, then the partial Gram sums
  return static_cast<size_t>(T) * n_q * kHeadDim * sizeof(float) +
         static_cast<size_t>(kGramParts) * n_kv * kHeadDim * kHeadDim * sizeof(float);
}

hipError_t launch_calib(const LayerShape& L, const void* q, const void* k, const void* v, int T, float sm_scale,
                        float* work, float* sigma_k, float* sigma_v, hipStream_t stream) {
  const float scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  float* o_work = work;
  float* part = work + static_cast<size_t>(T) * L.n_q * kHeadDim;
  hipLaunchKernelGGL(calib_gram_kernel<uint16_t>, dim3(L.n_kv, kGramParts), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), T, L.n_q, L.gq, part);
  hipLaunchKernelGGL(calib_gram_reduce, dim3(L.n_kv, 64), dim3(256), 0, stream, part, L.n_kv, sigma_k);
  hipLaunchKernelGGL(calib_attn_kernel, dim3((T + kTileTokens - 1) / kTileTokens, L.n_q), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), T, L.n_q, L.n_kv, L.gq, scale_log2, o_work);
  hipLaunchKernelGGL(calib_gram_kernel<float>, dim3(L.n_kv, kGramParts), dim3(256), 0, stream,
                     static_cast<const float*>(o_work), T, L.n_q, L.gq, part);
  hipLaunchKernelGGL(calib_gram_reduce, dim3(L.n_kv, 64), dim3(256), 0, stream, part, L.n_kv, sigma_v);
  return hipGetLastError();
}

}  // namespace oscar
