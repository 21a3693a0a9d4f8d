// BF16 sink/recent pass of decode attention: device code shared by the standalone window
// kernel and the fused decode kernels.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the sink (first 64
// tokens) and the recent window (last 256 tokens) stay in BF16 and are handled by a BF16
// kernel, separately from the INT2 history.
//
// A workgroup serves one (window split of 64 slots, KV head, request) with 4 waves. Every
// global read (K and V of the split's slots, the query heads, the window length) is
// issued before any arithmetic, so the pass waits on memory once. Wave w scores slots
// 16w..16w+15 against the KV head's query heads on the matrix cores (bf16 x bf16 products
// are exact, sums in fp32: 16 slots x 16 head columns x 128 dims in four
// v_mfma_f32_16x16x32_bf16), then the per-head maximum and weights, and the value sum on
// the vector units, thread (dim pair, 16-slot group).

#pragma once

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace window {

typedef float wf32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 wbf16x8 __attribute__((ext_vector_type(8)));

// LDS: per-wave head maxima and sums [4][16], weights [GQ][64], value partials [4][GQ][128]
template <int GQ>
constexpr int window_smem_bytes() {
  return 4 * (2 * 4 * 16 + GQ * kPageTokens + 4 * GQ * kHeadDim);
}

// One workgroup of the BF16 window pass: slots 64 c .. 64 c + 63 of KV head kv of request b
// for its query heads h0 .. h0 + GQ - 1 (GQ <= 16; the KV head's heads, or a group of them
// when several workgroups share a KV head). `smem` holds window_smem_bytes<GQ>(). The pass
// uses four waves; a workgroup of NWB waves (4 or 8) lets the others pass its barriers
// idle, or with kDual (8 waves) runs split c + 1 on them (smem then holds twice as much; a
// half past the last split does nothing). kCoherent: the partial goes out with agent-scope
// stores (for a merge inside the same launch).
template <int GQ, int NWB = 4, bool kCoherent = false, bool kDual = false>
__device__ __forceinline__ void window_split(
    unsigned char* __restrict__ smem, int c, int kv, int h0, int b, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_win, const uint16_t* __restrict__ v_win,
    const int32_t* __restrict__ win_len, int n_q, int n_kv, int window, int n_wsplits, double scale_log2,
    float* __restrict__ out_m, float* __restrict__ out_l, float* __restrict__ out_acc, int gqv = GQ, int nqt = 1) {
  static_assert(GQ >= 1 && GQ <= 16, "one 16-column score tile holds the KV head's query heads");
  static_assert(!kDual || NWB == 8, "two splits need eight waves");
  // with kDual, waves 4..7 run split c + 1 as a pass of their own
  const int half = kDual ? static_cast<int>(threadIdx.x >> 8) : 0;
  c += half;
  smem += half * window_smem_bytes<GQ>();
  float(*mx_s)[16] = reinterpret_cast<float(*)[16]>(smem);
  float(*l_s)[16] = reinterpret_cast<float(*)[16]>(smem + 4 * 64);
  float(*p_s)[kPageTokens] = reinterpret_cast<float(*)[kPageTokens]>(smem + 4 * 128);
  float(*acc_s)[GQ][kHeadDim] = reinterpret_cast<float(*)[GQ][kHeadDim]>(smem + 4 * 128 + 4 * GQ * kPageTokens);
  static_assert(NWB == 4 || NWB == 8, "4 or 8 waves");
  const int tid = kDual ? static_cast<int>(threadIdx.x & 255) : static_cast<int>(threadIdx.x);  // within the pass
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // wave-uniform: the waves that do a pass (with kDual, both halves while their split exists)
  const bool act = (NWB == 4 || kDual || wave < 4) && c < n_wsplits;
  const int t0 = c * kPageTokens;
  const size_t base = ((static_cast<size_t>(b) * n_kv + kv) * window + t0) * kHeadDim;
  // the window length first: the score mask needs it as soon as K and q have arrived
  const int wl = min(win_len[b], window);
  const int ntok = max(0, min(kPageTokens, wl - t0));

  // ---- every read, issued up front. Slots past the window length are read too (they lie
  // in the window buffer) and masked below.
  // score operands: lane (r, g) = (lane & 15, lane >> 4) holds dims 32s + 8g .. 32s + 8g + 7
  // of slot 16 wave + r (A) and of query head r (B, zero past GQ)
  const int r = lane & 15;
  const int g = lane >> 4;
  const int kslot = 16 * wave + r;
  // slots of this split that head r sees: query token t of a multi-query decode sees the
  // window up to its own position, nqt - 1 - t slots short of the window length
  const int ntok_r =
      r < GQ ? max(0, min(kPageTokens, wl - (nqt - 1 - query_token(h0 + r, gqv, nqt)) - t0)) : 0;
  uint4 ka[4], qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    ka[s] = act && t0 + kslot < window
                ? *reinterpret_cast<const uint4*>(k_win + base + static_cast<size_t>(kslot) * kHeadDim + 32 * s + 8 * g)
                : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qb[s] = act && r < GQ ? *reinterpret_cast<const uint4*>(q + query_row(b, h0 + r, n_q, gqv, nqt) * kHeadDim + 32 * s + 8 * g)
                   : make_uint4(0, 0, 0, 0);
  // value operands: thread (dim pair dp, slot group sg)
  const int dp = tid & 63;
  const int sg = tid >> 6;
  uint32_t vv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = 16 * sg + i;
    vv[i] = act && t0 + t < window ? *reinterpret_cast<const uint32_t*>(v_win + base + static_cast<size_t>(t) * kHeadDim + 2 * dp)
                            : 0u;
  }

  // ---- scores: C[slot][head], lane holds head r of slots 16 wave + 4g + j
  wf32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(wbf16x8, ka[s]), __builtin_bit_cast(wbf16x8, qb[s]),
                                                  acc, 0, 0, 0);
  const float sl2 = static_cast<float>(scale_log2);
  float sc[4];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool valid = 16 * wave + 4 * g + j < ntok_r;
    sc[j] = valid ? acc[j] * sl2 : -INFINITY;
    mx = fmaxf(mx, sc[j]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (act && g == 0) mx_s[wave][r] = mx;
  __syncthreads();
  // per head: reference point = the largest score, weights, their sum
  const float big = fmaxf(fmaxf(mx_s[0][r], mx_s[1][r]), fmaxf(mx_s[2][r], mx_s[3][r]));
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = 16 * wave + 4 * g + j;
    const float pt = slot < ntok_r ? exp2f(sc[j] - big) : 0.f;
    if (act && r < GQ) p_s[r][slot] = pt;
    ls += pt;
  }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  if (act && g == 0) l_s[wave][r] = ls;
  __syncthreads();

  // ---- value sum: slots past ntok have weight 0 but their V words may hold anything
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (16 * sg + i >= ntok) vv[i] = 0u;
  float a0[GQ], a1[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) a0[h] = a1[h] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v0 = __uint_as_float(vv[i] << 16);
    const float v1 = __uint_as_float(vv[i] & 0xFFFF0000u);
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float pt = p_s[h][16 * sg + i];
      a0[h] = fmaf(pt, v0, a0[h]);
      a1[h] = fmaf(pt, v1, a1[h]);
    }
  }
  if (act) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      acc_s[sg][h][2 * dp] = a0[h];
      acc_s[sg][h][2 * dp + 1] = a1[h];
    }
  }
  __syncthreads();
  // (without kDual every thread stores: idle waves hold no data of their own but take part)
  for (int idx = tid; (!kDual || act) && idx < GQ * kHeadDim; idx += 64 * (kDual ? 4 : NWB)) {
    const int h = idx >> 7;
    const int d = idx & 127;
    const size_t o = (static_cast<size_t>(b) * n_q + h0 + h) * n_wsplits + c;
    auto put = [](float* p, float v) {
      if constexpr (kCoherent)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        *p = v;
    };
    put(out_acc + o * kHeadDim + d, (acc_s[0][h][d] + acc_s[1][h][d]) + (acc_s[2][h][d] + acc_s[3][h][d]));
    if (d == 0) {
      put(out_m + o, fmaxf(fmaxf(mx_s[0][h], mx_s[1][h]), fmaxf(mx_s[2][h], mx_s[3][h])));  // -inf: no slot
      put(out_l + o, (l_s[0][h] + l_s[1][h]) + (l_s[2][h] + l_s[3][h]));
    }
  }
}

}  // namespace window
}  // namespace oscar
