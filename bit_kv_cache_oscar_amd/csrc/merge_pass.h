// Online-softmax merge of the INT2 and BF16 segments of every query head of one KV head,
// with the value un-rotation: device code run by the last workgroup of the fused decode
// kernel to finish for a (request, KV head).
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the BF16 and INT2 parts
// of decode are combined by an online-softmax merge. The INT2 value sum lives in the
// rotated basis of R_V (values were rotated before quantisation), so it is multiplied by
// R_V^T before joining the BF16 part; un-rotating after the reduction is exact because
// the un-rotation is linear.
//
// All partials of a head (INT2 splits, then window splits) are merged against one common
// maximum M: weights w = 2^(m - M), L = sum w l, and
//   out = ((sum_INT2 w acc) R_V^T + sum_window w acc) / L.
// Heads go in passes of up to eight. Every load of a pass is issued before any of its
// arithmetic: R_V (staged into LDS, first pass), every (m, l), up to kBatch INT2 value
// sums per thread (thread = head, split slice, 4 dims) and the window value sums, so a
// pass with up to kBatch splits per slice costs about one memory round trip.

#pragma once

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace merge {

constexpr int kMaxSplits = 256;  // INT2 splits the in-launch merge accepts
constexpr int kBatch = 16;       // independent 16-byte loads per thread and batch
constexpr int kRvRow = 272;      // bytes of one R_V row in LDS: 256 + 16 (conflict-free 16-byte row reads)

template <int GQT>
struct Shape {
  static constexpr int HP = GQT < 8 ? GQT : 8;  // heads per pass
  static constexpr int SL = 8 / HP;             // split slices per (head, 4 dims)
};

// LDS of merge_group for GQT heads per KV head and up to kMaxSplits INT2 splits
template <int GQT>
__host__ __device__ constexpr int smem_bytes() {
  constexpr int HP = Shape<GQT>::HP;
  constexpr int SL = Shape<GQT>::SL;
  return 4 * (2 * HP * (kMaxSplits + 8) + HP * SL * kHeadDim + HP * kHeadDim + 2 * HP) + kHeadDim * kRvRow;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 bytes at byte offset `off` of a buffer, read at agent scope (sees stores that other
// workgroups of the same launch completed with agent scope)
__device__ __forceinline__ f32x4 load16_agent(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16 /* sc1 */));
}

// Merge of the GQT query heads of KV head kv of request b: `ns` INT2 partials per head
// (rotated V basis, written by this launch with agent-scope stores) and `nw` window
// partials per head (written by an earlier launch) into out[b][h][128]. 256 threads;
// ns <= kMaxSplits, nw <= 8.
template <int GQT>
__device__ __forceinline__ void merge_group(unsigned char* __restrict__ smem, int b, int kv, int n_q,
                                            const PartialsView& hist, int ns, const PartialsView& win, int nw,
                                            const uint16_t* __restrict__ rot_v, float* __restrict__ out) {
  constexpr int HP = Shape<GQT>::HP;
  constexpr int SL = Shape<GQT>::SL;
  const int np = ns + nw;
  float* w_s = reinterpret_cast<float*>(smem);       // [HP][np]: m, then the weights
  float* l_s = w_s + HP * np;                        // [HP][np]
  float* part_s = w_s + 2 * HP * (kMaxSplits + 8);   // [HP][SL][128] INT2 sums per slice
  float* accw_s = part_s + HP * SL * kHeadDim;       // [HP][128] window sums
  float* sc_s = accw_s + HP * kHeadDim;              // [HP]: L
  unsigned char* rv_s = smem + 4 * (2 * HP * (kMaxSplits + 8) + HP * SL * kHeadDim + HP * kHeadDim + 2 * HP);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int d = tid & (kHeadDim - 1);
  // phase-2 role: head g, split slice, dims 4 quad .. 4 quad + 3
  const int g2 = tid / (32 * SL);
  const int slice = (tid >> 5) % SL;
  const int quad = tid & 31;

  // R_V of the KV head, requested first; its LDS copy is written once the other loads of
  // the first pass are in flight
  uint4 rv[8];
  const uint4* rsrc = reinterpret_cast<const uint4*>(rot_v + static_cast<size_t>(kv) * kHeadDim * kHeadDim);
#pragma unroll
  for (int k = 0; k < 8; ++k) rv[k] = rsrc[tid + 256 * k];

  for (int p0 = 0; p0 < GQT; p0 += HP) {
    const size_t row0 = static_cast<size_t>(b) * n_q + static_cast<size_t>(kv) * GQT + p0;
    const size_t row2 = row0 + g2;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(hist.acc + row2 * ns * kHeadDim, 0, ns * kHeadDim * 4, 0x00020000);
    // first batch of INT2 value sums (loads past ns read 0: outside the buffer)
    f32x4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      v[k] = load16_agent(rs, static_cast<uint32_t>((slice + k * SL) * kHeadDim + 4 * quad) * 4);
    // window value sums (slice 0 threads)
    f32x4 vw[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      vw[c] = (slice == 0 && c < nw) ? *reinterpret_cast<const f32x4*>(win.acc + (row2 * nw + c) * kHeadDim + 4 * quad)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
    // (m, l) of every partial of the pass's heads
    for (int i = tid; i < HP * np; i += 256) {
      const int g = i / np;
      const int s = i - g * np;
      const size_t row = row0 + g;
      float m, l;
      if (s < ns) {
        m = __hip_atomic_load(hist.m + row * ns + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        l = __hip_atomic_load(hist.l + row * ns + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        m = win.m[row * nw + (s - ns)];
        l = win.l[row * nw + (s - ns)];
      }
      w_s[i] = m;
      l_s[i] = l;
    }
    if (p0 == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = tid + 256 * k;  // 16-byte chunk i: row i / 16, chunk i % 16
        *reinterpret_cast<uint4*>(rv_s + (i >> 4) * kRvRow + 16 * (i & 15)) = rv[k];
      }
    }
    __syncthreads();
    // per head (wave w: heads w, w + 4): common maximum, weights, L
    for (int g = wave; g < HP; g += 4) {
      float M = -INFINITY;
      for (int s = lane; s < np; s += 64) M = fmaxf(M, w_s[g * np + s]);
      M = wave_max(M);
      float L = 0.f;
      for (int s = lane; s < np; s += 64) {
        const float m = w_s[g * np + s];
        const float wt = m == -INFINITY ? 0.f : exp2f(m - M);
        w_s[g * np + s] = wt;
        L = fmaf(wt, l_s[g * np + s], L);
      }
      L = wave_sum(L);
      if (lane == 0) sc_s[g] = L;
    }
    __syncthreads();
    // weighted value sums
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = slice;; ) {
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int s = s0 + k * SL;
        const float wt = s < ns ? w_s[g2 * np + s] : 0.f;
        a += wt * v[k];
      }
      s0 += SL * kBatch;
      if (s0 >= ns) break;
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        v[k] = load16_agent(rs, static_cast<uint32_t>((s0 + k * SL) * kHeadDim + 4 * quad) * 4);
    }
    *reinterpret_cast<f32x4*>(part_s + (g2 * SL + slice) * kHeadDim + 4 * quad) = a;
    if (slice == 0) {
      f32x4 aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < nw) aw += w_s[g2 * np + ns + c] * vw[c];
      *reinterpret_cast<f32x4*>(accw_s + g2 * kHeadDim + 4 * quad) = aw;
    }
    __syncthreads();
    // fold the slices into slice 0
    if (SL > 1 && slice == 0) {
      f32x4 t = *reinterpret_cast<const f32x4*>(part_s + g2 * SL * kHeadDim + 4 * quad);
#pragma unroll
      for (int sl = 1; sl < SL; ++sl) t += *reinterpret_cast<const f32x4*>(part_s + (g2 * SL + sl) * kHeadDim + 4 * quad);
      *reinterpret_cast<f32x4*>(part_s + g2 * SL * kHeadDim + 4 * quad) = t;
    }
    __syncthreads();
    // un-rotation and output: thread (d, half) for heads half, half + 2, ... of the pass
    for (int g = tid >> 7; g < HP; g += 2) {
      const f32x4* acc4 = reinterpret_cast<const f32x4*>(part_s + g * SL * kHeadDim);
      const uint4* rrow = reinterpret_cast<const uint4*>(rv_s + d * kRvRow);
      float oh = 0.f;
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const uint4 r = rrow[i];
        const f32x4 x0 = acc4[2 * i];
        const f32x4 x1 = acc4[2 * i + 1];
        oh = fmaf(x0.x, __uint_as_float(r.x << 16), oh);
        oh = fmaf(x0.y, __uint_as_float(r.x & 0xFFFF0000u), oh);
        oh = fmaf(x0.z, __uint_as_float(r.y << 16), oh);
        oh = fmaf(x0.w, __uint_as_float(r.y & 0xFFFF0000u), oh);
        oh = fmaf(x1.x, __uint_as_float(r.z << 16), oh);
        oh = fmaf(x1.y, __uint_as_float(r.z & 0xFFFF0000u), oh);
        oh = fmaf(x1.z, __uint_as_float(r.w << 16), oh);
        oh = fmaf(x1.w, __uint_as_float(r.w & 0xFFFF0000u), oh);
      }
      const float L = sc_s[g];
      out[(row0 + g) * kHeadDim + d] = L > 0.f ? (oh + accw_s[g * kHeadDim + d]) / L : 0.f;
    }
    __syncthreads();  // the next pass reuses the LDS
  }
}

}  // namespace merge
}  // namespace oscar
