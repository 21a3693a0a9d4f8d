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
// Heads go in passes of up to eight. The R_V fragments of the un-rotation are loaded
// with the partials (load_rv). Every global load of a pass is issued before any of its
// arithmetic, so a pass whose splits fit one batch costs one memory round trip:
//   - the (m, l) of the first 64 partials of each head of the wave, first, since the
//     weights need only these,
//   - up to kBatch INT2 value sums per thread (thread = head, split slice, 4 dims) and the
//     window value sums of the same heads.
// All loads go through wave-uniform buffer descriptors over the pass's rows; a thread
// with nothing to load at a position gives an offset past the range and reads 0.
// The weights of a head are computed by the wave(s) that sum its values, so they pass
// through wave-private LDS with no workgroup barrier. Each thread sums a contiguous block
// of splits, so its weights are vector reads. The slices are then folded once per
// element, and the folded INT2 sums are split into a bf16 high part and a bf16 low part
// (about 16 significant bits together) laid out as the A operand of the un-rotation,
// which runs on the matrix cores: [16 rows = the pass's heads] x [128] x [128 dims] in
// bf16 with fp32 accumulation (two products); R_V itself is bf16 and exact.

#pragma once

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace merge {

constexpr int kMaxSplits = 256;  // INT2 splits the in-launch merge accepts
constexpr int kMaxWin = 8;       // window splits the merge accepts
constexpr int kMaxParts = kMaxSplits + kMaxWin;
constexpr int kBatch = 16;       // independent 16-byte value-sum loads per thread and batch
constexpr int kRow = kHeadDim + 4;           // floats of one value-sum row in LDS (16 bytes of bank spread)
constexpr int kARow = kHeadDim / 2 + 4;      // words of one packed bf16 A-operand row in LDS
constexpr uint32_t kNoLoad = 0x80000000u;    // buffer offset past every range: the load reads 0

// GQT query heads per KV head, NW waves (4 or 8)
template <int GQT, int NW>
struct Shape {
  static constexpr int HP = GQT < 8 ? GQT : 8;       // heads per pass
  static constexpr int SL = 2 * NW / HP;             // split slices per (head, 4 dims)
  static constexpr int HW = SL == 1 ? 2 : 1;         // heads per wave
  static constexpr int CW = (kMaxWin + SL - 1) / SL;  // window partials per thread
  static constexpr int NTW = 8 / NW;                 // 16-dim output tiles per wave
  static_assert((NW == 4 || NW == 8) && SL >= 1, "4 or 8 waves, at most 2 NW heads per pass");
};

// LDS of merge_group: per wave HW rows of kMaxParts weights and as many l values, the
// per-slice INT2 and window value sums of a pass, the packed bf16 high and low parts of
// the folded INT2 sums, and 1/L per head
template <int GQT, int NW>
__host__ __device__ constexpr int smem_bytes() {
  constexpr int HP = Shape<GQT, NW>::HP;
  constexpr int SL = Shape<GQT, NW>::SL;
  constexpr int HW = Shape<GQT, NW>::HW;
  return 4 * (NW * 2 * HW * kMaxParts + 2 * HP * SL * kRow + 2 * HP * kARow + HP);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 16 bytes at byte offset `off` of a buffer, read at agent scope (sees stores that other
// workgroups of the same launch completed with agent scope)
__device__ __forceinline__ f32x4 load16_agent(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16 /* sc1 */));
}
__device__ __forceinline__ f32x4 load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}
__device__ __forceinline__ float load4_agent(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 16 /* sc1 */));
}
__device__ __forceinline__ float load4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

// max / sum over the 64 lanes of the wave (every lane receives the result)
__device__ __forceinline__ float wave64_max(float v) {
  v = row16_max(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave64_sum(float v) {
  v = row16_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// x = hi + lo + e with hi the nearest bf16 of x, lo = (x - hi) truncated to bf16 (the
// difference is exact in fp32), |e| <= 2^-16 |x|; returns the packed bf16 pairs of two
// values
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t u0 = __float_as_uint(x0);
  const uint32_t u1 = __float_as_uint(x1);
  const uint32_t h0 = (u0 + 0x7FFFu + ((u0 >> 16) & 1u)) & 0xFFFF0000u;
  const uint32_t h1 = (u1 + 0x7FFFu + ((u1 >> 16) & 1u)) & 0xFFFF0000u;
  const uint32_t l0 = __float_as_uint(x0 - __uint_as_float(h0));
  const uint32_t l1 = __float_as_uint(x1 - __uint_as_float(h1));
  hi = (h0 >> 16) | h1;
  lo = (l0 >> 16) | (l1 & 0xFFFF0000u);
}

// B fragments of the un-rotation for wave `wave`'s dim tiles NTW wave + nt: column n =
// dim 16 tile + n, rows k = 32 ks + 8 (lane / 16) .. + 7, i.e. R_V[dim][k]. Loaded by the
// merging workgroup just before the partials, so both arrive in one round trip.
template <int NW>
__device__ __forceinline__ void load_rv(const uint16_t* __restrict__ rot_v, int kv, uint4 (&rb)[8 / NW][4]) {
  constexpr int NTW = 8 / NW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint16_t* rv = rot_v + static_cast<size_t>(kv) * kHeadDim * kHeadDim;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      rb[nt][ks] = *reinterpret_cast<const uint4*>(rv + (16 * (NTW * wave + nt) + (lane & 15)) * kHeadDim + 32 * ks +
                                                   8 * (lane >> 4));
}

// Un-rotation on the matrix cores of up to 16 vectors x (rotated basis, 128 dims each),
// held in LDS as packed bf16 pairs: x = hi + lo (split2), rows of kARow words; rows at or
// past `rows` are not read (zero). Gives x R_V^T for this wave's output tiles: put(row,
// dim, value) for every row < rows and the 16 NTW dims of the wave's tiles. [16 rows] x
// [128] x [16 dims] per tile in bf16 with fp32 accumulation (two products); R_V itself is
// bf16 and exact. rb from load_rv<NW>.
template <int NW, typename Put>
__device__ __forceinline__ void unrotate_tiles(const uint32_t* ahi_s, const uint32_t* alo_s, int rows,
                                               const uint4 (&rb)[8 / NW][4], Put put) {
  constexpr int NTW = 8 / NW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // A fragment: row = lane % 16, k = 32 ks + 8 (lane / 16) .. + 7
  uint4 ahi[4], alo[4];
  {
    const int g = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int w0 = g * kARow + 16 * ks + 4 * (lane >> 4);
      ahi[ks] = g < rows ? *reinterpret_cast<const uint4*>(ahi_s + w0) : make_uint4(0, 0, 0, 0);
      alo[ks] = g < rows ? *reinterpret_cast<const uint4*>(alo_s + w0) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bk = __builtin_bit_cast(bf16x8, rb[nt][ks]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ahi[ks]), bk, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo[ks]), bk, c, 0, 0, 0);
    }
    // C fragment: rows 4 (lane / 16) + j, column dim 16 tile + lane % 16
    const int d = 16 * (NTW * wave + nt) + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = 4 * (lane >> 4) + j;
      if (g < rows) put(g, d, c[j]);
    }
  }
}

// Merge of the GQT query heads of KV head kv of request b: `ns` INT2 partials per head
// (rotated V basis, written by this launch with agent-scope stores) and `nw` window
// partials per head into out[b][h][128]. 64 NW threads; 1 <= ns <= kMaxSplits,
// nw <= kMaxWin; rb from load_rv<NW>. kWinAgent: the window partials were written by this
// launch with agent-scope stores (else by an earlier launch) and are read at agent scope.
// kRot: the INT2 partials are in the rotated basis of R_V (else they were un-rotated when
// written, and the merge is a weighted sum in one basis; rb is then not read).
template <int GQT, int NW, bool kWinAgent = false, bool kRot = true>
__device__ __forceinline__ void merge_group(unsigned char* __restrict__ smem, int b, int kv, int n_q,
                                            const PartialsView& hist, int ns, const PartialsView& win, int nw,
                                            const uint4 (&rb)[8 / NW][4], float* __restrict__ out, int nqt = 1) {
  constexpr int HP = Shape<GQT, NW>::HP;
  constexpr int SL = Shape<GQT, NW>::SL;
  constexpr int HW = Shape<GQT, NW>::HW;
  constexpr int CW = Shape<GQT, NW>::CW;
  constexpr int NTW = Shape<GQT, NW>::NTW;
  const int np = ns + nw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float* wt_s = reinterpret_cast<float*>(smem) + wave * (2 * HW * kMaxParts);  // [HW][kMaxParts] m, then w
  float* wl_s = wt_s + HW * kMaxParts;                                           // [HW][kMaxParts] l
  float* part_s = reinterpret_cast<float*>(smem) + NW * 2 * HW * kMaxParts;    // [HP][SL][kRow] INT2 sums
  float* accw_s = part_s + HP * SL * kRow;                                      // [HP][SL][kRow] window sums
  uint32_t* ahi_s = reinterpret_cast<uint32_t*>(accw_s + HP * SL * kRow);      // [HP][kARow] bf16 pairs
  uint32_t* alo_s = ahi_s + HP * kARow;                                         // [HP][kARow]
  float* inv_s = reinterpret_cast<float*>(alo_s + HP * kARow);                  // [HP] 1 / L
  // value-sum role: head g2 of the pass, split slice (splits slice kBatch .. + kBatch - 1
  // of each batch), dims 4 quad .. 4 quad + 3; the heads of wave w are gbase .. + HW - 1
  const int g2 = tid / (32 * SL);
  const int slice = (tid >> 5) % SL;
  const int quad = tid & 31;
  const int gbase = (2 * wave) / SL;

  for (int p0 = 0; p0 < GQT; p0 += HP) {
    const size_t row0 = static_cast<size_t>(b) * n_q + static_cast<size_t>(kv) * GQT + p0;
    const __amdgpu_buffer_rsrc_t rs_acc = buffer_rsrc(hist.acc + row0 * ns * kHeadDim, HP * ns * kHeadDim * 4);
    const __amdgpu_buffer_rsrc_t rs_wacc = buffer_rsrc(win.acc + row0 * nw * kHeadDim, HP * nw * kHeadDim * 4);
    const __amdgpu_buffer_rsrc_t rs_m = buffer_rsrc(hist.m + row0 * ns, HP * ns * 4);
    const __amdgpu_buffer_rsrc_t rs_l = buffer_rsrc(hist.l + row0 * ns, HP * ns * 4);
    const __amdgpu_buffer_rsrc_t rs_wm = buffer_rsrc(win.m + row0 * nw, HP * nw * 4);
    const __amdgpu_buffer_rsrc_t rs_wl = buffer_rsrc(win.l + row0 * nw, HP * nw * 4);
    // (m, l) of partial `lane` of each head of the wave, requested first: the weights
    // need only these
    float m0[HW], l0[HW];
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      const int g = gbase + j;
      const uint32_t ho = lane < ns ? static_cast<uint32_t>((g * ns + lane) * 4) : kNoLoad;
      const uint32_t wo = lane >= ns && lane < np ? static_cast<uint32_t>((g * nw + lane - ns) * 4) : kNoLoad;
      m0[j] = load4_agent(rs_m, ho) + (kWinAgent ? load4_agent(rs_wm, wo) : load4(rs_wm, wo));
      l0[j] = load4_agent(rs_l, ho) + (kWinAgent ? load4_agent(rs_wl, wo) : load4(rs_wl, wo));
    }
    const uint32_t vbase = static_cast<uint32_t>((g2 * ns * kHeadDim + 4 * quad) * 4);
    // first batch of INT2 value sums: splits slice kBatch + k
    f32x4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int s = slice * kBatch + k;
      v[k] = load16_agent(rs_acc, s < ns ? vbase + static_cast<uint32_t>(s * kHeadDim * 4) : kNoLoad);
    }
    // window value sums: window partials slice + c SL
    f32x4 vw[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int cw = slice + c * SL;
      const uint32_t off = cw < nw ? static_cast<uint32_t>((((g2 * nw + cw) * kHeadDim) + 4 * quad) * 4) : kNoLoad;
      vw[c] = kWinAgent ? load16_agent(rs_wacc, off) : load16(rs_wacc, off);
    }

    // weights of the wave's heads: common maximum, w = 2^(m - M), 1 / L
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      const int g = gbase + j;
      float* wm = wt_s + j * kMaxParts;
      float* wl = wl_s + j * kMaxParts;
      const float mj = lane < np ? m0[j] : -INFINITY;
      float mx = mj;
      if (np > 64) {
        // more partials than lanes: the rest go through the wave's LDS rows
        for (int c0 = 64; c0 < np; c0 += 64) {
          const int s = c0 + lane;
          const uint32_t ho = s < ns ? static_cast<uint32_t>((g * ns + s) * 4) : kNoLoad;
          const uint32_t wo = s >= ns && s < np ? static_cast<uint32_t>((g * nw + s - ns) * 4) : kNoLoad;
          const float m =
              s < np ? load4_agent(rs_m, ho) + (kWinAgent ? load4_agent(rs_wm, wo) : load4(rs_wm, wo)) : -INFINITY;
          const float l = load4_agent(rs_l, ho) + (kWinAgent ? load4_agent(rs_wl, wo) : load4(rs_wl, wo));
          if (s < np) {
            wm[s] = m;
            wl[s] = l;
          }
          mx = fmaxf(mx, m);
        }
      }
      const float M = wave64_max(mx);
      const float w0 = mj == -INFINITY ? 0.f : exp2f(mj - M);
      wm[lane] = w0;
      float L = w0 * l0[j];
      if (np > 64) {
        for (int s = 64 + lane; s < np; s += 64) {
          const float m = wm[s];
          const float w = m == -INFINITY ? 0.f : exp2f(m - M);
          wm[s] = w;
          L = fmaf(w, wl[s], L);
        }
      }
      L = wave64_sum(L);
      if (lane == 0 && (2 * wave) % SL == 0) inv_s[g] = L > 0.f ? 1.f / L : 0.f;
    }
    // the weights were written by other lanes of this wave: LDS keeps a wave's accesses
    // in order, so only the compiler must not move the reads above the writes
    asm volatile("" ::: "memory");

    // weighted value sums of this thread's splits and window partials
    const float* wm = wt_s + (g2 - gbase) * kMaxParts;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = slice * kBatch;;) {
#pragma unroll
      for (int k4 = 0; k4 < kBatch; k4 += 4) {
        // weights past ns are not read from LDS (the rows hold window weights, then stale data)
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(wm + s0 + k4);
#pragma unroll
        for (int i = 0; i < 4; ++i) a += (s0 + k4 + i < ns ? w4[i] : 0.f) * v[k4 + i];
      }
      s0 += SL * kBatch;
      if (s0 >= ns) break;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int s = s0 + k;
        v[k] = load16_agent(rs_acc, s < ns ? vbase + static_cast<uint32_t>(s * kHeadDim * 4) : kNoLoad);
      }
    }
    f32x4 aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int cw = slice + c * SL;
      const float w = cw < nw ? wm[ns + cw] : 0.f;
      aw += w * vw[c];
    }
    *reinterpret_cast<f32x4*>(part_s + (g2 * SL + slice) * kRow + 4 * quad) = a;
    *reinterpret_cast<f32x4*>(accw_s + (g2 * SL + slice) * kRow + 4 * quad) = aw;
    __syncthreads();

    // fold the slices, once per dim pair: the INT2 sums into the packed bf16 high / low A
    // rows, the window sums into slice 0 of their rows
    for (int pr = tid; pr < HP * (kHeadDim / 2); pr += 64 * NW) {
      const int g = pr / (kHeadDim / 2);
      const int d = 2 * (pr % (kHeadDim / 2));
      float2 x = *reinterpret_cast<const float2*>(part_s + g * SL * kRow + d);
      float2 y = *reinterpret_cast<const float2*>(accw_s + g * SL * kRow + d);
#pragma unroll
      for (int sl = 1; sl < SL; ++sl) {
        const float2 xs = *reinterpret_cast<const float2*>(part_s + (g * SL + sl) * kRow + d);
        const float2 ys = *reinterpret_cast<const float2*>(accw_s + (g * SL + sl) * kRow + d);
        x.x += xs.x;
        x.y += xs.y;
        y.x += ys.x;
        y.y += ys.y;
      }
      if constexpr (kRot) {
        split2(x.x, x.y, ahi_s[g * kARow + d / 2], alo_s[g * kARow + d / 2]);
        if (SL > 1) *reinterpret_cast<float2*>(accw_s + g * SL * kRow + d) = y;
      } else {
        float* o = out + query_row(b, kv * GQT + p0 + g, n_q, GQT, nqt) * kHeadDim + d;
        o[0] = (x.x + y.x) * inv_s[g];
        o[1] = (x.y + y.y) * inv_s[g];
      }
    }
    if constexpr (!kRot) {
      if (p0 + HP < GQT) __syncthreads();  // the next pass reuses the LDS
      continue;
    }
    __syncthreads();

    unrotate_tiles<NW>(ahi_s, alo_s, HP, rb, [&](int g, int d, float c) {
      out[query_row(b, kv * GQT + p0 + g, n_q, GQT, nqt) * kHeadDim + d] = (c + accw_s[g * SL * kRow + d]) * inv_s[g];
    });
    if (p0 + HP < GQT) __syncthreads();  // the next pass reuses the LDS
  }
}

}  // namespace merge
}  // namespace oscar
