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
// Page layout of a head block (4096 + 512 n_g bytes, n_g = 128 / G): the K and V codes as in
// the one-group layout (bytes 0..4095), then the K (s16, z16) of slot t, group g at
// 4096 + 4 (n_g t + g), then the V pairs the same way.
//
// Demotion: one 256-thread workgroup per (token, KV head, K or V), as the one-group per-row
// kernel: fp64 dot products with an error bound per dim, decisions at both ends of the
// intervals, compensated sums when they do not settle; the extremes, scale and zero point are
// taken per group (a group's dims are held by 64 / n_g consecutive lanes of wave 0).
// INT2 pass: a plain dequantise-and-FMA pass on the vector ALU (the one-group path's matrix-
// core pass is not generalised) after the query rotation on bf16 MFMA: grid (split, KV head,
// request), 256 threads; per page, thread
// (token, quarter of the dims) scores its token against every query head of the KV head; the
// weights take an online softmax in log2 units and are multiplied by each slot's V scale of
// every group (the zero points summed once per page); thread (dim, half of the slots) adds
// weight-times-scale times code. The code and metadata words of the next two pages load
// during the current page.

#include "demote_pass.h"

namespace oscar {
namespace {

typedef float gf32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));

template <int NG>
constexpr int grouped_block_bytes() {
  return 4096 + 512 * NG;
}

// max (SEL 0) or min (SEL 1) over aligned segments of W lanes
template <int W, int SEL>
__device__ __forceinline__ double seg_ext(double v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) {
    const double u = __shfl_xor(v, o, 64);
    v = SEL == 0 ? fmax(v, u) : fmin(v, u);
  }
  return v;
}

template <int NG>
__global__ __launch_bounds__(256) void demote_grouped_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int n_kv,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ dst_slot, const uint16_t* __restrict__ rot_k,
    const uint16_t* __restrict__ rot_v, const float* __restrict__ clip_k, const float* __restrict__ clip_v,
    uint8_t* __restrict__ pool) {
#pragma clang fp contract(off)
  constexpr int kLanes = 64 / NG;  // lanes of wave 0 holding one group (two dims each)
  __shared__ double part[3][64][4];
  const int item = blockIdx.x;
  const int row = item >> 1;
  const int is_v = item & 1;
  const int tok = row / n_kv;
  const int head = row - tok * n_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* src = (is_v ? v_src : k_src) + static_cast<size_t>(row) * kHeadDim;
  const uint16_t* rot = (is_v ? rot_v : rot_k) + static_cast<size_t>(head) * kHeadDim * kHeadDim;

  uint32_t xw[16], rw[32];
  const uint32_t* xp = reinterpret_cast<const uint32_t*>(src + 32 * wave);
#pragma unroll
  for (int k = 0; k < 16; ++k) xw[k] = xp[k];
  const uint32_t* rp = reinterpret_cast<const uint32_t*>(rot + 32 * wave * kHeadDim + 2 * lane);
#pragma unroll
  for (int i = 0; i < 32; ++i) rw[i] = rp[i * (kHeadDim / 2)];
  int page = 0, slot = 0;
  float crf = 0.f;
  if (wave == 0) {
    page = dst_page[tok];
    slot = dst_slot[tok];
    crf = is_v ? clip_v[head] : clip_k[head];
  }
  double s0 = 0.0, s1 = 0.0, a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t xb = (i & 1) ? (xw[i >> 1] & 0xFFFF0000u) : (xw[i >> 1] << 16);
    const double xd = static_cast<double>(__uint_as_float(xb));
    const double r0 = static_cast<double>(__uint_as_float(rw[i] << 16));
    const double r1 = static_cast<double>(__uint_as_float(rw[i] & 0xFFFF0000u));
    s0 = fma(xd, r0, s0);
    s1 = fma(xd, r1, s1);
    a0 = fma(fabs(xd), fabs(r0), a0);
    a1 = fma(fabs(xd), fabs(r1), a1);
  }
  if (wave > 0) {
    double* pp = part[wave - 1][lane];
    pp[0] = s0;
    pp[1] = s1;
    pp[2] = a0;
    pp[3] = a1;
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const double* pp = part[w][lane];
    s0 = s0 + pp[0];
    s1 = s1 + pp[1];
    a0 = a0 + pp[2];
    a1 = a1 + pp[3];
  }
  double y0 = s0, y1 = s1;
  double d0 = demote::kBound * a0, d1 = demote::kBound * a1;
  const double cr = static_cast<double>(crf);
  demote::ScaleZero sz;
  int c0, c1;
  for (int pass = 0;; ++pass) {
    // the extremes of this lane's group (both of its dims lie in it)
    const double ymax = seg_ext<kLanes, 0>(fmax(y0, y1));
    const double ymin = seg_ext<kLanes, 1>(fmin(y0, y1));
    const double dm = seg_ext<kLanes, 0>(fmax(d0, d1));
    sz = demote::scale_zero(cr, ymax - dm, ymin + dm);
    const demote::ScaleZero sz2 = demote::scale_zero(cr, ymax + dm, ymin - dm);
    const double s16d = f16_bits_to_f64(sz.s16);
    const double z16d = f16_bits_to_f64(sz.z16);
    c0 = demote::code_of(y0 - d0, z16d, s16d, 0u);
    c1 = demote::code_of(y1 - d1, z16d, s16d, 0u);
    const bool group_ok = (sz.s16 == sz2.s16) && (sz.z16 == sz2.z16) && dm <= 1e300;
    const bool lane_ok = (c0 == demote::code_of(y0 + d0, z16d, s16d, 0u)) &&
                         (c1 == demote::code_of(y1 + d1, z16d, s16d, 0u));
    if (pass == 1 || __all(group_ok && lane_ok)) break;
    const demote::Pair e = demote::exact_pair(src, rot, lane);
    y0 = e.y0;
    y1 = e.y1;
    d0 = d1 = 0.0;
  }

  uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * grouped_block_bytes<NG>();
  if (lane % kLanes == 0) {
    const int g = lane / kLanes;
    uint32_t* meta = reinterpret_cast<uint32_t*>(blk + 4096 + (is_v ? 256 * NG : 0) + 4 * (NG * slot + g));
    *meta = static_cast<uint32_t>(sz.s16) | (static_cast<uint32_t>(sz.z16) << 16);
  }
  const int dd = 2 * lane;
  if (is_v) {
    const int r = slot & 15;
    const int sh = 8 * (r & 3) + 2 * (r >> 2);
    uint32_t* w0 = reinterpret_cast<uint32_t*>(blk + v_word_offset(dd, slot >> 4));
    uint32_t* w1 = reinterpret_cast<uint32_t*>(blk + v_word_offset(dd + 1, slot >> 4));
    atomicAnd(w0, ~(3u << sh));
    atomicAnd(w1, ~(3u << sh));
    atomicOr(w0, static_cast<uint32_t>(c0) << sh);
    atomicOr(w1, static_cast<uint32_t>(c1) << sh);
    return;
  }
  uint32_t bits = (static_cast<uint32_t>(c0) << demote::k_shift(dd)) |
                  (static_cast<uint32_t>(c1) << demote::k_shift(dd + 1));
  bits |= __shfl_xor(bits, 1, 64);
  bits |= __shfl_xor(bits, 2, 64);
  bits |= __shfl_xor(bits, 4, 64);
  if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(blk + k_word_offset(slot, lane >> 3)) = bits;
}

// The words one thread loads for a page: K words of its token's quarter of the dims, V words
// of its dim's half of the slots, and one K and one V metadata word (thread t < 64 n_g).
struct GPage {
  uint32_t k0, k1, v0, v1, km, vm;
};

template <int NG>
__device__ __forceinline__ GPage grouped_load(const uint8_t* blk, int tok, int part, int d, int half) {
  GPage r;
  r.k0 = *reinterpret_cast<const uint32_t*>(blk + k_word_offset(tok, 2 * part));
  r.k1 = *reinterpret_cast<const uint32_t*>(blk + k_word_offset(tok, 2 * part + 1));
  r.v0 = *reinterpret_cast<const uint32_t*>(blk + v_word_offset(d, 2 * half));
  r.v1 = *reinterpret_cast<const uint32_t*>(blk + v_word_offset(d, 2 * half + 1));
  const int t = threadIdx.x;
  r.km = t < 64 * NG ? *reinterpret_cast<const uint32_t*>(blk + 4096 + 4 * t) : 0u;
  r.vm = t < 64 * NG ? *reinterpret_cast<const uint32_t*>(blk + 4096 + 256 * NG + 4 * t) : 0u;
  return r;
}

// code of index i (0..15) of a packed word: index 4m + j at bits 8j + 2m
__device__ __forceinline__ float code_at(uint32_t w, int i) {
  return static_cast<float>((w >> (8 * (i & 3) + 2 * (i >> 2))) & 3u);
}

template <int NG, int GQ>
__global__ __launch_bounds__(256) void decode_grouped_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rot_k, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ hist_len, int n_q, int n_kv,
    int n_splits, float scale_log2, float* __restrict__ out_m, float* __restrict__ out_l,
    float* __restrict__ out_acc) {
  constexpr int G = kHeadDim / NG;
  constexpr int kHB = grouped_block_bytes<NG>();
  __shared__ float qr_s[GQ][kHeadDim];
  __shared__ __align__(16) uint16_t rot_s[64][kHeadDim + 8];  // half of R_K's rows, padded
  __shared__ __align__(16) uint16_t q_s[GQ][kHeadDim];
  __shared__ float sp_s[GQ][4];     // sum of q_rot over each quarter of the dims
  __shared__ float w_s[GQ][64];     // scores of the page's slots
  __shared__ float ws_s[GQ][NG][64];  // weight * V scale of (head, group, slot)
  __shared__ float zs_s[GQ][NG];      // sum over the page of weight * V zero point
  __shared__ uint32_t meta_s[2][64 * NG];
  __shared__ float m_s[GQ], l_s[GQ], al_s[GQ];
  const int t = threadIdx.x;
  const int split = blockIdx.x;
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
  const int h0 = kv * GQ;

  // ---- q_rot = q R_K of the KV head's query heads: the queries and R_K, in two halves of 64
  // rows, pass through LDS in 16-byte loads that are all in flight at once
  for (int idx = t; idx < GQ * kHeadDim / 8; idx += 256) {
    const int h = idx >> 4;
    const int ch = idx & 15;
    *reinterpret_cast<uint4*>(&q_s[h][8 * ch]) =
        *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(b) * n_q + h0 + h) * kHeadDim + 8 * ch);
  }
  // q_rot on the matrix cores (v_mfma_f32_16x16x32_bf16; bf16 products are exact, sums fp32):
  // A = the query rows (head n of lane (g, n), zero past GQ), B = R_K columns; wave w owns
  // dims 32 w .. 32 w + 31 (two 16-dim tiles); lane (g, n) ends with heads 4 g + i of dim n
  {
    const int lane = t & 63;
    const int wave = t >> 6;
    const int g = lane >> 4;
    const int n = lane & 15;
    gf32x4 qc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int hf = 0; hf < 2; ++hf) {
      __syncthreads();  // the previous half is no longer read
      for (int idx = t; idx < 64 * kHeadDim / 8; idx += 256) {
        const int row = idx >> 4;
        const int ch = idx & 15;
        *reinterpret_cast<uint4*>(&rot_s[row][8 * ch]) = *reinterpret_cast<const uint4*>(
            rot_k + (static_cast<size_t>(kv) * kHeadDim + 64 * hf + row) * kHeadDim + 8 * ch);
      }
      __syncthreads();
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int r0 = 32 * st + 8 * g;  // first R_K row (within the half) of this lane's k range
        const uint4 av = n < GQ ? *reinterpret_cast<const uint4*>(&q_s[n < GQ ? n : 0][64 * hf + r0])
                                : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = 32 * wave + 16 * j + n;
          uint32_t bw[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            bw[k] = static_cast<uint32_t>(rot_s[r0 + 2 * k][col]) | (static_cast<uint32_t>(rot_s[r0 + 2 * k + 1][col]) << 16);
          const uint4 bv = make_uint4(bw[0], bw[1], bw[2], bw[3]);
          qc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, av),
                                                         __builtin_bit_cast(gbf16x8, bv), qc[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < GQ) qr_s[4 * g + i][32 * wave + 16 * j + n] = qc[j][i];
  }
  if (t < GQ) {
    m_s[t] = -INFINITY;
    l_s[t] = 0.f;
  }
  __syncthreads();
  if (t < GQ * 4) {
    const int h = t / 4;
    const int pq = t % 4;
    float s = 0.f;
    for (int i = 0; i < 32; ++i) s += qr_s[h][32 * pq + i];
    sp_s[h][pq] = s;
  }
  __syncthreads();

  const int nh = hist_len[b];
  const int n_pages = (nh + kPageTokens - 1) / kPageTokens;
  const int pps = (n_pages + n_splits - 1) / n_splits;
  const int p_begin = split * pps;
  const int p_end = min(n_pages, p_begin + pps);
  const int32_t* table = block_table + static_cast<size_t>(b) * max_pages;
  const size_t page_stride = static_cast<size_t>(n_kv) * kHB;
  const uint8_t* head_base = pool + static_cast<size_t>(kv) * kHB;
  // score role: token tok, dims 32 part .. + 31 (group gk); value role: dim d, slots 32 half ..
  const int tok = t >> 2;
  const int part = t & 3;
  const int gk = (32 * part) / G;
  const int d = t >> 1;
  const int half = t & 1;
  const int gv = d / G;
  float acc[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) acc[h] = 0.f;

  // pages two ahead in flight, and the block-table entry of the page after them, so that no
  // page waits on a table load followed by a data load
  GPage cur = {0u, 0u, 0u, 0u, 0u, 0u}, nxt = cur;
  int id_ahead = 0;
  if (p_begin < p_end) cur = grouped_load<NG>(head_base + static_cast<size_t>(table[p_begin]) * page_stride, tok, part, d, half);
  if (p_begin + 1 < p_end) nxt = grouped_load<NG>(head_base + static_cast<size_t>(table[p_begin + 1]) * page_stride, tok, part, d, half);
  if (p_begin + 2 < p_end) id_ahead = table[p_begin + 2];
  for (int p = p_begin; p < p_end; ++p) {
    const int ntok = min(kPageTokens, nh - p * kPageTokens);
    __syncthreads();  // the previous page's metadata and weights are no longer read
    if (t < 64 * NG) {
      meta_s[0][t] = cur.km;
      meta_s[1][t] = cur.vm;
    }
    const GPage now = cur;
    cur = nxt;
    if (p + 2 < p_end) nxt = grouped_load<NG>(head_base + static_cast<size_t>(id_ahead) * page_stride, tok, part, d, half);
    if (p + 3 < p_end) id_ahead = table[p + 3];
    __syncthreads();  // metadata of the page in LDS
    // ---- scores: token tok against every head, dims of quarter `part`
    {
      const uint32_t km = meta_s[0][NG * tok + gk];
      const float sk = f16_to_f32(km);
      const float zk = f16_to_f32(km >> 16);
      float c[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        c[i] = code_at(now.k0, i);
        c[16 + i] = code_at(now.k1, i);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) dot = fmaf(qr_s[h][32 * part + i], c[i], dot);
        float sc = fmaf(sk, dot, zk * sp_s[h][part]);
        sc += __shfl_xor(sc, 1, 64);
        sc += __shfl_xor(sc, 2, 64);
        if (part == 0) w_s[h][tok] = tok < ntok ? sc * scale_log2 : -INFINITY;
      }
    }
    __syncthreads();
    // ---- online softmax per head (32 lanes per head, two slots each)
    for (int h = t / 32; h < GQ; h += 8) {
      const int j = t % 32;
      const float x0 = w_s[h][2 * j], x1 = w_s[h][2 * j + 1];
      float mx = fmaxf(x0, x1);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, mx);  // finite: a page holds at least one token
      const float p0 = __builtin_amdgcn_exp2f(x0 - m_new);
      const float p1 = __builtin_amdgcn_exp2f(x1 - m_new);
      // the dequantisation folded into the weights: per group g, weight * scale of each slot,
      // and the page's sum of weight * zero point (slots past the history end take 0: their
      // metadata may hold anything)
      const bool ok0 = 2 * j < ntok, ok1 = 2 * j + 1 < ntok;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint32_t m0 = meta_s[1][NG * (2 * j) + g];
        const uint32_t m1 = meta_s[1][NG * (2 * j + 1) + g];
        ws_s[h][g][2 * j] = ok0 ? p0 * f16_to_f32(m0) : 0.f;
        ws_s[h][g][2 * j + 1] = ok1 ? p1 * f16_to_f32(m1) : 0.f;
        float zz = (ok0 ? p0 * f16_to_f32(m0 >> 16) : 0.f) + (ok1 ? p1 * f16_to_f32(m1 >> 16) : 0.f);
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) zz += __shfl_xor(zz, o, 64);
        if (j == 0) zs_s[h][g] = zz;
      }
      float ps = p0 + p1;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 64);
      if (j == 0) {
        const float al = __builtin_amdgcn_exp2f(m_old - m_new);
        al_s[h] = al;
        l_s[h] = fmaf(l_s[h], al, ps);
        m_s[h] = m_new;
      }
    }
    __syncthreads();
    // ---- values: dim d, slots 32 half .. + 31: sum of (weight * scale) * code over the
    // slots, plus (once, in half 0) the page's sum of weight * zero point of d's group
    {
#pragma unroll
      for (int h = 0; h < GQ; ++h) acc[h] *= al_s[h];
#pragma unroll 8
      for (int i = 0; i < 32; ++i) {
        const int slot = 32 * half + i;
        const float code = code_at(i < 16 ? now.v0 : now.v1, i & 15);
#pragma unroll
        for (int h = 0; h < GQ; ++h) acc[h] = fmaf(ws_s[h][gv][slot], code, acc[h]);
      }
      if (half == 0) {
#pragma unroll
        for (int h = 0; h < GQ; ++h) acc[h] += zs_s[h][gv];
      }
    }
  }
  __syncthreads();
  // ---- partials: the two halves of the slots add up; (m, l) from the last page
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const float a = acc[h] + __shfl_xor(acc[h], 1, 64);
    const size_t o = (static_cast<size_t>(b) * n_q + h0 + h) * n_splits + split;
    if (half == 0) out_acc[o * kHeadDim + d] = a;
    if (t == 0) {
      out_m[o] = m_s[h];
      out_l[o] = l_s[h];
    }
  }
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

template <int NG, int GQ>
hipError_t launch_decode_grouped_gq(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                                    const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch,
                                    float sm_scale, int n_splits, const PartialsView& out, hipStream_t stream) {
  const float scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  hipLaunchKernelGGL((decode_grouped_kernel<NG, GQ>), dim3(n_splits, L.n_kv, batch), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(rot_k),
                     static_cast<const uint8_t*>(pool), block_table, max_pages, hist_len, L.n_q, L.n_kv, n_splits,
                     scale_log2, out.m, out.l, out.acc);
  return hipGetLastError();
}

template <int NG>
hipError_t launch_decode_grouped_ng(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                                    const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch,
                                    float sm_scale, int n_splits, const PartialsView& out, hipStream_t stream) {
  switch (L.gq) {
    case 1: return launch_decode_grouped_gq<NG, 1>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 2: return launch_decode_grouped_gq<NG, 2>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 4: return launch_decode_grouped_gq<NG, 4>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 8: return launch_decode_grouped_gq<NG, 8>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 16: return launch_decode_grouped_gq<NG, 16>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    default: return hipErrorInvalidValue;
  }
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
  switch (group) {
    case 128: return launch_decode_grouped_ng<1>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 64: return launch_decode_grouped_ng<2>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 32: return launch_decode_grouped_ng<4>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
