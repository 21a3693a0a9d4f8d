// INT2 history pass of decode attention on the gfx950 matrix cores: device code shared
// by the standalone INT2 kernels and the fused decode kernels.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the INT2 kernel unpacks
// the 2-bit codes, dequantises with the per-group scale and zero point and accumulates
// in floating point; its result is joined with the BF16 sink/recent pass by an
// online-softmax merge.
//
// Both contractions run on the raw codes, with the dequantisation folded out:
//   score_t = s_t (q_rot . (c_t - 2)) + (z_t + 2 s_t) sum(q_rot)
//   acc     = sum_t (p_t s^V_t) c^V_t + sum_t p_t z^V_t
// K side, per page: [4 heads x 4 rows] x [128 dims] x [64 tokens] on
//   v_mfma_i32_16x16x64_i8. q_rot is a 22-bit fixed-point integer Q (|Q| <= 2^21) in three
//   signed 8-bit limbs (rows 0..2 of a head; row 3 is zero), read from LDS each page. The
//   three limb rows combine exactly in int32 into Q . c; the per-head term -2 sum Q, which
//   seeds the accumulator, centres it to Q . (c - 2) (|.| <= 2^29). Centring the codes at 2
//   keeps the two terms of the fold small, so the fold runs in fp32. (Fewer query bits
//   would let the codes enter with the cheaper scaled unpacking of the V side, but 22 bits
//   are what keeps the score error well inside the output tolerance.)
// V side, per page: [4 heads x 4 rows] x [64 tokens] x [16 dims] per dim tile. The
//   codes enter as int8 straight from the packed word with one mask per byte field
//   (unpack16_scaled): field m (bits 2m..2m+1 of each byte) yields c 4^m for m < 3 and,
//   after a shift by 2, 16 c for m = 3, so every code carries a factor (1, 4, 16, 16)[m].
//   The weight P'_t = round(p_t s^V_t 2^E / (2 factor_t)) is an integer below 2^23 (E
//   wave-uniform, chosen from the largest V scale seen so that p s 2^E < 2^24), read
//   straight from the bits of the float p s 2^E / factor + 2^24; the code of slot t sits in
//   field ((t % 16) / 4), so factor_t is constant per lane and P'_t times the scaled code is
//   round(p s 2^E / 2) c up to rounding (P' keeps at least 19 significant bits). Its three low bytes, each in signed range after an
//   XOR with 0x80 (the exponent bit already sets it for the top one), are rows 0..2 of the
//   head, so the MFMA yields sum_t (byte_l - 128) c'_t with c' the scaled code. Row 3 is
//   constant 1 and yields sum_t c'_t, which restores the 128 (1 + 2^8 + 2^16) offset.
//   The int32 accumulators run across pages and are folded into fp32 sums only when a
//   head's reference maximum or the fixed-point exponent must change. A reference maximum
//   moves only when a score exceeds it by more than kTau (log2 units), so p <= 2^kTau.
//
// Lloyd-Max codebook variant (QbitAI article on OSCAR, comparison with TurboQuant: a
// stronger Lloyd-Max codebook in place of the uniform levels): a code c dequantises to
// z + s k_c / 16 with four levels k_c per (KV head, K or V). The codes are unpacked as
// above and mapped through the levels by one byte permute per four codes. K takes the
// levels centred, k_c - mid (mid the integer centre of the levels, |k_c - mid| <= 24), so
// the MFMA yields Q . (k - mid) with no centring seed (the query preparation keeps
// sum |Q| < 2^26 + 64 for it), and the fold is s 2^-sh Q . (k - mid) / 16 + (z + s mid / 16)
// sum(q_rot). V takes the levels themselves (0..48, the same bound as the scaled codes),
// every lane with the factor 16.
//
// Quantisation groups (QbitAI article on OSCAR, section on aiming the rotation at attention:
// a scale and zero point per group of G = 128 / NG rotated dims, NG = 2 or 4): the K product
// runs once per group against a copy of the query limbs that is zero outside the group's
// dims, and group g's term s_g Q_g . (c - 2) + (z_g + 2 s_g) S_g joins the score, with
// S_g = sum of Q over the group (from the same copy times a B of ones) standing in for the
// exact sum of the rotated query; the V side takes one set of P' limbs per group (each dim
// tile lies in one group) and one zero-point sum per group. Query heads come in tiles of
// four there (the per-group metadata leaves no registers for two tiles).
//
// A workgroup serves one (history split, KV head x head group, request), 4 waves, at most 8
// query heads (16 query heads per KV head run as two groups of 8). Wave w walks
// pages split_begin + w, + 4, ... of its split with two page buffers in flight. In a page,
// MFMA column n of K tile nt is slot 4n + nt, so lane (G, n) holds head G's scores of
// slots 4n..4n+3; byte permutes turn its four P' values into one dword per limb, and a
// wave-private LDS block carries them into the A layout of the V MFMA (slots 16G..16G+15
// per lane). Wave partials are merged through LDS and one (m, l, acc) partial per
// (request, query head, split) is written.

#pragma once

#include "device_common.h"
#include "merge_pass.h"
#include "launch.h"

namespace oscar {
namespace int2 {

constexpr int kWaves = 4;
constexpr int kPRow = 80;    // bytes of one P-limb row in LDS: 64 slots + 16 bytes of bank spread
constexpr int kTau = 2;      // headroom of the softmax weights above the reference maximum (log2)
typedef char i8x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// register m holds the codes at bits 2m..2m+1 of the packed word's four bytes
__device__ __forceinline__ i8x16 unpack16(uint32_t w) {
  uint4 u;
  u.x = w & 0x03030303u;
  u.y = (w >> 2) & 0x03030303u;
  u.z = (w >> 4) & 0x03030303u;
  u.w = (w >> 6) & 0x03030303u;
  return __builtin_bit_cast(i8x16, u);
}

// as unpack16, with register m's codes times (1, 4, 16, 16)[m]: three masks and a shift
__device__ __forceinline__ i8x16 unpack16_scaled(uint32_t w) {
  uint4 u;
  u.x = w & 0x03030303u;
  u.y = w & 0x0C0C0C0Cu;
  u.z = w & 0x30303030u;
  u.w = (w >> 2) & 0x30303030u;
  return __builtin_bit_cast(i8x16, u);
}

// as unpack16, each code replaced by byte `code` of the lookup word `lut`
__device__ __forceinline__ i8x16 unpack16_lut(uint32_t w, uint32_t lut) {
  uint4 u;
  u.x = __builtin_amdgcn_perm(lut, lut, w & 0x03030303u);
  u.y = __builtin_amdgcn_perm(lut, lut, (w >> 2) & 0x03030303u);
  u.z = __builtin_amdgcn_perm(lut, lut, (w >> 4) & 0x03030303u);
  u.w = __builtin_amdgcn_perm(lut, lut, (w >> 6) & 0x03030303u);
  return __builtin_bit_cast(i8x16, u);
}

__device__ __forceinline__ i32x4 mfma16(i8x16 a, i8x16 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 2^e as a double, e in [-1022, 1023]
__device__ __forceinline__ double pow2d(int e) { return __longlong_as_double(static_cast<long long>(e + 1023) << 52); }
// 2^e as a float, e in [-126, 127]
__device__ __forceinline__ float pow2f(int e) { return __int_as_float((e + 127) << 23); }

// sum_t P'_t c_t of one accumulator fragment: rows 0..2 hold sum (byte_l - 128) c, row 3
// sum c, so byte sums are c_l + 128 c_3 >= 0 and combine without cancellation in fp32
__device__ __forceinline__ float v_combo(const i32x4& c) {
  const int c3 = c[3] << 7;
  const float b0 = static_cast<float>(c[0] + c3);
  const float b1 = static_cast<float>(c[1] + c3);
  const float b2 = static_cast<float>(c[2] + c3);
  return fmaf(b2, 65536.f, fmaf(b1, 256.f, b0));
}

template <int NG = 1>
struct PageRegs {
  uint4 k[2];    // K words: slots 4n..4n+3 (two words each: dims 32G..32G+15, 32G+16..32G+31)
  uint4 km[NG];  // K (scale, zero) of slots 4n..4n+3, NG groups each
  uint4 vm[NG];  // V (scale, zero) of slots 4n..4n+3, NG groups each
  uint4 v[2];    // V words of dims 16dt + n, dt = 0..7, slots 16G..16G+15

  __device__ __forceinline__ uint32_t kword(int nt, int h) const {
    const uint4& c = k[nt >> 1];
    return (nt & 1) ? (h ? c.w : c.z) : (h ? c.y : c.x);
  }
  static __device__ __forceinline__ uint32_t pick(const uint4& c, int i) {
    return i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w;
  }
  // pair of slot 4n + nt, group g
  __device__ __forceinline__ uint32_t kmeta(int nt, int g = 0) const { return pick(km[(NG * nt + g) >> 2], (NG * nt + g) & 3); }
  __device__ __forceinline__ uint32_t vmeta(int nt, int g = 0) const { return pick(vm[(NG * nt + g) >> 2], (NG * nt + g) & 3); }
  __device__ __forceinline__ uint32_t vword(int dt) const { return pick(v[dt >> 2], dt & 3); }
};

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int imm) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + imm, 0, 0));
}

// Lane l = 16 G + n reads its page data as 4 + 2 NG 16-byte loads (the page layout keeps
// each lane's K and V words, and the pairs of its four slots, contiguous) through a raw
// buffer descriptor of the page's head block, built in scalar registers from the
// wave-uniform page address. `meta16` is kKMeta + 16 NG n; `bytes` is the head block's
// size, or 0 for a request that reads nothing (every load then returns 0 without touching
// memory).
template <int NG>
__device__ __forceinline__ void load_page(PageRegs<NG>& r, const uint8_t* page, uint32_t lane32, uint32_t meta16,
                                          int bytes = head_block_bytes<NG>()) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(page), 0, bytes, kRsrcWord3);
  r.k[0] = load16(rs, lane32, kKCodes);
  r.k[1] = load16(rs, lane32, kKCodes + 16);
#pragma unroll
  for (int i = 0; i < NG; ++i) r.km[i] = load16(rs, meta16, 16 * i);
#pragma unroll
  for (int i = 0; i < NG; ++i) r.vm[i] = load16(rs, meta16, 256 * NG + 16 * i);
  r.v[0] = load16(rs, lane32, kVCodes);
  r.v[1] = load16(rs, lane32, kVCodes + 16);
}

// The rotated query of one (request, query head) h of request b: q_rot = q R_K in fp64
// (bf16 products are exact), as Q = rint(q_rot 2^sh) with max|q_rot| 2^sh < 2^21, in three
// signed 8-bit limbs (limb row 3 zero); the centring term -2 sum_d Q_d; the score scale
// 2^-sh sm_scale log2(e) and sm_scale log2(e) sum_d q_rot_d. Every read (the query row, the
// rotation's column pairs) is issued first; wave w sums rows 32 w .. +31 at columns
// 2 lane, 2 lane + 1, waves 1..3 hand their sums to wave 0 through LDS (one barrier), and
// wave 0 does the rest alone.
constexpr int kQprepSmem = 3 * 64 * 2 * 8;

__device__ __forceinline__ void qprep_head(unsigned char* smem, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ rot_k, int n_q, int gq, double scale_log2,
                                           char* __restrict__ qlimb, QueryScal* __restrict__ qscal, int h, int b,
                                           int nqt = 1, const uint32_t* __restrict__ codebook = nullptr) {
  double(*part_s)[64][2] = reinterpret_cast<double(*)[64][2]>(smem);
  const int kv = h / gq;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const size_t head = static_cast<size_t>(b) * n_q + h;

  // ---- reads: this wave's 32 query values (the same for every lane) and rotation rows
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(q + query_row(b, h, n_q, gq, nqt) * kHeadDim + 32 * w);
  uint32_t qq[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) qq[u] = qw[u];
  const uint32_t* rcol = reinterpret_cast<const uint32_t*>(rot_k + static_cast<size_t>(kv) * kHeadDim * kHeadDim +
                                                           static_cast<size_t>(32 * w) * kHeadDim) + lane;
  uint32_t rr[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) rr[u] = rcol[u * (kHeadDim / 2)];
  const uint32_t klv = codebook ? codebook[2 * kv] : 0u;  // K codebook word (0: uniform levels)
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const double qv = static_cast<double>(__uint_as_float((u & 1) ? (qq[u >> 1] & 0xFFFF0000u) : (qq[u >> 1] << 16)));
    a0 = fma(qv, static_cast<double>(__uint_as_float(rr[u] << 16)), a0);
    a1 = fma(qv, static_cast<double>(__uint_as_float(rr[u] & 0xFFFF0000u)), a1);
  }
  if (w > 0) {
    part_s[w - 1][lane][0] = a0;
    part_s[w - 1][lane][1] = a1;
  }
  __syncthreads();
  if (w > 0) return;  // uniform per wave; no barrier follows

  // ---- wave 0: q_rot at dims 2 lane, 2 lane + 1
  const double x0 = ((a0 + part_s[0][lane][0]) + part_s[1][lane][0]) + part_s[2][lane][0];
  const double x1 = ((a1 + part_s[0][lane][1]) + part_s[1][lane][1]) + part_s[2][lane][1];
  // amax rounded to float can only move up to the next power of two: the bound holds
  const float amax = wave_max_f32(static_cast<float>(fmax(fabs(x0), fabs(x1))));
  const double sm = wave_sum_f64(x0 + x1);
  int k = 0;
  if (amax > 0.f) frexpf(amax, &k);  // amax < 2^k
  int sh = 21 - k;
  if (klv != 0u) {
    // codebook levels enter the K dot centred, as k - mid with |k - mid| <= 24: sum |Q| is
    // held below 2^26 + 64 (the computed sum of |q_rot| is within 1e-14 of the true one),
    // so Q . (k - mid) stays below 2^31
    const double l1 = wave_sum_f64(fabs(x0) + fabs(x1));
    int kl = 0;
    if (l1 > 0.0) frexp(l1, &kl);  // l1 < 2^kl
    sh = min(sh, 26 - kl);
  }
  const int Q0 = static_cast<int>(rint(x0 * pow2d(sh)));
  const int Q1 = static_cast<int>(rint(x1 * pow2d(sh)));
  // signed 8-bit limbs: Q = l0 + 2^8 l1 + 2^16 l2, |l2| <= 33
  auto limbs = [](int Q, int& l0, int& l1, int& l2) {
    l0 = static_cast<signed char>(Q & 0xFF);
    const int r1 = (Q - l0) >> 8;
    l1 = static_cast<signed char>(r1 & 0xFF);
    l2 = (r1 - l1) >> 8;
  };
  int a[3], c[3];
  limbs(Q0, a[0], a[1], a[2]);
  limbs(Q1, c[0], c[1], c[2]);
  uint16_t* dst = reinterpret_cast<uint16_t*>(qlimb + head * 512) + lane;
#pragma unroll
  for (int r = 0; r < 3; ++r)
    dst[r * (kHeadDim / 2)] = static_cast<uint16_t>((a[r] & 0xFF) | ((c[r] & 0xFF) << 8));
  dst[3 * (kHeadDim / 2)] = 0;
  // exact integer sum of Q over the 128 dims: the centring term -2 sum Q
  int sq = Q0 + Q1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
  if (lane == 0) {
    QueryScal o;
    // the codebook's dot is in sixteenths of the scale and needs no centring term
    o.qsc = static_cast<float>(pow2d(-sh) * scale_log2 * (klv != 0u ? 0.0625 : 1.0));
    o.sig = static_cast<float>(sm * scale_log2);
    o.kcent = klv != 0u ? 0 : -2 * sq;
    o.pad[0] = o.pad[1] = o.pad[2] = o.pad[3] = o.pad[4] = 0;
    qscal[head] = o;
  }
}

// Per-wave online-softmax state held in registers (this lane: head 4 mt + G of tile mt).
// "Pending" sums are in units of 2^E relative to the reference maximum m (the V sums in the
// int32 MFMA accumulators, in units of 2^(E-1)). The "flushed" sums (true values relative
// to m: sum p s^V c^V per dim, l and sum p z^V) live in LDS, touched only when flushing.
template <int MT, int NG = 1>
struct WaveState {
  float m[MT];        // reference maximum, log2 units; -inf before the first page
  float bias[MT];     // E - m (0 before the first page); -inf for padding heads
  float lq[MT];       // pending sum of p 2^E over this lane's slots
  float zq[MT][NG];   // pending sum of p 2^E z^V per quantisation group
  i32x4 acci[MT][8];  // pending fragments (rows: 3 XORed limbs + code sum), dims 16 dt + n
};

constexpr int kQRow = 144;  // bytes of one query-limb row in LDS: 128 dims + 16 of bank spread
// flushed values per lane and tile: 8 dim tiles, l, sum p z per quantisation group
template <int NG>
constexpr int flushed_values() {
  return 9 + NG;
}

// GQ is the number of query heads one workgroup serves (at most 8); a KV head whose group
// is larger is served by n_groups = (query heads per KV head) / GQ workgroups along y.
// NW is the number of waves of the workgroup; NG the quantisation groups per vector (the
// query limbs are then held once per group, each copy zero outside the group's dims, and
// the P' limbs once per group).
template <int GQ, int NW = kWaves, int NG = 1>
constexpr int int2_smem_bytes() {
  constexpr int MT = (GQ + 3) / 4;
  constexpr int loop = NW * MT * NG * 16 * kPRow + NW * MT * flushed_values<NG>() * 64 * 4;
  constexpr int wacc = NW * GQ * kHeadDim * 4;
  return NG * 4 * MT * 4 * kQRow + loop + wacc + 2 * NW * GQ * 4;
}

// Partial-result store: with kCoherent, an agent-scope store that is visible to every
// workgroup of the launch once it has completed (for a merge inside the same launch).
template <bool kCoherent>
__device__ __forceinline__ void store_partial(float* p, float v) {
  if constexpr (kCoherent)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Options of the one-launch decode step: the query is prepared inside the workgroup (from q
// and R_K) instead of read from an earlier launch's workspace; the last `n_excl` history
// tokens of each request are left out (the step's appended token, which its own workgroup
// attends); partials are written with `pstride` split columns per head.
struct InlineQuery {
  const uint16_t* q = nullptr;      // bf16 [B][Hq][128]; null: query data from qlimb / qscal
  const uint16_t* rot_k = nullptr;  // bf16 [Hkv][128][128]
  double scale_log2 = 0.0;
  int n_excl = 0;
  int pstride = 0;                  // 0: n_splits
  int nqt = 1;                      // query tokens per request: q rows of virtual heads (query_row)
  int gqv = 0;                      // virtual heads per KV head (with nqt > 1)
};

// One workgroup (NW waves) of the INT2 pass: history split `split` of request b for the
// query heads gy*GQ .. gy*GQ+GQ-1 (KV head gy / n_groups). `smem` holds
// int2_smem_bytes<GQ, NW>(). With CB, `codebook` holds the codebook words [n_kv][K, V].
// With kUnrot the split's value sum is un-rotated (times R_V^T, rot_v [n_kv][128][128])
// before it is written, so its partial is in the basis of the BF16 window's; otherwise it
// stays in the rotated basis of R_V.
template <int GQ, bool kCoherent = false, int NW = kWaves, bool CB = false, bool kUnrot = false, int NG = 1>
__device__ __forceinline__ void int2_split(
    unsigned char* __restrict__ smem, int split, int gy, int b, const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ hist_len, int n_q, int n_kv, int n_groups, int n_splits,
    const char* __restrict__ qlimb, const QueryScal* __restrict__ qscal, float* __restrict__ out_m,
    float* __restrict__ out_l, float* __restrict__ out_acc, const uint32_t* __restrict__ codebook = nullptr,
    const InlineQuery& iq = InlineQuery(), const uint16_t* __restrict__ rot_v = nullptr) {
  constexpr int MT = (GQ + 3) / 4;  // 16-row M tiles
  static_assert(NG == 1 || NG == 2 || NG == 4, "one, two or four quantisation groups per vector");
  static_assert(NG == 1 || !CB, "codebooks are defined for one group per vector");
  constexpr int kFl = flushed_values<NG>();
  constexpr int kPBytes = NW * MT * NG * 16 * kPRow;
  constexpr int kFBytes = NW * MT * kFl * 64 * 4;
  constexpr int kLoopBytes = kPBytes + kFBytes;
  constexpr int kWaccBytes = NW * GQ * kHeadDim * 4;
  constexpr int kQCopy = 4 * MT * 4 * kQRow;  // one copy of the query limb rows
  constexpr int kBlock = head_block_bytes<NG>();

  // page loop: query limbs (one copy per quantisation group); P' limbs and flushed sums of
  // each wave. Epilogue: wave partials in a space of their own, so a wave writes its partial
  // as soon as its pages are done.
  unsigned char* q_s = smem;
  unsigned char* scratch_s = smem + NG * kQCopy;
  float (*wacc_s)[GQ][kHeadDim] = reinterpret_cast<float (*)[GQ][kHeadDim]>(scratch_s + kLoopBytes);
  float(*wm_s)[GQ] = reinterpret_cast<float(*)[GQ]>(scratch_s + kLoopBytes + kWaccBytes);
  float(*wl_s)[GQ] = reinterpret_cast<float(*)[GQ]>(scratch_s + kLoopBytes + kWaccBytes + NW * GQ * 4);

  const int kv = gy / n_groups;
  // codebook variant: lookup words of the centred K levels (k - mid as int8) and of the V
  // levels, and the fold's centre mid / 16 (2 for the uniform codes, centred at 2)
  uint32_t klut = 0u, vlut = 0u;
  float kmid = 2.f;
  if constexpr (CB) {
    const uint32_t kw = codebook[2 * kv];
    vlut = codebook[2 * kv + 1];
    const int mid = codebook_mid(kw);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      klut |= (static_cast<uint32_t>(static_cast<int>((kw >> (8 * c)) & 0xFFu) - mid) & 0xFFu) << (8 * c);
    kmid = static_cast<float>(mid) * 0.0625f;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // MFMA column / row index
  const int G = lane >> 4;  // lane group
  const int h0 = gy * GQ;  // first query head of this workgroup

  const int nh = max(0, hist_len[b] - iq.n_excl);
  const int pstride = iq.pstride > 0 ? iq.pstride : n_splits;
  const int n_pages = (nh + kPageTokens - 1) / kPageTokens;
  const int pps = (n_pages + n_splits - 1) / n_splits;
  const int p_begin = split * pps;
  const int p_end = min(n_pages, p_begin + pps);
  const int32_t* table = block_table + static_cast<size_t>(b) * max_pages;
  const uint8_t* head_base = pool + static_cast<size_t>(kv) * kBlock;
  const size_t page_stride = static_cast<size_t>(n_kv) * kBlock;
  const uint32_t lane32 = 32u * lane;
  const uint32_t meta16 = kKMeta + 16u * NG * n;
  const size_t head0 = static_cast<size_t>(b) * n_q + h0;

  // Prologue, in two memory round trips: the query operands (which do not depend on the
  // block table) and the block ids, then the first two pages.
  // query limbs of the workgroup's heads, bound for LDS: row 4 g + l holds limb l of head
  // g (rows of heads beyond GQ are zero); one 16-byte chunk per thread
  constexpr int kQChunks = 4 * MT * 4 * (kHeadDim / 16);
  static_assert(kQChunks <= 64 * NW, "one query-limb chunk per thread");
  const int qrow = tid >> 3;
  const int qc = tid & 7;
  const bool inline_q = NG == 1 && iq.q != nullptr;  // uniform (groups take the prepared query)
  uint4 qv = {0u, 0u, 0u, 0u};
  if (!inline_q && tid < kQChunks && (qrow >> 2) < GQ)
    qv = *reinterpret_cast<const uint4*>(qlimb + (head0 + (qrow >> 2)) * 512 + (qrow & 3) * kHeadDim + 16 * qc);
  float qsc[MT], sig[MT];
  int kcent[MT];
  bool head_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int g = 4 * mt + G;
    head_ok[mt] = g < GQ;
    kcent[mt] = 0;
    qsc[mt] = sig[mt] = 0.f;
    if (head_ok[mt] && !inline_q) {
      const QueryScal s = qscal[head0 + g];
      kcent[mt] = s.kcent;
      qsc[mt] = s.qsc;
      sig[mt] = s.sig;
    }
  }
  // inline query preparation: wave w holds rows RW w .. RW w + RW - 1 of R_K at this lane's
  // columns 2 lane, 2 lane + 1 (requested here, with the block ids below)
  constexpr int RW = kHeadDim / NW;
  uint32_t rk[RW];
  // the wave's query values (dims RW w .. + RW - 1 of each head), 16 bytes per lane for
  // lanes < GQ RW / 8, bound for wave-private LDS: requested before the block ids and the
  // pages, so that waiting for them never waits for a page
  constexpr int kQLanes = GQ * RW / 8;
  static_assert(kQLanes <= 64, "one 16-byte query chunk per lane");
  uint4 qchunk = {0u, 0u, 0u, 0u};
  if (inline_q) {
    const uint32_t* rp = reinterpret_cast<const uint32_t*>(iq.rot_k + static_cast<size_t>(kv) * kHeadDim * kHeadDim +
                                                           static_cast<size_t>(RW * wave) * kHeadDim) + lane;
#pragma unroll
    for (int r = 0; r < RW; ++r) rk[r] = rp[r * (kHeadDim / 2)];
    if (lane < kQLanes) {
      const int g = lane / (RW / 8);
      const size_t row = iq.nqt > 1 ? query_row(b, h0 + g, n_q, iq.gqv, iq.nqt) : head0 + g;
      qchunk = *reinterpret_cast<const uint4*>(iq.q + row * kHeadDim + RW * wave + 8 * (lane % (RW / 8)));
    }
  }

  // block ids of this wave's pages p0, p0 + NW, ...: lane i of blk_lane holds the id of the
  // wave's page 64 chunk + i
  const int p0 = p_begin + wave;
  const int n_mine = p0 < p_end ? (p_end - p0 + NW - 1) / NW : 0;
  int chunk = 0;
  int blk_lane = (lane < n_mine) ? table[p0 + NW * lane] : 0;
  // Everything requested so far has arrived here: none of it counts as outstanding in the
  // page loop, whose waits then let the next pages keep loading.
  asm volatile("" ::"v"(blk_lane), "v"(qv.x), "v"(qv.y), "v"(qv.z), "v"(qv.w));
  asm volatile("" ::"v"(qchunk.x), "v"(qchunk.y), "v"(qchunk.z), "v"(qchunk.w));
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) asm volatile("" ::"v"(kcent[mt]), "v"(qsc[mt]), "v"(sig[mt]));
  if (!inline_q && tid < kQChunks) {
    if constexpr (NG == 1) {
      *reinterpret_cast<uint4*>(q_s + qrow * kQRow + 16 * qc) = qv;
    } else {
      // copy g keeps the dims of group g (chunk qc holds dims 16 qc .. 16 qc + 15)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        *reinterpret_cast<uint4*>(q_s + g * kQCopy + qrow * kQRow + 16 * qc) =
            (qc * NG) / 8 == g ? qv : uint4{0u, 0u, 0u, 0u};
    }
  }
  auto page_of = [&](int j) -> const uint8_t* {  // j wave-uniform, 0 <= j < n_mine
    if ((j >> 6) != chunk) {
      chunk = j >> 6;
      const int i = 64 * chunk + lane;
      blk_lane = (i < n_mine) ? table[p0 + NW * i] : 0;
      // wait for the new ids here, on this rare path: the page loads in flight are then
      // never counted as something the id reads below depend on
      asm volatile("" ::"v"(blk_lane));
    }
    return head_base + static_cast<size_t>(__builtin_amdgcn_readlane(blk_lane, j & 63)) * page_stride;
  };
  // Inline query preparation: q_rot = q R_K for the workgroup's heads, each wave over its
  // RW rows with bf16 pair dot products (exact products, fp32 sums), joined through LDS;
  // then per head (one wave each) the 22-bit fixed point, its limbs into the LDS rows of
  // the page loop, and the head's scalars, as the separate query preparation computes
  // them. The join uses the page loop's LDS; a head's scalars go to the spare bytes past
  // the 128 dims of its first limb row, which nothing writes afterwards. The dot products come
  // before the first page loads are issued: issuing those of all waves takes the compute
  // unit's vector-memory path several hundred nanoseconds, which the query would wait out.
  static_assert(NW * GQ * 64 * 8 + NW * GQ * RW * 2 <= kLoopBytes + kWaccBytes, "the query join fits the loop's LDS");
  static_assert(kQRow - kHeadDim >= 16, "a head's scalars fit its row's spare bytes");
  float2(*qpart)[GQ][64] = reinterpret_cast<float2(*)[GQ][64]>(scratch_s);
  if (inline_q) {
    // wave-private staging of the wave's query values: [GQ][RW] bf16 (the wave's own LDS
    // accesses run in order, so no barrier is needed before reading them back)
    uint32_t* qst = reinterpret_cast<uint32_t*>(scratch_s + NW * GQ * 64 * 8) + wave * (GQ * RW / 2);
    if (lane < kQLanes) *reinterpret_cast<uint4*>(qst + 4 * lane) = qchunk;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // R_K pairs along the rows: (R[r][c], R[r + 1][c]) for this lane's columns c = 2 lane
    // (low halves) and 2 lane + 1 (high halves)
    uint32_t rc0[RW / 2], rc1[RW / 2];
#pragma unroll
    for (int j = 0; j < RW / 2; ++j) {
      rc0[j] = __builtin_amdgcn_perm(rk[2 * j + 1], rk[2 * j], 0x05040100u);
      rc1[j] = __builtin_amdgcn_perm(rk[2 * j + 1], rk[2 * j], 0x07060302u);
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < RW / 2; ++j) {
        const uint32_t qq = qst[g * (RW / 2) + j];  // (q[r], q[r + 1]), wave-uniform
        a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qq), __builtin_bit_cast(bf16x2_t, rc0[j]), a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qq), __builtin_bit_cast(bf16x2_t, rc1[j]), a1, false);
      }
      qpart[wave][g][lane] = make_float2(a0, a1);
    }
    // padding rows (heads past GQ, and every head's zero row 3) of the limb block
    for (int i = tid; i < 4 * MT * 4 * (kHeadDim / 16); i += 64 * NW) {
      const int row = i >> 3;
      if ((row >> 2) >= GQ || (row & 3) == 3) *reinterpret_cast<uint4*>(q_s + row * kQRow + 16 * (i & 7)) = uint4{0, 0, 0, 0};
    }
  }
  // keep the page loads below the dot products
  __builtin_amdgcn_sched_barrier(0);

  // three page buffers: pages i + 1 and i + 2 load while page i is processed (two with
  // the larger per-group metadata of four groups, or of two groups over two head tiles:
  // page i + 1 loads while page i is processed). A wave without pages issues the same
  // loads against an empty buffer, so every path carries the same loads into the loop.
  constexpr int NB = (NG == 1 || (NG == 2 && MT == 1)) ? 3 : 2;
  const int rec = n_mine > 0 ? kBlock : 0;
  PageRegs<NG> buf[NB];
  load_page(buf[0], page_of(0), lane32, meta16, rec);
  load_page(buf[1], page_of(n_mine > 1 ? 1 : 0), lane32, meta16, rec);
  if (inline_q) {
    __syncthreads();
    uint32_t klv = 0u;
    if constexpr (CB) klv = codebook[2 * kv];
    for (int g = wave; g < GQ; g += NW) {
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const float2 v = qpart[w2][g][lane];
        x0 += v.x;
        x1 += v.y;
      }
      const float amax = wave_max_f32(fmaxf(fabsf(x0), fabsf(x1)));
      const float sm = wave_sum_f32(x0 + x1);
      int k = 0;
      if (amax > 0.f) frexpf(amax, &k);  // amax < 2^k
      int sh = 21 - k;
      if (klv != 0u) {
        const float l1 = wave_sum_f32(fabsf(x0) + fabsf(x1));
        int kl = 0;
        if (l1 > 0.f) frexpf(l1, &kl);
        sh = min(sh, 26 - kl);
      }
      // x 2^sh is exact (a power of two); |Q| <= 2^21
      const int Q0 = static_cast<int>(rintf(x0 * pow2f(sh)));
      const int Q1 = static_cast<int>(rintf(x1 * pow2f(sh)));
      auto limbs = [](int Q, int& l0, int& l1, int& l2) {
        l0 = static_cast<signed char>(Q & 0xFF);
        const int r1 = (Q - l0) >> 8;
        l1 = static_cast<signed char>(r1 & 0xFF);
        l2 = (r1 - l1) >> 8;
      };
      int la[3], lc[3];
      limbs(Q0, la[0], la[1], la[2]);
      limbs(Q1, lc[0], lc[1], lc[2]);
#pragma unroll
      for (int r = 0; r < 3; ++r)
        *reinterpret_cast<uint16_t*>(q_s + (4 * g + r) * kQRow + 2 * lane) =
            static_cast<uint16_t>((la[r] & 0xFF) | ((lc[r] & 0xFF) << 8));
      // exact integer sum of Q over the 128 dims (|Q| <= 2^21): row butterflies, then the rows
      int sq = Q0 + Q1;
      sq += __builtin_amdgcn_update_dpp(0, sq, kDppQuadXor1, 0xF, 0xF, false);
      sq += __builtin_amdgcn_update_dpp(0, sq, kDppQuadXor2, 0xF, 0xF, false);
      sq += __builtin_amdgcn_update_dpp(0, sq, kDppHalfMirror, 0xF, 0xF, false);
      sq += __builtin_amdgcn_update_dpp(0, sq, kDppMirror, 0xF, 0xF, false);
      sq = (__builtin_amdgcn_readlane(sq, 0) + __builtin_amdgcn_readlane(sq, 16)) +
           (__builtin_amdgcn_readlane(sq, 32) + __builtin_amdgcn_readlane(sq, 48));
      if (lane == 0) {
        // (qsc, sig, kcent) as the separate query preparation's QueryScal holds them
        uint4 o;
        o.x = __float_as_uint(static_cast<float>(pow2d(-sh) * iq.scale_log2 * (klv != 0u ? 0.0625 : 1.0)));
        o.y = __float_as_uint(static_cast<float>(static_cast<double>(sm) * iq.scale_log2));
        o.z = static_cast<uint32_t>(klv != 0u ? 0 : -2 * sq);
        o.w = 0u;
        *reinterpret_cast<uint4*>(q_s + 4 * g * kQRow + kHeadDim) = o;
      }
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int g = 4 * mt + G;
      if (head_ok[mt]) {
        const uint4 o = *reinterpret_cast<const uint4*>(q_s + 4 * g * kQRow + kHeadDim);
        qsc[mt] = __uint_as_float(o.x);
        sig[mt] = __uint_as_float(o.y);
        kcent[mt] = static_cast<int>(o.z);
      }
    }
  }

  WaveState<MT, NG> st;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st.m[mt] = -INFINITY;
    st.bias[mt] = head_ok[mt] ? 0.f : -INFINITY;
    st.lq[mt] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) st.zq[mt][g] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acci[mt][dt] = i32x4{0, 0, 0, 0};
  }
  int E = 0;            // fixed-point exponent of the pending sums (wave-uniform)
  float thr = kTau;     // E + kTau: frame-relative scores above it move the reference
  // the codes of this lane's slots carry the factor (1, 4, 16, 16)[n % 4]: the V scales
  // are taken over it (powers of two, exact)
  // (with a codebook every lane's V levels carry the factor 16 of the sixteenths)
  const float vscale = CB ? 0.0625f : ((n & 3) == 0 ? 1.f : ((n & 3) == 1 ? 0.25f : 0.0625f));
  const float vunscale = CB ? 16.f : ((n & 3) == 0 ? 1.f : ((n & 3) == 1 ? 4.f : 16.f));
  float vcap_l = -1.f;  // V scales below vcap_l / vscale fit the current E
  bool fresh = true;    // no page processed yet

  // wave-private P'-limb rows: row (mt NG + group) 16 + 4 g + l; rows with l == 3 hold
  // constant ones
  unsigned char* pl = scratch_s + wave * (MT * NG * 16 * kPRow);
  // flushed sums per lane and tile: k < 8: dim tile k, 8: l, 9 + group: sum p z. One tile of
  // one or two groups keeps them in registers; otherwise they live in wave-private LDS,
  // [mt][k][lane]
  constexpr bool kFlReg = MT == 1 && NG <= 2;
  float flr[kFlReg ? kFl : 1];
  float* fl = reinterpret_cast<float*>(scratch_s + kPBytes) + wave * (MT * kFl * 64) + lane;
#pragma unroll
  for (int k = 0; k < (kFlReg ? kFl : 1); ++k) flr[k] = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
      *reinterpret_cast<uint32_t*>(pl + ((mt * NG + g) * 16 + 4 * G + 3) * kPRow + 4 * n) = 0x01010101u;
    if constexpr (!kFlReg) {
#pragma unroll
      for (int k = 0; k < kFl; ++k) fl[(mt * kFl + k) * 64] = 0.f;
    }
  }
  // flushed value k of tile mt
  auto flv = [&](int mt, int k) -> float& { return kFlReg ? flr[k] : fl[(mt * kFl + k) * 64]; };

  // the centring seed and the offset weight of each (tile, group): -2 sum Q and sig with
  // one group; with groups, from the group sums S_g of the fixed-point query (below)
  int kcg[MT][NG];
  float sgg[MT][NG];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    kcg[mt][0] = kcent[mt];
    sgg[mt][0] = sig[mt];
  }

  // fold tile mt's pending sums into the flushed ones, rescaled to the reference m_new
  auto flush_tile = [&](int mt, float m_new) {
    if (!fresh) {
      const float alpha = st.m[mt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m[mt] - m_new);
      const float down = pow2f(-E);
      const float down_v = pow2f(1 - E);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) flv(mt, dt) = fmaf(v_combo(st.acci[mt][dt]), down_v, flv(mt, dt)) * alpha;
      flv(mt, 8) = fmaf(st.lq[mt], down, flv(mt, 8)) * alpha;
#pragma unroll
      for (int g = 0; g < NG; ++g) flv(mt, 9 + g) = fmaf(st.zq[mt][g], down, flv(mt, 9 + g)) * alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acci[mt][dt] = i32x4{0, 0, 0, 0};
    st.lq[mt] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) st.zq[mt][g] = 0.f;
    st.m[mt] = m_new;
  };

  auto process = [&](const PageRegs<NG>& cur, int ntok) {
    // K side: rows (head, limb) x 16 slots per tile. With groups, one product per group,
    // from the query copy that is zero outside the group's dims, each folded into the
    // scores as it completes.
    float x[MT][4];  // scores relative to the frame: x = score_log2 - m + E
    float sv[NG][4], zv[NG][4];
    if constexpr (NG == 1) {
      i8x16 aK[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          aK[mt][ks] = *reinterpret_cast<const i8x16*>(q_s + (16 * mt + n) * kQRow + 32 * G + 16 * ks);
      i32x4 d[MT][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        i8x16 b0, b1;
        if constexpr (CB) {
          b0 = unpack16_lut(cur.kword(nt, 0), klut);
          b1 = unpack16_lut(cur.kword(nt, 1), klut);
        } else {
          b0 = unpack16(cur.kword(nt, 0));
          b1 = unpack16(cur.kword(nt, 1));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          d[mt][nt] = mfma16(aK[mt][1], b1, mfma16(aK[mt][0], b0, i32x4{kcg[mt][0], 0, 0, 0}));
      }
      // slot metadata of this lane's slots 4n..4n+3
      float sk[4], u[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t km = cur.kmeta(nt);
        const uint32_t vm = cur.vmeta(nt);
        sk[nt] = f16_to_f32(km);
        u[nt] = fmaf(kmid, sk[nt], f16_to_f32(km >> 16));  // z + 2 s (codebook: z + s mid / 16)
        sv[0][nt] = f16_to_f32(vm) * vscale;  // V scale over the factor of this lane's codes
        zv[0][nt] = f16_to_f32(vm >> 16);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const i32x4 c = d[mt][nt];
          // Q . (c - 2), exact (the partial terms may wrap; the sum fits)
          const int D = static_cast<int>(static_cast<uint32_t>(c[0]) + (static_cast<uint32_t>(c[1]) << 8) +
                                         (static_cast<uint32_t>(c[2]) << 16));
          x[mt][nt] = fmaf(static_cast<float>(D) * sk[nt], qsc[mt], fmaf(u[nt], sgg[mt][0], st.bias[mt]));
        }
    } else {
      i8x16 b0[4], b1[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        b0[nt] = unpack16(cur.kword(nt, 0));
        b1[nt] = unpack16(cur.kword(nt, 1));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) x[mt][nt] = st.bias[mt];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float sk[4], u[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const uint32_t km = cur.kmeta(nt, g);
          sk[nt] = f16_to_f32(km);
          u[nt] = fmaf(2.f, sk[nt], f16_to_f32(km >> 16));  // z + 2 s
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const unsigned char* qa = q_s + g * kQCopy + (16 * mt + n) * kQRow + 32 * G;
          const i8x16 a0 = *reinterpret_cast<const i8x16*>(qa);
          const i8x16 a1 = *reinterpret_cast<const i8x16*>(qa + 16);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const i32x4 c = mfma16(a1, b1[nt], mfma16(a0, b0[nt], i32x4{kcg[mt][g], 0, 0, 0}));
            // Q_g . (c - 2) over the group's dims, exact
            const int D = static_cast<int>(static_cast<uint32_t>(c[0]) + (static_cast<uint32_t>(c[1]) << 8) +
                                           (static_cast<uint32_t>(c[2]) << 16));
            x[mt][nt] = fmaf(static_cast<float>(D) * sk[nt], qsc[mt], fmaf(u[nt], sgg[mt][g], x[mt][nt]));
          }
        }
      }
      // the V metadata once the K codes are done with
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const uint32_t vm = cur.vmeta(nt, g);
          sv[g][nt] = f16_to_f32(vm) * vscale;
          zv[g][nt] = f16_to_f32(vm >> 16);
        }
    }
    if (ntok < kPageTokens) {
      // slots past the history end may hold stale bits: no weight, no scale
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bool valid = 4 * n + nt < ntok;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          sv[g][nt] = valid ? sv[g][nt] : 0.f;
          zv[g][nt] = valid ? zv[g][nt] : 0.f;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) x[mt][nt] = valid ? x[mt][nt] : -INFINITY;
      }
    }
    float xm[MT];
    bool over = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      xm[mt] = fmaxf(fmaxf(x[mt][0], x[mt][1]), fmaxf(x[mt][2], x[mt][3]));
      over = over || xm[mt] > thr;
    }
    float svm = fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3]));
#pragma unroll
    for (int g = 1; g < NG; ++g) svm = fmaxf(svm, fmaxf(fmaxf(sv[g][0], sv[g][1]), fmaxf(sv[g][2], sv[g][3])));
    const bool vover = svm > vcap_l;
    if (fresh || __any(over || vover)) {
      // a new exponent for the wave's V scales moves every tile's frame
      int e_new = E;
      if (__any(vover)) {
        int k = 0;
        frexpf(wave_max_f32(svm * vunscale), &k);  // largest V scale < 2^k
        e_new = 24 - k - kTau;                     // p s 2^E < 2^24 while p <= 2^kTau and s < 2^k
        vcap_l = pow2f(k) * vscale;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // a head's reference moves to the page maximum when that exceeds it by kTau
        const float r = row16_max(xm[mt]) - st.bias[mt];
        const float m_new = head_ok[mt] ? (r > st.m[mt] + kTau ? r : st.m[mt]) : -INFINITY;
        if (fresh || e_new != E || __any(m_new != st.m[mt])) {
          const float bias_new = head_ok[mt] ? static_cast<float>(e_new) - m_new : -INFINITY;
          const float shift = head_ok[mt] ? bias_new - st.bias[mt] : 0.f;
          flush_tile(mt, m_new);
          st.bias[mt] = bias_new;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) x[mt][nt] = head_ok[mt] ? x[mt][nt] + shift : -INFINITY;
        }
      }
      E = e_new;
      thr = static_cast<float>(E + kTau);
      fresh = false;
    }
    // probabilities (units of 2^E), pending sums, P' limbs (per group: the V scales differ).
    // A (tile, group) whose P' are all zero (every weight p s^V 2^E below one unit) adds
    // exactly nothing to the V sums: its limb rows then hold -128 c per code and the
    // constant row c, which cancel in v_combo. When every pair is so, the V side is skipped
    // (wave-uniform).
    bool vskip[MT][NG];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float pe[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        pe[nt] = __builtin_amdgcn_exp2f(x[mt][nt]);
        st.lq[mt] += pe[nt];
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        uint32_t P[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          st.zq[mt][g] = fmaf(pe[nt], zv[g][nt], st.zq[mt][g]);
          // pe sv < 2^24: the float pe sv + 2^24 holds round(pe sv / 2) in its mantissa, and
          // its exponent's low bit is bit 23
          P[nt] = __float_as_uint(fmaf(pe[nt], sv[g][nt], 16777216.f));
        }
        vskip[mt][g] = __all((P[0] | P[1] | P[2] | P[3]) == 0x4B800000u);  // 2^24: P' = 0
        // with several head tiles the limbs are written whatever vskip says: a tile whose P'
        // are all zero then gets rows encoding P' = 0 (each dword 0x80808080), which add
        // exactly nothing, and the V products below run for every tile in straight-line
        // code (per-tile branches there cost more than the products they skip)
        if (MT > 1 || !vskip[mt][g]) {
          // byte l of the four P' values into one dword per limb, in signed range
          const uint32_t t01 = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);
          const uint32_t t23 = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
          const uint32_t u01 = __builtin_amdgcn_perm(P[1], P[0], 0x0C0C0602u);
          const uint32_t u23 = __builtin_amdgcn_perm(P[3], P[2], 0x0C0C0602u);
          const uint32_t L0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u) ^ 0x80808080u;
          const uint32_t L1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u) ^ 0x80808080u;
          const uint32_t L2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);  // bit 7 set by the exponent
          unsigned char* row = pl + ((mt * NG + g) * 16 + 4 * G) * kPRow + 4 * n;
          *reinterpret_cast<uint32_t*>(row) = L0;
          *reinterpret_cast<uint32_t*>(row + kPRow) = L1;
          *reinterpret_cast<uint32_t*>(row + 2 * kPRow) = L2;
        }
      }
    }
    bool vall = true;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g = 0; g < NG; ++g) vall = vall && vskip[mt][g];
    if (!vall) {
      // the wave's LDS operations run in order: the reads below see the writes above
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      i8x16 aP[MT][NG];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          aP[mt][g] = *reinterpret_cast<const i8x16*>(pl + ((mt * NG + g) * 16 + n) * kPRow + 16 * G);
      // V side: rows (head, limb) x 64 slots x 16 dims per dim tile, accumulated in int32;
      // dim tile dt lies in group dt NG / 8
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        constexpr int kTilesPerGroup = 8 / NG;
        const int g = dt / kTilesPerGroup;
        i8x16 bv;
        if constexpr (CB)
          bv = unpack16_lut(cur.vword(dt), vlut);
        else
          bv = unpack16_scaled(cur.vword(dt));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (MT > 1 || NG == 1 || !vskip[mt][g]) st.acci[mt][dt] = mfma16(aP[mt][g], bv, st.acci[mt][dt]);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // The prefetch is unconditional (past the last page the last page asks for itself again,
  // an L2 hit), so no path without it joins between the loads and the use of a page.
  auto ntok_of = [&](int j) { return min(kPageTokens, nh - (p0 + NW * j) * kPageTokens); };
  auto next_of = [&](int j) { return page_of(j < n_mine ? j : n_mine - 1); };
  // query limbs in LDS (the inline preparation's last barrier already covers them; the
  // page loop's set-up above writes only wave-private LDS)
  if (!inline_q) __syncthreads();
  if constexpr (NG > 1) {
    // S_g = sum of Q over group g's dims, exact in int32 (|S_g| <= 64 2^21), as the group's
    // query copy times a B of ones on the matrix cores. The group's centring seed is -2 S_g
    // and its offset weight qsc S_g: the fold then takes the fixed-point query for both of
    // its terms, so the group's score term is qsc Q_g . (s c + z), the dequantised key's dot
    // with the query as the K product sees it.
    const i8x16 ones = __builtin_bit_cast(i8x16, uint4{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u});
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const unsigned char* qa = q_s + g * kQCopy + (16 * mt + n) * kQRow + 32 * G;
        const i32x4 c = mfma16(*reinterpret_cast<const i8x16*>(qa + 16), ones,
                               mfma16(*reinterpret_cast<const i8x16*>(qa), ones, i32x4{0, 0, 0, 0}));
        const int S = static_cast<int>(static_cast<uint32_t>(c[0]) + (static_cast<uint32_t>(c[1]) << 8) +
                                       (static_cast<uint32_t>(c[2]) << 16));
        kcg[mt][g] = -2 * S;
        sgg[mt][g] = qsc[mt] * static_cast<float>(S);
      }
  }
  // Whole triples (pairs) of pages in a loop with one exit, then the last one or two: with
  // a single back edge the compiler's wait for a page covers only that page, and the next
  // one keeps loading.
  int i = 0;
  if constexpr (NB == 3) {
    for (; i + 3 <= n_mine; i += 3) {
      load_page(buf[2], next_of(i + 2), lane32, meta16);
      process(buf[0], ntok_of(i));
      load_page(buf[0], next_of(i + 3), lane32, meta16);
      process(buf[1], ntok_of(i + 1));
      load_page(buf[1], next_of(i + 4), lane32, meta16);
      process(buf[2], ntok_of(i + 2));
    }
    if (i < n_mine) {
      process(buf[0], ntok_of(i));
      if (i + 1 < n_mine) process(buf[1], ntok_of(i + 1));
    }
  } else {
    for (; i + 2 <= n_mine; i += 2) {
      process(buf[0], ntok_of(i));
      load_page(buf[0], next_of(i + 2), lane32, meta16);
      process(buf[1], ntok_of(i + 1));
      load_page(buf[1], next_of(i + 3), lane32, meta16);
    }
    if (i < n_mine) process(buf[0], ntok_of(i));
  }

  // R_V fragments of the un-rotation, requested now: they arrive while the waves' partials
  // are joined
  uint4 rb[8 / NW][4];
  if constexpr (kUnrot) merge::load_rv<NW>(rot_v, kv, rb);

  // ---- wave partials: lane (G, n) holds head 4mt + G, dims 16dt + n
  float accf[MT][8], lf[MT], zf[MT][NG];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (!fresh) flush_tile(mt, st.m[mt]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) accf[mt][dt] = flv(mt, dt);
    lf[mt] = flv(mt, 8);
#pragma unroll
    for (int q = 0; q < NG; ++q) zf[mt][q] = flv(mt, 9 + q);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int g = 4 * mt + G;
    const float l = row16_sum(lf[mt]);
    float zs[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) zs[q] = row16_sum(zf[mt][q]);
    if (g < GQ) {
      if (n == 0) {
        wm_s[wave][g] = st.m[mt];
        wl_s[wave][g] = l;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) wacc_s[wave][g][16 * dt + n] = accf[mt][dt] + zs[dt / (8 / NG)];
    }
  }
  __syncthreads();

  if constexpr (kUnrot) {
    // join the waves per (head, dim pair) into packed bf16 high / low A rows (the page
    // loop's LDS is free now), then un-rotate on the matrix cores and write
    static_assert(2 * 16 * merge::kARow * 4 <= kLoopBytes, "the A rows fit the loop's LDS");
    uint32_t* ahi_s = reinterpret_cast<uint32_t*>(scratch_s);
    uint32_t* alo_s = ahi_s + 16 * merge::kARow;
    for (int idx = tid; idx < GQ * (kHeadDim / 2); idx += 64 * NW) {
      const int g = idx / (kHeadDim / 2);
      const int dd = 2 * (idx % (kHeadDim / 2));
      float big = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) big = fmaxf(big, wm_s[w][g]);
      float l = 0.f, a0 = 0.f, a1 = 0.f;
      if (big != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float sc = wm_s[w][g] == -INFINITY ? 0.f : exp2f(wm_s[w][g] - big);
          l = fmaf(sc, wl_s[w][g], l);
          const float2 v = *reinterpret_cast<const float2*>(&wacc_s[w][g][dd]);
          a0 = fmaf(sc, v.x, a0);
          a1 = fmaf(sc, v.y, a1);
        }
      }
      merge::split2(a0, a1, ahi_s[g * merge::kARow + dd / 2], alo_s[g * merge::kARow + dd / 2]);
      if (dd == 0) {
        const size_t o = (static_cast<size_t>(b) * n_q + h0 + g) * pstride + split;
        store_partial<kCoherent>(out_m + o, big);
        store_partial<kCoherent>(out_l + o, l);
      }
    }
    __syncthreads();
    merge::unrotate_tiles<NW>(ahi_s, alo_s, GQ, rb, [&](int g, int d, float v) {
      const size_t o = (static_cast<size_t>(b) * n_q + h0 + g) * pstride + split;
      store_partial<kCoherent>(out_acc + o * kHeadDim + d, v);
    });
    return;
  }
  for (int idx = tid; idx < GQ * kHeadDim; idx += 64 * NW) {
    const int g = idx >> 7;
    const int dd = idx & 127;
    float big = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) big = fmaxf(big, wm_s[w][g]);
    float l = 0.f, a = 0.f;
    if (big != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float s = wm_s[w][g] == -INFINITY ? 0.f : exp2f(wm_s[w][g] - big);
        l = fmaf(s, wl_s[w][g], l);
        a = fmaf(s, wacc_s[w][g][dd], a);
      }
    }
    const size_t o = (static_cast<size_t>(b) * n_q + h0 + g) * pstride + split;
    store_partial<kCoherent>(out_acc + o * kHeadDim + dd, a);
    if (dd == 0) {
      store_partial<kCoherent>(out_m + o, big);
      store_partial<kCoherent>(out_l + o, l);
    }
  }
}

}  // namespace int2
}  // namespace oscar
