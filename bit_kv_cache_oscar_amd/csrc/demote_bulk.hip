// Bulk demotion (oscar_demote with many rows) on the matrix cores.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: tokens leaving the recent
// window are rotated, clipped, quantised and packed four 2-bit codes per byte into the INT2
// history, with a scale and zero point per group. The quantiser is the one demote_pass.h
// implements per row; this kernel reaches the same scales and codes for many rows at once.
//
// A workgroup (16 waves, one per CU) takes up to 2048 consecutive rows (tokens) of one
// (KV head, K or V) with R^T staged in LDS; a wave does one 16-token tile per iteration
// (kNT = 2 would give two tiles whose extremes, interval tests and exact sums are taken
// together, but at twice the registers: four waves per SIMD with one tile hide more
// latency than two waves with two):
//   y^T = R^T x^T as four 32-deep chunks on v_mfma_f32_16x16x32_bf16, each from a zero
//   accumulator, joined on the vector ALU as ((c0 + c1) + c2) + c3; lane (G, n) of a tile
//   holds dims 16 mt + 4 G + e (mt < 8, e < 4) of token n.
//
// Error of the fp32 values. A chunk is 32 exact products (a bf16 x bf16 product fits fp32)
// joined by at most 32 fp32 additions in whatever order and grouping the matrix core uses.
// Assuming only that each such addition lands within one fp32 ulp of its exact result (true
// of rounding to nearest, of truncation and of any faithful rounding) and that subnormal
// inputs and results may be flushed to zero, the classical bound for summation in any
// order (Higham, Accuracy and Stability of Numerical Algorithms, 2nd ed., section 4.2, with
// unit 2^-23 per addition) bounds a chunk's error by gamma_32 sum |p| over its products,
// gamma_32 < 32 2^-23 (1 + 2^-17); the three joins round to nearest (unit 2^-24), adding at
// most 3 2^-24 (1 + 2^-15) sum |p|, so 68 2^-24 sum |p| (plus 2^-116 for at most 259
// flushed products and partial sums of 2^-126 each) bounds a value's error. The sums
// S_j = sum_i |x_i| |R_ij| are bounded per group of 8 consecutive dims j: with
// M_gi = max over j in group g of |R_ij| (a bf16, exact), S_j <= T_g = sum_i |x_i| M_gi for
// every j of group g. The 16 T_g of a token come from the matrix cores (M |x^T|, one
// 128-deep accumulation, one 16-row tile): all their terms are >= 0, so in any order the
// fp32 result is within gamma_127 < 2^-16 of T_g (flushed products: at most 2^-119). Hence
//   delta = 68 2^-24 (1 + 2^-14) max_g T_g' + 2^-115
// bounds the error of every value of the token. The matrix cores' own summation order is
// thus never relied on, only this per-addition bound. (The group maxima make delta about
// 1.6 times the largest S_j on the workloads' rows, and more tokens take the fp64 path, but
// they cost 4 matrix products per tile where the S_j themselves cost 32 and the masking of
// every R^T fragment.)
//
// Scales and zero points (bit for bit the quantiser's):
//   - the exact extremes lie within delta of the fp32 ones and the quantiser's fp64 chain is
//     monotone in both: when both ends of those intervals round to the same fp16 scale and
//     zero point (evaluated in fp32 with outward margins), those are the values;
//   - otherwise the candidates (values within 3 delta of an fp32 extreme) are summed again
//     in fp64 from the exact products, 16 lanes per sum, one 16-lane group per (undecided
//     token, side), two tokens at a time (|error| <= 11 2^-53 sum |p| < 2^-31 delta), and the
//     same test runs in fp64;
//   - when even that interval holds an fp16 rounding boundary, compensated (two-sum) sums
//     over the wave give the extremes and the chain runs on them.
// Codes: from the fp32 values, except a value whose t = (y - z16) / s16 lies within the
// error bound of t of a rounding boundary (exact ties included): it is summed again in
// fp64 and decided on that interval, and by a compensated sum when the interval still
// holds the boundary, so ties round to even as the quantiser says. A token whose bound on
// t exceeds 2^-7 (its range tiny next to its norm) has all 128 values summed with
// compensation instead.
// With a codebook (the Lloyd-Max variant) the scale, zero point and every interval test are
// the same, and each code is the nearest codebook level of t instead (boundaries: the
// midpoints between levels).
// Packing goes through LDS: K words are a token's 16 consecutive dims, V words a dim's 16
// consecutive slots; a tile whose 16 tokens fill slots 16u..16u+15 of one page in order
// writes whole V words, any other tile merges its V codes into the shared words with 32-bit
// atomic and / or.

#include "demote_pass.h"

namespace oscar {
namespace {

constexpr int kNT = 1;                                   // 16-token tiles per wave and iteration
constexpr int kTokIter = 16 * kNT;                       // tokens per wave and iteration
constexpr int kBWaves = 16;                              // waves per workgroup
constexpr int kIters = 8;                                // iterations per wave
constexpr int kRowsPerBlock = kBWaves * kTokIter * kIters;
static_assert(kNT == 1 || kNT == 2, "tile bits of the candidate masks: two tiles at most");
constexpr int kRTRow = kHeadDim + 8;                   // bf16 per LDS row of R^T (16 bytes of bank spread)
constexpr int kXRow = kHeadDim + 8;                    // bf16 per LDS row of x (the same spread)
constexpr int kKRow = kHeadDim + 16;                   // bytes per token of the K code stage (bank spread)
constexpr float kGammaS = 68.f * 0x1p-24f * (1.f + 0x1p-14f);  // per computed sum |p|: the chunks, the joins, S's own error
constexpr float kFullT = 0x1p-7f;                      // bound on t above which a token is summed exactly

struct BulkSmem {
  uint16_t rt[kHeadDim * kRTRow];             // R^T: row j holds column j of R
  uint16_t xs[kBWaves][kNT][16 * kXRow];     // per wave, the x rows of the iteration's tiles (bf16 [16][kXRow] each)
  unsigned char cs[kBWaves][16 * kKRow];     // per wave, the codes of the current tile
  uint16_t gt[16 * kRTRow];                  // M: row g, column i holds max_{j in 8g..8g+7} |R_ij| (bf16)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// LDS-qualified types for the out-of-line helpers: through plain pointers their LDS accesses
// would compile to flat memory operations
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t ld1(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint32_t ld1(const lds_u16* p) { return *(const __attribute__((address_space(3))) uint32_t*)(p); }
__device__ __forceinline__ uint4 ld4(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 ld4(const lds_u16* p) {
  const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ double bf16lo(uint32_t w) { return static_cast<double>(__uint_as_float(w << 16)); }
__device__ __forceinline__ double bf16hi(uint32_t w) { return static_cast<double>(__uint_as_float(w & 0xFFFF0000u)); }

// fp16 bits -> double (exact)
__device__ __forceinline__ double h2d(uint16_t h) { return f16_bits_to_f64(h); }

// the quantiser's scale / zero-point chain on exact extremes (fp64, each operation rounded
// on its own)
__device__ __forceinline__ void scale_zero(double cr, double ymax, double ymin, uint16_t& s16, uint16_t& z16) {
#pragma clang fp contract(off)
  const double hi = cr * ymax;
  const double lo = cr * ymin;
  const double sc = (hi - lo) / 3.0;
  s16 = f64_to_f16_rne(sc);
  z16 = f64_to_f16_rne(lo);
}

// sum_i x_i R_ij in fp64 from the exact products, by the whole wave: lane L takes i = 2L, 2L+1
// and the 64 (sum, compensation) pairs are joined by two-sum steps; every lane gets the
// result (within 2^-52 of it plus 2^-100 sum |p| of the exact sum)
template <typename P>
__device__ __forceinline__ double coop_dot(P xrow, P rtrow, int lane) {
#pragma clang fp contract(off)
  const uint32_t xv = ld1(xrow + 2 * lane);
  const uint32_t rv = ld1(rtrow + 2 * lane);
  double s = bf16lo(xv) * bf16lo(rv);
  double c = 0.0;
  demote::two_sum_add(s, c, bf16hi(xv) * bf16hi(rv));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double so = __shfl_xor(s, o, 64);
    const double co = __shfl_xor(c, o, 64);
    c += co;
    demote::two_sum_add(s, c, so);
  }
  return s + c;
}

// a 64-bit value through a DPP row operation (both halves with the same control)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                                     static_cast<uint32_t>(lo)));
}

// y_j of one x row for the dim j of this lane's 16-lane group: lane q of the group takes
// i = 8q .. 8q + 7, the exact products are summed in fp64 in the lane and over the group by
// DPP (eleven rounded additions, |error| <= 11 2^-53 sum_i |x_i R_ij|); every lane of the
// group gets the sum
template <typename P>
__device__ __forceinline__ double group_dot(P xrow, P rtrow, int q) {
#pragma clang fp contract(off)
  const uint4 xv = ld4(xrow + 8 * q);
  const uint4 rv = ld4(rtrow + 8 * q);
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
  // fma: each product is exact in fp64, so the fused step rounds exactly as a sum does
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s = fma(bf16lo(xw[k]), bf16lo(rw[k]), s);
    s = fma(bf16hi(xw[k]), bf16hi(rw[k]), s);
  }
  s += dpp_f64<kDppQuadXor1>(s);
  s += dpp_f64<kDppQuadXor2>(s);
  s += dpp_f64<kDppHalfMirror>(s);
  s += dpp_f64<kDppMirror>(s);
  return s;
}

__device__ __forceinline__ double lane_f64(double v, int src) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), src);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), src);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), src);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// the fp32 neighbours of a finite fp32 value (one unit in the last place down / up)
__device__ __forceinline__ float f32_prev(float f) {
  const int b = __float_as_int(f);
  return f > 0.f ? __int_as_float(b - 1) : (f < 0.f ? __int_as_float(b + 1) : -__int_as_float(1));
}
__device__ __forceinline__ float f32_next(float f) {
  const int b = __float_as_int(f);
  return f > 0.f ? __int_as_float(b + 1) : (f < 0.f ? __int_as_float(b - 1) : __int_as_float(1));
}

// an fp32 value at or below / at or above the fp64 value x (|x| below the fp32 range)
__device__ __forceinline__ float f32_down(double x) {
  const float f = static_cast<float>(x);
  return static_cast<double>(f) > x ? f32_prev(f) : f;
}
__device__ __forceinline__ float f32_up(double x) {
  const float f = static_cast<float>(x);
  return static_cast<double>(f) < x ? f32_next(f) : f;
}

// fp16 bits of an fp32 value, rounded to nearest even by the hardware conversion
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ bool f16_finite(uint16_t h) { return (h & 0x7C00u) != 0x7C00u; }

// exact code of value y (fp64) under (s16, z16), as the quantiser defines it: uniform
// levels for lv == 0, else the nearest level of codebook word lv; every code is 0 when the
// scale is 0 or the scale or zero point overflowed fp16
__device__ __forceinline__ uint32_t exact_code(double y, uint16_t s16, uint16_t z16, uint32_t lv) {
#pragma clang fp contract(off)
  const double s = h2d(s16);
  if (s == 0.0 || !f16_finite(s16) || !f16_finite(z16)) return 0u;
  const double tq = (y - h2d(z16)) / s;
  if (lv != 0u) return static_cast<uint32_t>(codebook_code(tq, lv));
  const double t = rint(tq);
  return t < 0.0 ? 0u : (t > 3.0 ? 3u : static_cast<uint32_t>(t));
}

// distance from t to the nearest decision boundary of the code: the level midpoints of
// codebook word lv, or 0.5, 1.5, 2.5 for the uniform levels
template <typename T>
__device__ __forceinline__ T boundary_gap(T t, uint32_t lv) {
  if (lv != 0u) {
    const T th0 = static_cast<T>(static_cast<int>((lv & 0xFFu) + ((lv >> 8) & 0xFFu))) * static_cast<T>(0.03125);
    const T th1 = static_cast<T>(static_cast<int>(((lv >> 8) & 0xFFu) + ((lv >> 16) & 0xFFu))) * static_cast<T>(0.03125);
    const T th2 = static_cast<T>(static_cast<int>(((lv >> 16) & 0xFFu) + (lv >> 24))) * static_cast<T>(0.03125);
    return fmin(fmin(fabs(t - th0), fabs(t - th1)), fabs(t - th2));
  }
  const T b = fmin(fmax(floor(t) + static_cast<T>(0.5), static_cast<T>(0.5)), static_cast<T>(2.5));
  return fabs(t - b);
}

// Byte offset of token n, dim j in a tile's code stage: K codes token-major, V dim-major.
__device__ __forceinline__ int code_pos(bool is_v, int n, int j) { return is_v ? j * 16 + n : n * kKRow + j; }

// Dim of candidate bit b (= 4 mt + e) of a lane in lane group G.
__device__ __forceinline__ int dim_of(int b, int G) { return 16 * (b >> 2) + 4 * G + (b & 3); }

// Extremes of the undecided tokens of an iteration's tiles from their candidates:
// bits 32 tt + 4 mt + e of cmax / cmin are this lane's candidates in tile tt (its token n,
// its lane group's dims); xs2 holds the x rows of the tiles (tile tt, token n at row
// 16 tt + n). Every lane's masks go into `stage`; 16-lane groups 2k and 2k + 1 then take the
// token with candidates of rank 2r + k among the iteration's in round r, group 2k its cmax
// side and group 2k + 1 its cmin side: the group reads the token's four masks of its side and
// sums those candidates one at a time in fp64 (group_dot), keeping the largest (smallest);
// the token's lanes read both back from `stage`. (An open token has one candidate per side
// as a rule, so a round costs one sum per group.) Returns them per tile in every lane of a
// token. Out of line: its registers stay out of the kernel's main loop.
struct Extremes {
  double emax[2], emin[2];
};
constexpr int kStageMasks = 64 * 16;  // bytes: each lane's (cmax, cmin)
constexpr int kStageExt = 32 * 16;    // bytes: each token's (max, min)
static_assert(kStageMasks + kStageExt <= 16 * kKRow, "the candidate masks and extremes fit a wave's code stage");
__device__ __attribute__((noinline)) Extremes candidate_extremes(const lds_u16* xs2, const lds_u16* rt,
                                                                 uint64_t cmax, uint64_t cmin, lds_u8* stage) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  __attribute__((address_space(3))) uint64_t* masks = (__attribute__((address_space(3))) uint64_t*)(stage);
  __attribute__((address_space(3))) double* ext = (__attribute__((address_space(3))) double*)(stage + kStageMasks);
  masks[2 * lane] = cmax;
  masks[2 * lane + 1] = cmin;
  // the tokens with candidates: bit 16 tt + n (wave-uniform)
  uint32_t toks = 0u;
#pragma unroll
  for (int tt = 0; tt < kNT; ++tt) {
    const uint64_t m = __ballot(static_cast<uint32_t>((cmax | cmin) >> (32 * tt)) != 0u);
    toks |= static_cast<uint32_t>((m | (m >> 16) | (m >> 32) | (m >> 48)) & 0xFFFFull) << (16 * tt);
  }
  // (the wave's LDS operations run in order: the reads below see the writes above)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int side = g & 1;  // 0: the cmax candidates, 1: the cmin candidates
  while (toks) {
    // this round's two tokens, one per pair of lane groups (wave-uniform picks)
    const int p0 = __builtin_ctz(toks);
    toks &= toks - 1u;
    const int p1 = toks ? __builtin_ctz(toks) : -1;
    if (toks) toks &= toks - 1u;
    const int m = g < 2 ? p0 : p1;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    if (m >= 0) {
      const int tt = m >> 4, n = m & 15;
#pragma unroll
      for (int G = 0; G < 4; ++G) c[G] = static_cast<uint32_t>(masks[2 * (16 * G + n) + side] >> (32 * tt));
    }
    double e = side ? INFINITY : -INFINITY;
    const int xoff = (m < 0 ? 0 : m) * kXRow;
    for (;;) {
      // the group's next candidate: lane group G of the token, value bit b
      int G = -1;
      uint32_t u = 0u;
#pragma unroll
      for (int k = 3; k >= 0; --k)
        if (c[k]) {
          G = k;
          u = c[k];
        }
      if (!__any(G >= 0)) break;
      if (G >= 0) {
        const int b = __builtin_ctz(u);
        // (an opaque row offset: the row's loads and conversions hoisted out of the loop
        // would hold registers that the caller then saves around every call)
        int xo = xoff;
        asm volatile("" : "+v"(xo));
        const double y = group_dot(xs2 + xo, rt + dim_of(b, G) * kRTRow, lane & 15);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k == G) c[k] &= c[k] - 1u;
        e = side ? fmin(e, y) : fmax(e, y);
      }
    }
    if (m >= 0 && (lane & 15) == 0) ext[2 * m + side] = e;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  Extremes r;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    r.emax[tt] = -INFINITY;
    r.emin[tt] = INFINITY;
  }
#pragma unroll
  for (int tt = 0; tt < kNT; ++tt) {
    const int m = 16 * tt + (lane & 15);
    r.emax[tt] = ext[2 * m];
    r.emin[tt] = ext[2 * m + 1];
  }
  return r;
}

// Codes of the flagged values of a tile (flags: this lane's bits (mt, e)), decided from
// fp64 sums on an interval, and from compensated sums where that interval holds the
// boundary; written into the tile's code stage. sz: this lane's packed (s16, z16); dl: its
// token's error bound.
__device__ __attribute__((noinline)) void fix_codes(const lds_u16* xs, const lds_u16* rt, lds_u8* cs,
                                                    uint32_t flags, uint32_t sz, float dl, bool is_v, uint32_t lv) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  uint64_t lanes = __ballot(flags != 0u);
  while (lanes) {
    int js[4], ns[4], owner[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      owner[r] = -1;
      js[r] = 0;
      ns[r] = 0;
      if (lanes) {
        const int ls = __builtin_ctzll(lanes);
        const uint32_t fm = __builtin_amdgcn_readlane(flags, ls);
        const int b = __builtin_ctz(fm);
        if (lane == ls) flags &= flags - 1u;
        lanes = __ballot(flags != 0u);
        owner[r] = ls;
        ns[r] = ls & 15;
        js[r] = dim_of(b, ls >> 4);
      }
    }
    const int g = lane >> 4;
    const int jg = g == 0 ? js[0] : (g == 1 ? js[1] : (g == 2 ? js[2] : js[3]));
    const int ng = g == 0 ? ns[0] : (g == 1 ? ns[1] : (g == 2 ? ns[2] : ns[3]));
    const double y = group_dot(xs + ng * kXRow, rt + jg * kRTRow, lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (owner[r] < 0) continue;
      // wave-uniform from here: the value, its token's scale, zero point and bound
      const double yr = lane_f64(y, 16 * r);
      const uint32_t szr = __builtin_amdgcn_readlane(sz, owner[r]);
      const float dlr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dl), owner[r]));
      const uint16_t s16 = static_cast<uint16_t>(szr & 0xFFFFu);
      const uint16_t z16 = static_cast<uint16_t>(szr >> 16);
      const double s = h2d(s16);
      const double t = (yr - h2d(z16)) / s;
      // the fp64 sum is within 11 2^-53 sum|p| < 2^-31 dl of the exact value; two more
      // roundings for t
      const double bnd = static_cast<double>(dlr) * 0x1p-31 / s + 0x1p-50 * (fabs(t) + 1.0);
      uint32_t q;
      if (boundary_gap(t, lv) > bnd) {
        // the exact t lies on the same side of every boundary as this one
        if (lv == 0u) {
          const double r = rint(t);
          q = r < 0.0 ? 0u : (r > 3.0 ? 3u : static_cast<uint32_t>(r));
        } else {
          q = static_cast<uint32_t>(codebook_code(t, lv));
        }
      } else {
        const double ye = coop_dot(xs + ns[r] * kXRow, rt + js[r] * kRTRow, lane);
        q = exact_code(ye, s16, z16, lv);
      }
      if (lane == 0) cs[code_pos(is_v, ns[r], js[r])] = static_cast<unsigned char>(q);
    }
  }
}

// Every value of the tile's token nf summed with compensation (lane L: dims L and L + 64);
// its extremes give the scale and zero point and each value its code, written into the
// code stage. Returns the packed (s16, z16) (wave-uniform).
__device__ __attribute__((noinline)) uint32_t full_token(const lds_u16* xs, const lds_u16* rt, lds_u8* cs,
                                                         int nf, double cr, bool is_v, uint32_t lv) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const lds_u16* xrow = xs + nf * kXRow;
  double yv[2];
  double ymx = -INFINITY, ymn = INFINITY;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    const lds_u16* rr = rt + j * kRTRow;
    double s = 0.0, c = 0.0;
    for (int i = 0; i < kHeadDim; i += 8) {
      const uint4 xv = ld4(xrow + i);
      const uint4 rv = ld4(rr + i);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        demote::two_sum_add(s, c, bf16lo(xw[k]) * bf16lo(rw[k]));
        demote::two_sum_add(s, c, bf16hi(xw[k]) * bf16hi(rw[k]));
      }
    }
    yv[h] = s + c;
    ymx = fmax(ymx, yv[h]);
    ymn = fmin(ymn, yv[h]);
  }
  ymx = wave_max(ymx);
  ymn = wave_min(ymn);
  uint16_t s16, z16;
  scale_zero(cr, ymx, ymn, s16, z16);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    cs[code_pos(is_v, nf, j)] = static_cast<unsigned char>(exact_code(yv[h], s16, z16, lv));
  }
  return static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16);
}

// CB: the Lloyd-Max codebook variant (codebook words [n_kv][K, V])
template <bool CB>
__global__ __launch_bounds__(64 * kBWaves) void demote_bulk_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int n, int n_kv,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ dst_slot,
    const uint16_t* __restrict__ rot_k, const uint16_t* __restrict__ rot_v, const float* __restrict__ clip_k,
    const float* __restrict__ clip_v, uint8_t* __restrict__ pool, const uint32_t* __restrict__ codebook) {
  __shared__ __align__(16) BulkSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_ = lane & 15;  // MFMA column: token of the tile
  const int G = lane >> 4;   // lane group: dims 4 G .. 4 G + 3 of each 16-dim tile
  const int head = blockIdx.y;
  const int is_v = blockIdx.z;
  const uint16_t* src = is_v ? v_src : k_src;
  const uint16_t* rot = (is_v ? rot_v : rot_k) + static_cast<size_t>(head) * kHeadDim * kHeadDim;
  const double cr = static_cast<double>(is_v ? clip_v[head] : clip_k[head]);
  const uint32_t lv = CB ? codebook[2 * head + is_v] : 0u;  // codebook word (0: uniform levels)
  const size_t head_stride = static_cast<size_t>(n_kv) * kHeadDim;  // elements between tokens
  const int meta_off = is_v ? kVMeta : kKMeta;

  // x fragments (B operand) of one iteration: lane (G, n) holds token tb + 16 tt + n,
  // elements 32 ks + 8 G .. + 7 (tokens past the end read the last row; nothing of theirs is
  // stored), with the tokens' destination page and slot
  uint4 bx[kNT][4];
  int pg[kNT], sl[kNT];
  auto load_iter = [&](int it) {
    const int tb = blockIdx.x * kRowsPerBlock + (it * kBWaves + wave) * kTokIter;
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
      const int t = min(tb + 16 * tt + n_, n - 1);
      const uint16_t* xr = src + static_cast<size_t>(t) * head_stride + static_cast<size_t>(head) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bx[tt][ks] = *reinterpret_cast<const uint4*>(xr + 32 * ks + 8 * G);
      pg[tt] = dst_page[t];
      sl[tt] = dst_slot[t];
    }
  };
  const int tb0 = blockIdx.x * kRowsPerBlock + wave * kTokIter;
  if (tb0 < n) load_iter(0);  // in flight while R^T is staged

  // R^T into LDS: thread (i, half) of the first 256 copies row i, columns 64 half .. + 63
  if (tid < 256) {
    const int i = tid >> 1;
    const int c0 = 64 * (tid & 1);
    const uint4* rrow = reinterpret_cast<const uint4*>(rot + i * kHeadDim + c0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = rrow[q];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = c0 + 8 * q + 2 * k;
        sm.rt[j * kRTRow + i] = static_cast<uint16_t>(w4[k] & 0xFFFFu);
        sm.rt[(j + 1) * kRTRow + i] = static_cast<uint16_t>(w4[k] >> 16);
      }
    }
  }
  __syncthreads();
  // the group maxima of |R^T| (magnitude order of bf16 is the integer order of its bits
  // with the sign cleared)
  for (int e = tid; e < 16 * kHeadDim; e += 64 * kBWaves) {
    const int g = e / kHeadDim, i = e % kHeadDim;
    uint16_t m = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint16_t v = sm.rt[(8 * g + r) * kRTRow + i] & 0x7FFFu;
      m = v > m ? v : m;
    }
    sm.gt[g * kRTRow + i] = m;
  }
  __syncthreads();
  unsigned char* cs = sm.cs[wave];

  for (int it = 0; it < kIters; ++it) {
    const int tb = blockIdx.x * kRowsPerBlock + (it * kBWaves + wave) * kTokIter;  // first token of the iteration
    if (tb >= n) break;  // wave-uniform (this iteration's rows were requested before R^T was
                         // staged, or by the iteration before)
    // this iteration's rows into LDS (for the exact paths), and |x| beside them
    int cpg[kNT], csl[kNT];
    uint4 bxa[kNT][4];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        *reinterpret_cast<uint4*>(sm.xs[wave][tt] + n_ * kXRow + 32 * ks + 8 * G) = bx[tt][ks];
        bxa[tt][ks] = make_uint4(bx[tt][ks].x & 0x7FFF7FFFu, bx[tt][ks].y & 0x7FFF7FFFu, bx[tt][ks].z & 0x7FFF7FFFu,
                                 bx[tt][ks].w & 0x7FFF7FFFu);
      }
      cpg[tt] = pg[tt];
      csl[tt] = sl[tt];
    }
    float smax[kNT];
    // The token's error bound: T = M |x^T| (row g: the sum of |x_i| times the group maxima
    // of |R_ij|, at least S_j for every dim j of group g) from one 128-deep accumulation, whose
    // terms are all >= 0, so the fp32 result is within gamma_127 < 2^-16 of T whatever the
    // order (products below the fp32 range flushed: at most 2^-119 in all).
    // dl = 68 2^-24 max T (1 + 2^-14) + 2^-115 then holds for every value of the token.
    {
      f32x4 sb[kNT];
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) sb[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 ga = *reinterpret_cast<const uint4*>(sm.gt + n_ * kRTRow + 32 * ks + 8 * G);
#pragma unroll
        for (int tt = 0; tt < kNT; ++tt)
          sb[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ga),
                                                          __builtin_bit_cast(bf16x8, bxa[tt][ks]), sb[tt], 0, 0, 0);
      }
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt)
        smax[tt] = fmaxf(fmaxf(sb[tt][0], sb[tt][1]), fmaxf(sb[tt][2], sb[tt][3]));
    }
    // y^T = R^T x^T: rows dims 16 mt + 4 G + e, column token n; four chunks from zero,
    // joined in a fixed order with rounding to nearest.
    f32x4 acc[8][kNT];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 ch[4][kNT];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(sm.rt + (16 * mt + n_) * kRTRow + 32 * ks + 8 * G);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < kNT; ++tt) {
          ch[ks][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, bx[tt][ks]), z, 0, 0, 0);
        }
      }
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) {
#pragma clang fp contract(off)
        acc[mt][tt] = ((ch[0][tt] + ch[1][tt]) + ch[2][tt]) + ch[3][tt];
      }
    }
    // ---- the iteration's tiles: extremes, norms, error bounds and the fp32 interval test of
    // the scale and zero point
    float mx[kNT], mn[kNT], dl[kNT];
    bool valid[kNT], known[kNT], full[kNT];
    uint16_t s16[kNT], z16[kNT];
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
      valid[tt] = tb + 16 * tt + n_ < n;
      float a = -INFINITY, b = INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a = fmaxf(a, acc[mt][tt][e]);
          b = fminf(b, acc[mt][tt][e]);
        }
      mx[tt] = a;
      mn[tt] = b;
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1)
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) {
        mx[tt] = fmaxf(mx[tt], __shfl_xor(mx[tt], o, 64));
        mn[tt] = fminf(mn[tt], __shfl_xor(mn[tt], o, 64));
        smax[tt] = fmaxf(smax[tt], __shfl_xor(smax[tt], o, 64));
      }
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
#pragma clang fp contract(off)
      // the bound of every fp32 value of this token (fp32 rounding of the product and sum
      // covered by the factor 1 + 2^-14 in kGammaS)
      dl[tt] = fmaf(kGammaS, smax[tt], 0x1p-115f);
      // The exact extremes lie within dl of mx and mn; the chain below evaluates the
      // quantiser's steps on those ends in fp32 and widens the results by more than every
      // rounding of either evaluation (fp32 here, fp64 in the quantiser), so they bound the
      // true scale and zero point. Rounding to fp16 is monotone: equal ends mean a determined
      // value.
      const float d = dl[tt];
      const float c32 = static_cast<float>(cr);
      s16[tt] = z16[tt] = 0;
      known[tt] = false;
      full[tt] = false;
      if (cr > 0.0 && d < INFINITY && mx[tt] != -INFINITY) {
        const float hA = c32 * (mx[tt] - d), hB = c32 * (mx[tt] + d);
        const float lC = c32 * (mn[tt] - d), lD = c32 * (mn[tt] + d);
        const float ms = 0x1p-21f * (fabsf(hB) + fabsf(lC)) + 0x1p-140f;
        const float mz = 0x1p-21f * fabsf(lC) + 0x1p-140f;
        const float sLo = (hA - lD) * (1.f / 3.f) - ms, sHi = (hB - lC) * (1.f / 3.f) + ms;
        s16[tt] = f32_to_f16_bits(sLo);
        z16[tt] = f32_to_f16_bits(lC - mz);
        known[tt] = sLo >= 0.f && s16[tt] == f32_to_f16_bits(sHi) && z16[tt] == f32_to_f16_bits(lD + mz);
      } else {
        full[tt] = true;  // a clip ratio of 0 or less, or a non-finite row: every value exact
      }
      if (!valid[tt]) {  // nothing to do for tokens past the end
        known[tt] = true;
        full[tt] = false;
      }
    }

    // ---- the undecided tokens of the tiles: their candidates' fp64 sums, then the same
    // test in fp64; compensated sums when even that leaves the fp16 values open
    bool und[kNT];
    bool any_und = false;
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
      und[tt] = !known[tt] && !full[tt];
      any_und = any_und || und[tt];
    }
    if (__any(any_und)) {
      uint64_t cmax = 0ull, cmin = 0ull;
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) {
        // candidates: values within 3 dl of an fp32 extreme (the thresholds' own rounding is
        // below dl / 256, so this holds every value within 2 dl of the exact extreme)
        const float thi = und[tt] ? mx[tt] - 3.f * dl[tt] : INFINITY;
        const float tlo = und[tt] ? mn[tt] + 3.f * dl[tt] : -INFINITY;
        uint32_t a = 0u, b = 0u;
        if (__any(und[tt])) {  // (a tile with no undecided token has no candidates)
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a |= acc[mt][tt][e] >= thi ? (1u << (4 * mt + e)) : 0u;
              b |= acc[mt][tt][e] <= tlo ? (1u << (4 * mt + e)) : 0u;
            }
        }
        // a token with more than two candidates on one side in one lane (a range comparable
        // to its bound) takes the full path instead
        const uint64_t many = __ballot(und[tt] && (__builtin_popcount(a) > 2 || __builtin_popcount(b) > 2));
        const uint32_t toks = static_cast<uint32_t>((many | (many >> 16) | (many >> 32) | (many >> 48)) & 0xFFFFull);
        if ((toks >> n_) & 1u) {
          full[tt] = true;
          a = b = 0u;
        }
        cmax |= static_cast<uint64_t>(a) << (32 * tt);
        cmin |= static_cast<uint64_t>(b) << (32 * tt);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const Extremes ce = candidate_extremes((const lds_u16*)sm.xs[wave][0], (const lds_u16*)sm.rt, cmax, cmin,
                                             (lds_u8*)cs);
      bool settled[kNT];
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) settled[tt] = true;
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) {
#pragma clang fp contract(off)
        if (!known[tt] && !full[tt]) {
          // the sums are within 11 2^-53 sum|p| < 2^-31 dl of the exact extremes; then room
          // for rounding the chain in fp64, and the fp16 decision on fp32 ends rounded outward
          const double emax = ce.emax[tt], emin = ce.emin[tt];
          const double d64 =
              static_cast<double>(dl[tt]) * 0x1p-31 + 0x1p-50 * fmax(fabs(emax), fabs(emin)) + 0x1p-1000;
          const double hA = cr * (emax - d64), hB = cr * (emax + d64);
          const double lC = cr * (emin - d64), lD = cr * (emin + d64);
          const double m = 0x1p-50 * (fabs(hB) + fabs(lC)) + 0x1p-1000;
          const double sLo = (hA - lD) * (1.0 / 3.0) - m, sHi = (hB - lC) * (1.0 / 3.0) + m;
          s16[tt] = f32_to_f16_bits(f32_down(sLo));
          z16[tt] = f32_to_f16_bits(f32_down(lC - m));
          settled[tt] = sLo >= 0.0 && s16[tt] == f32_to_f16_bits(f32_up(sHi)) &&
                        z16[tt] == f32_to_f16_bits(f32_up(lD + m));
        }
      }
      // the vanishing remainder: compensated sums of the candidates, token by token
      uint64_t rest = 0ull;
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) rest |= __ballot(!settled[tt] && G == 0) << (16 * tt);
      while (rest) {
        const int m = __builtin_ctzll(rest);  // token 16 tt + n of the iteration
        rest &= rest - 1;
        const int tt = m >> 4;
        const int nf = m & 15;
        double ex = -INFINITY, en = INFINITY;
        for (int g = 0; g < 4; ++g) {
          const int ls = 16 * g + nf;
          const uint32_t cxm = static_cast<uint32_t>(lane_u64(cmax, ls) >> (32 * tt));
          const uint32_t cnm = static_cast<uint32_t>(lane_u64(cmin, ls) >> (32 * tt));
          uint32_t cm = cxm | cnm;
          while (cm) {
            const int b = __builtin_ctz(cm);
            cm &= cm - 1u;
            const double y = coop_dot(sm.xs[wave][tt] + nf * kXRow, sm.rt + dim_of(b, g) * kRTRow, lane);
            if ((cxm >> b) & 1u) ex = fmax(ex, y);
            if ((cnm >> b) & 1u) en = fmin(en, y);
          }
        }
        uint16_t a16, b16;
        scale_zero(cr, ex, en, a16, b16);
#pragma unroll
        for (int t2 = 0; t2 < kNT; ++t2)
          if (n_ == nf && t2 == tt) {
            s16[t2] = a16;
            z16[t2] = b16;
          }
      }
    }

    // the next iteration's rows: they load while this iteration's codes are made and stored
    if (it + 1 < kIters && tb + kBWaves * kTokIter < n) load_iter(it + 1);

    // ---- per tile: codes, the exact decisions near boundaries, packing and stores
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
      const int t0 = tb + 16 * tt;  // first token of the tile
      if (t0 >= n) break;           // wave-uniform
      const uint16_t* xs = sm.xs[wave][tt];
      const int page = cpg[tt];
      const int slot = csl[tt];

      // codes of this lane's 32 values: v = (y - z16) / s16 as one fused step (|v - t| <=
      // dt + (8 + 4.1 |z16 / s16|) 2^-24 near a boundary), the code v on [0, 3] rounded to
      // nearest by the packing conversion (v_cvt_pk_u8_f32 rounds to nearest: a GPU test
      // pins it on every bf16 value of t from 1/4 to 3); values with v within bt of a
      // half-integer may lie on the other side of it than the exact value and take the exact
      // path, which also rounds exact ties to even (-1/2 and 7/2 are no boundaries: flagging
      // them only costs an exact sum)
      const float sf = f16_to_f32(s16[tt]);
      const float zf = f16_to_f32(z16[tt]);
      const bool usable = sf != 0.f && f16_finite(s16[tt]) && f16_finite(z16[tt]);
      const float inv_s = usable ? 1.f / sf : 0.f;
      const float zs = zf * inv_s;
      const float cb = -zs;
      const float dt = dl[tt] * inv_s * (1.f + 0x1p-20f);
      bool fullt = full[tt] || (valid[tt] && usable && dt > kFullT);
      const float bt = (valid[tt] && usable && !fullt) ? dt + (1.f + 0.6f * fabsf(zs)) * 0x1p-21f : -1.f;
      float gmax = 0.f;  // codebook: largest closeness to a boundary of this lane's values
      float gmin = 1.f;  // uniform levels: smallest distance to a half-integer
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = fmaf(acc[mt][tt][e], inv_s, cb);
          if constexpr (CB) {
            w |= static_cast<uint32_t>(codebook_code(v, lv)) << (8 * e);
            gmax = fmaxf(gmax, 1.f - boundary_gap(v, lv));
          } else {
            w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(v, 0.f, 3.f), e, w);
            gmin = fminf(gmin, fabsf(__builtin_amdgcn_fractf(v) - 0.5f));
          }
        }
        if (!usable) w = 0u;
        if (!is_v) {
          *reinterpret_cast<uint32_t*>(cs + n_ * kKRow + 16 * mt + 4 * G) = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[(16 * mt + 4 * G + e) * 16 + n_] = static_cast<unsigned char>(w >> (8 * e));
        }
      }
      // uniform levels: |fract(v) - 1/2| <= bt means v within bt of a half-integer (exact for
      // fract(v) >= 1/4, and at least 1/4 otherwise); the codebook's 1 - gap >= 1 - bt means
      // v within bt of a level midpoint
      const bool flagged = CB ? (gmax >= 1.f - bt) : (gmin <= bt);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      uint32_t sz = static_cast<uint32_t>(s16[tt]) | (static_cast<uint32_t>(z16[tt]) << 16);
      if (__any(flagged && bt >= 0.f)) {
        // which of this lane's values: the same v again
        uint32_t flags = 0u;
        if (flagged && bt >= 0.f) {
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = fmaf(acc[mt][tt][e], inv_s, cb);
              bool near;
              if constexpr (CB) {
                near = boundary_gap(v, lv) <= bt;
              } else {
                near = fabsf(__builtin_amdgcn_fractf(v) - 0.5f) <= bt;
              }
              if (near) flags |= 1u << (4 * mt + e);
            }
        }
        fix_codes((const lds_u16*)xs, (const lds_u16*)sm.rt, (lds_u8*)cs, flags, sz, dl[tt], is_v, lv);
      }
      uint64_t fulls = __ballot(fullt && G == 0);
      while (fulls) {
        const int nf = __builtin_ctzll(fulls);
        fulls &= fulls - 1;
        const uint32_t r = full_token((const lds_u16*)xs, (const lds_u16*)sm.rt, (lds_u8*)cs, nf, cr, is_v, lv);
        if (n_ == nf) sz = r;
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);

      // scale and zero point of the token
      if (valid[tt] && G == 0) {
        uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * kHeadBlock;
        *reinterpret_cast<uint32_t*>(blk + meta_off + 4 * slot) = sz;
      }
      // the lane's store offsets are formed here from an opaque copy of the lane index:
      // offsets made once ahead of the loop would each hold a register through it (and spill)
      int lane_s = lane;
      asm volatile("" : "+v"(lane_s));
      if (!is_v) {
        // K words: word q = lane + 64 r is (token q / 8 of the tile, dims 16 (q % 8) ..)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int q = lane_s + 64 * r;
          const int tk = q >> 3;
          const int w = q & 7;
          // page and slot of the word's token from lane tk, which loaded them (every lane
          // of the wave takes part in the shuffles)
          const int pgw = __shfl(page, tk, 64);
          const int slw = __shfl(slot, tk, 64);
          if (t0 + tk < n) {
            const uint4 b = *reinterpret_cast<const uint4*>(cs + tk * kKRow + 16 * w);
            const uint32_t word = b.x | (b.y << 2) | (b.z << 4) | (b.w << 6);
            uint8_t* blk = pool + (static_cast<size_t>(pgw) * n_kv + head) * kHeadBlock;
            *reinterpret_cast<uint32_t*>(blk + k_word_offset(slw, w)) = word;
          }
        }
      } else {
        // V: whole words when the tile fills slots 16u..16u+15 of one page in order
        const int page0 = __shfl(page, 0, 64);
        const int slot0 = __shfl(slot, 0, 64);
        const bool mine_ok = valid[tt] && page == page0 && slot == (slot0 & ~15) + n_;
        const bool aligned = (slot0 & 15) == 0 && __ballot(G == 0 && mine_ok) == 0xFFFFull;
        if (aligned) {
          uint8_t* blk = pool + (static_cast<size_t>(page0) * n_kv + head) * kHeadBlock;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int d = lane_s + 64 * r;
            const uint4 b = *reinterpret_cast<const uint4*>(cs + d * 16);
            const uint32_t word = b.x | (b.y << 2) | (b.z << 4) | (b.w << 6);
            *reinterpret_cast<uint32_t*>(blk + v_word_offset(d, slot0 >> 4)) = word;
          }
        } else if (valid[tt]) {
          // this lane's 32 codes into their shared words, two bits each
          uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * kHeadBlock;
          const int rs = slot & 15;
          const int sh = 8 * (rs & 3) + 2 * (rs >> 2);
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int d = 16 * mt + 4 * G + e;
              uint32_t* w = reinterpret_cast<uint32_t*>(blk + v_word_offset(d, slot >> 4));
              atomicAnd(w, ~(3u << sh));
              atomicOr(w, static_cast<uint32_t>(cs[d * 16 + n_] & 3u) << sh);
            }
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  }
}

}  // namespace

hipError_t launch_demote_bulk(const LayerShape& L, const void* k_src, const void* v_src, int n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k,
                              const void* rot_v, const float* clip_k, const float* clip_v, void* pool,
                              hipStream_t stream, const uint32_t* codebook) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((n + kRowsPerBlock - 1) / kRowsPerBlock);
  if (codebook)
    hipLaunchKernelGGL(demote_bulk_kernel<true>, dim3(blocks, L.n_kv, 2), dim3(64 * kBWaves), 0, stream,
                       static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), n, L.n_kv, dst_page,
                       dst_slot, static_cast<const uint16_t*>(rot_k), static_cast<const uint16_t*>(rot_v), clip_k,
                       clip_v, static_cast<uint8_t*>(pool), codebook);
  else
    hipLaunchKernelGGL(demote_bulk_kernel<false>, dim3(blocks, L.n_kv, 2), dim3(64 * kBWaves), 0, stream,
                       static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), n, L.n_kv, dst_page,
                       dst_slot, static_cast<const uint16_t*>(rot_k), static_cast<const uint16_t*>(rot_v), clip_k,
                       clip_v, static_cast<uint8_t*>(pool), nullptr);
  return hipGetLastError();
}

}  // namespace oscar
