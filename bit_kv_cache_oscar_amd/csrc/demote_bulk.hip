// Bulk demotion (oscar_demote with many rows) on the matrix cores.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: tokens leaving the recent
// window are rotated, clipped, quantised and packed four 2-bit codes per byte into the INT2
// history, with a scale and zero point per group. The quantiser is the one demote_pass.h
// implements per row; this kernel reaches the same scales and codes for many rows at once.
//
// A workgroup (4 waves) takes up to 256 consecutive rows (tokens) of one (KV head, K or V)
// with R^T staged in LDS; a wave does 32 tokens per iteration as two 16-token tiles:
//   y^T = R^T x^T on v_mfma_f32_16x16x32_bf16 (bf16 products are exact, sums in fp32), so
//   lane (G, n) of a tile holds dims 16 mt + 4 G + e (mt < 8, e < 4) of token n.
// The fp32 sums differ from the exact ones by at most delta = 16 2^-24 |x| max_j |R_:,j|
// (Cauchy-Schwarz bounds sum_i |x_i R_ij| by |x| |R_:,j|; the matrix cores' fp32
// accumulation was measured below 2.3 2^-24 |x| |R_:,j|, and below 6.4 2^-24 sum |x_i R_ij|,
// on adversarial magnitude mixes, so 16 leaves a margin of 7).
// Scales and zero points are then fixed exactly:
//   - the exact extremes lie within delta of the fp32 ones; the fp64 chain of the quantiser
//     is monotone in both, so when both ends of that interval round to the same fp16 scale
//     and zero point, those are the values the exact extremes give;
//   - otherwise the candidates (dims within 2 delta of an fp32 extreme) are summed again in
//     fp64 from the exact products, four at a time (one per 16-lane group, a DPP tree), with
//     an error bound of its own, and the same interval test runs on those sums; when even
//     that leaves the fp16 values open, compensated (two-sum) sums across the wave give the
//     exact extremes and the chain runs on them.
// Codes come from the fp32 y when delta / s16 <= 9e-5, which keeps every code on the side of
// its rounding boundary the exact value is on unless the exact value lies within 1e-4 of
// the boundary; a token failing that test has all 128 values summed exactly instead.
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

constexpr int kBWaves = 4;
constexpr int kIters = 8;                              // 32-token iterations per wave
constexpr int kRowsPerBlock = kBWaves * 32 * kIters;   // 1024
constexpr int kRTRow = kHeadDim + 8;                   // bf16 per LDS row of R^T (16 bytes of bank spread)
constexpr double kAccUlps = 16.0;                      // fp32 accumulation budget, units of 2^-24 |x| max|R_:,j|
constexpr double kCodeSlack = 9e-5;                    // largest tolerated error of t = (y - z16) / s16

struct BulkSmem {
  uint16_t rt[kHeadDim * kRTRow];   // R^T: row j holds column j of R
  uint32_t stage[kBWaves][1024];    // per wave, one tile: x rows (bf16 [16][128]) or codes (bytes)
  uint32_t fb[kBWaves][16][8];      // per wave, one tile: exact 2-bit codes of tokens summed exactly
  float colmax2;                    // max_j |R_:,j|^2
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
// and the 64 (sum, compensation) pairs are joined by two-sum steps; every lane gets the result
__device__ __forceinline__ double coop_dot(const uint16_t* xrow, const uint16_t* rtrow, int lane) {
#pragma clang fp contract(off)
  const uint32_t xv = *reinterpret_cast<const uint32_t*>(xrow + 2 * lane);
  const uint32_t rv = *reinterpret_cast<const uint32_t*>(rtrow + 2 * lane);
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
__device__ __forceinline__ double group_dot(const uint16_t* xrow, const uint16_t* rtrow, int q) {
#pragma clang fp contract(off)
  const uint4 xv = *reinterpret_cast<const uint4*>(xrow + 8 * q);
  const uint4 rv = *reinterpret_cast<const uint4*>(rtrow + 8 * q);
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s += bf16lo(xw[k]) * bf16lo(rw[k]);
    s += bf16hi(xw[k]) * bf16hi(rw[k]);
  }
  s += dpp_f64<kDppQuadXor1>(s);
  s += dpp_f64<kDppQuadXor2>(s);
  s += dpp_f64<kDppHalfMirror>(s);
  s += dpp_f64<kDppMirror>(s);
  return s;
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

// exact code of value y (fp64) under (s16, z16), as the quantiser defines it: uniform
// levels for lv == 0, else the nearest level of codebook word lv
__device__ __forceinline__ uint32_t exact_code(double y, uint16_t s16, uint16_t z16, uint32_t lv) {
#pragma clang fp contract(off)
  const double s = h2d(s16);
  if (s == 0.0) return 0u;
  const double tq = (y - h2d(z16)) / s;
  if (lv != 0u) return static_cast<uint32_t>(codebook_code(tq, lv));
  const double t = rint(tq);
  return t < 0.0 ? 0u : (t > 3.0 ? 3u : static_cast<uint32_t>(t));
}

// Exact scale and zero point for the tokens of a tile listed in `todo` (bit n: token n of
// the tile), whose x rows are in xs (bf16 [16][128]); where fp32 values cannot give a
// token's codes, its exact codes go to fbw (2 bits per dim, 8 words per token). Per lane:
// cand = candidate bits (mt, e) of this lane's token, delta its error bound, sz its packed
// (s16, z16) so far. Returns the lane's (s16 | z16 << 16), with bit 32 set when its token's
// codes are in fbw. Out of line: the path is rare, and its registers stay out of the kernel's
// main loop.
__device__ __attribute__((noinline)) uint64_t exact_tokens(const uint16_t* xs, const uint16_t* rt, uint32_t* fbw,
                                                          uint64_t todo, uint32_t cand, double delta, uint32_t sz,
                                                          double cr, uint32_t lv) {
  const int lane = threadIdx.x & 63;
  const int n_ = lane & 15;
  uint16_t s16 = static_cast<uint16_t>(sz & 0xFFFFu);
  uint16_t z16 = static_cast<uint16_t>(sz >> 16);
  bool fbk = false;
  while (todo) {
    const int nf = __builtin_ctzll(todo);  // wave-uniform token of the tile
    todo &= todo - 1;
    const uint16_t* xrow = xs + nf * kHeadDim;
    const double fdl = __shfl(delta, nf, 64);
    uint32_t cnf = n_ == nf ? cand : 0u;
    // first fp64 sums of the candidates with an error bound of their own, four at a time;
    // the compensated sums only when that interval still leaves the fp16 results open
    const uint32_t cnf0 = cnf;
    double emax = -INFINITY, emin = INFINITY;
    uint64_t lanes = __ballot(cnf != 0u);
    while (lanes) {
      int js[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        js[r] = -1;
        if (lanes) {
          const int ls = __builtin_ctzll(lanes);
          const uint32_t cm = __builtin_amdgcn_readlane(cnf, ls);
          const int b = __builtin_ctz(cm);
          if (lane == ls) cnf &= cnf - 1u;
          lanes = __ballot(cnf != 0u);
          js[r] = 16 * (b >> 2) + 4 * (ls >> 4) + (b & 3);
        }
      }
      const int g = lane >> 4;
      const int jg = g == 0 ? js[0] : (g == 1 ? js[1] : (g == 2 ? js[2] : js[3]));
      const double y = group_dot(xrow, rt + (jg < 0 ? 0 : jg) * kRTRow, lane & 15);
      const uint64_t yu = static_cast<uint64_t>(__double_as_longlong(y));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (js[r] < 0) continue;
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(yu)), 16 * r);
        const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(yu >> 32)), 16 * r);
        const double yr = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
        emax = fmax(emax, yr);
        emin = fmin(emin, yr);
      }
    }
    uint16_t es16 = 0, ez16 = 0;
    bool known = false;
    if (cr > 0.0) {
#pragma clang fp contract(off)
      // sum |x_i R_ij| <= fdl 2^20 (fdl = 16 2^-24 times that bound), so the sums are within
      // 11 2^-53 2^20 fdl < 2^-28 fdl; then room for rounding the chain in fp64, and the fp16
      // decision on fp32 ends rounded outward
      const double d64 = fdl * 0x1p-28 + 0x1p-50 * fmax(fabs(emax), fabs(emin)) + 0x1p-1000;
      const double hA = cr * (emax - d64), hB = cr * (emax + d64);
      const double lC = cr * (emin - d64), lD = cr * (emin + d64);
      const double m = 0x1p-50 * (fabs(hB) + fabs(lC)) + 0x1p-1000;
      const double sLo = (hA - lD) * (1.0 / 3.0) - m, sHi = (hB - lC) * (1.0 / 3.0) + m;
      es16 = f32_to_f16_bits(f32_down(sLo));
      ez16 = f32_to_f16_bits(f32_down(lC - m));
      known = sLo >= 0.0 && es16 == f32_to_f16_bits(f32_up(sHi)) && ez16 == f32_to_f16_bits(f32_up(lD + m));
    }
    if (!known) {
      cnf = cnf0;
      emax = -INFINITY;
      emin = INFINITY;
      lanes = __ballot(cnf != 0u);
      while (lanes) {
        const int ls = __builtin_ctzll(lanes);
        const uint32_t cm = __builtin_amdgcn_readlane(cnf, ls);
        const int b = __builtin_ctz(cm);
        if (lane == ls) cnf &= cnf - 1u;
        lanes = __ballot(cnf != 0u);
        const int j = 16 * (b >> 2) + 4 * (ls >> 4) + (b & 3);
        const double y = coop_dot(xrow, rt + j * kRTRow, lane);
        emax = fmax(emax, y);
        emin = fmin(emin, y);
      }
      scale_zero(cr, emax, emin, es16, ez16);
    }
    const double esv = h2d(es16);
    const bool full = !(cr > 0.0) || (esv != 0.0 && !(fdl <= kCodeSlack * esv));
    if (full) {
      // every value of token nf exact: lane L takes dims L and L + 64
      if (lane < 8) fbw[nf * 8 + lane] = 0u;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      double ymx2 = -INFINITY, ymn2 = INFINITY;
      double yv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        const uint16_t* rr = rt + j * kRTRow;
        double s = 0.0, c = 0.0;
        for (int i = 0; i < kHeadDim; i += 8) {
          const uint4 xv = *reinterpret_cast<const uint4*>(xrow + i);
          const uint4 rv = *reinterpret_cast<const uint4*>(rr + i);
          const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
          const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            demote::two_sum_add(s, c, bf16lo(xw[k]) * bf16lo(rw[k]));
            demote::two_sum_add(s, c, bf16hi(xw[k]) * bf16hi(rw[k]));
          }
        }
        yv[h] = s + c;
        ymx2 = fmax(ymx2, yv[h]);
        ymn2 = fmin(ymn2, yv[h]);
      }
      ymx2 = wave_max(ymx2);
      ymn2 = wave_min(ymn2);
      scale_zero(cr, ymx2, ymn2, es16, ez16);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        const uint32_t q = exact_code(yv[h], es16, ez16, lv);
        // fb word (token nf, mt = j / 16) holds dim 16 mt + 4 g + e at bits 8 g + 2 e
        const int r = j & 15;
        atomicOr(&fbw[nf * 8 + (j >> 4)], q << (8 * (r >> 2) + 2 * (r & 3)));
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (n_ == nf) {
      s16 = es16;
      z16 = ez16;
      fbk = full;
    }
  }
  return static_cast<uint64_t>(s16) | (static_cast<uint64_t>(z16) << 16) | (static_cast<uint64_t>(fbk) << 32);
}

// CB: the Lloyd-Max codebook variant (codebook words [n_kv][K, V])
template <bool CB>
__global__ __launch_bounds__(256) void demote_bulk_kernel(
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

  // R^T into LDS: thread (i, half) copies row i, columns 64 half .. + 63
  {
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
  // largest squared column norm of R (threads 0..127: column tid)
  if (tid < kHeadDim) {
    float a = 0.f;
    const uint4* row = reinterpret_cast<const uint4*>(sm.rt + tid * kRTRow);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint4 v = row[q];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = __uint_as_float(w4[k] << 16);
        const float hi = __uint_as_float(w4[k] & 0xFFFF0000u);
        a = fmaf(lo, lo, fmaf(hi, hi, a));
      }
    }
    a = wave_max(a);
    if (lane == 0) sm.fb[wave][0][0] = __float_as_uint(a);
  }
  __syncthreads();
  const float colmax2 = fmaxf(__uint_as_float(sm.fb[0][0][0]), __uint_as_float(sm.fb[1][0][0]));
  __syncthreads();  // fb is reused below

  uint16_t* xs = reinterpret_cast<uint16_t*>(sm.stage[wave]);        // x rows of a tile [16][128]
  unsigned char* cs = reinterpret_cast<unsigned char*>(sm.stage[wave]);  // codes of a tile
  uint32_t* fbw = &sm.fb[wave][0][0];
  const size_t head_stride = static_cast<size_t>(n_kv) * kHeadDim;  // elements between tokens
  const int meta_off = is_v ? kVMeta : kKMeta;

  for (int it = 0; it < kIters; ++it) {
    const int tb = blockIdx.x * kRowsPerBlock + (it * kBWaves + wave) * 32;  // first token of the iteration
    if (tb >= n) break;  // wave-uniform
    // x fragments (B operand): lane (G, n) holds token tb + 16 tt + n, elements 32 ks + 8 G .. + 7
    // (tokens past the end read the last row; nothing of theirs is stored)
    uint4 bx[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = min(tb + 16 * tt + n_, n - 1);
      const uint16_t* xr = src + static_cast<size_t>(t) * head_stride + static_cast<size_t>(head) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bx[tt][ks] = *reinterpret_cast<const uint4*>(xr + 32 * ks + 8 * G);
    }
    // y^T = R^T x^T: rows dims 16 mt + 4 G + e, column token n
    f32x4 acc[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      acc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(sm.rt + (16 * mt + n_) * kRTRow + 32 * ks + 8 * G);
        const bf16x8 av = __builtin_bit_cast(bf16x8, a);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bx[0][ks]), acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bx[1][ks]), acc[mt][1], 0, 0, 0);
      }
    }

#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t0 = tb + 16 * tt;  // first token of the tile
      if (t0 >= n) break;           // wave-uniform
      const int tok = t0 + n_;
      const bool valid = tok < n;
      const int page = dst_page[valid ? tok : t0];
      const int slot = dst_slot[valid ? tok : t0];

      // per-token extremes and |x|^2 (lane-local, then over the 4 lane groups)
      float mx = -INFINITY, mn = INFINITY, nx = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx = fmaxf(mx, acc[mt][tt][e]);
          mn = fminf(mn, acc[mt][tt][e]);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t w4[4] = {bx[tt][ks].x, bx[tt][ks].y, bx[tt][ks].z, bx[tt][ks].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          nx = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w4[k]), __builtin_bit_cast(bf16x2, w4[k]), nx,
                                               false);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mn = fminf(mn, __shfl_xor(mn, 16, 64));
      mn = fminf(mn, __shfl_xor(mn, 32, 64));
      nx += __shfl_xor(nx, 16, 64);
      nx += __shfl_xor(nx, 32, 64);
      // error bound of every fp32 value of this token (the norms carry their own fp32
      // rounding, covered by the last factor)
      const float dl = static_cast<float>(kAccUlps * 0x1p-24) * sqrtf(nx * colmax2) * (1.f + 0x1p-10f);

      // scale and zero point from the interval of the extremes. The exact extremes lie in
      // [mx - dl, mx + dl] and [mn - dl, mn + dl]; the chain below evaluates the quantiser's
      // steps on those ends in fp32 and widens the results by more than every rounding of
      // either evaluation (fp32 here, fp64 in the quantiser), so they bound the true scale
      // and zero point. Rounding to fp16 is monotone: equal ends mean a determined value.
      uint16_t s16 = 0, z16 = 0;
      bool exact = true;
      {
#pragma clang fp contract(off)
        const float c32 = static_cast<float>(cr);
        if (cr > 0.0 && dl < INFINITY && mx != -INFINITY) {
          const float hA = c32 * (mx - dl), hB = c32 * (mx + dl);
          const float lC = c32 * (mn - dl), lD = c32 * (mn + dl);
          const float ms = 0x1p-21f * (fabsf(hB) + fabsf(lC)) + 0x1p-140f;
          const float mz = 0x1p-21f * fabsf(lC) + 0x1p-140f;
          const float sLo = (hA - lD) * (1.f / 3.f) - ms, sHi = (hB - lC) * (1.f / 3.f) + ms;
          s16 = f32_to_f16_bits(sLo);
          z16 = f32_to_f16_bits(lC - mz);
          exact = sLo >= 0.f && s16 == f32_to_f16_bits(sHi) && z16 == f32_to_f16_bits(lD + mz);
          const float sv = f16_to_f32(s16);
          if (exact && sv != 0.f) exact = dl <= static_cast<float>(kCodeSlack) * sv;
        } else {
          exact = false;
        }
        if (!valid) exact = true;  // nothing to do for tokens past the end
      }
      const double delta = dl;

      // tokens whose interval test failed: exact candidates, then the exact chain; tokens
      // whose codes cannot come from fp32 values: all 128 values exact
      bool fbk = false;  // this lane's token takes its codes from fb
      uint64_t todo = __ballot(!exact && G == 0);
      if (todo) {
        // candidate dims of this lane's token: fp32 values within 3 delta of an fp32 extreme
        // (fp32 rounding of the thresholds is below delta / 16, so this holds every value
        // within 2 delta exactly), one bit per (mt, e)
        uint32_t cand = 0u;
        if (!exact) {
          const float thi = mx - 3.f * dl;
          const float tlo = mn + 3.f * dl;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (acc[mt][tt][e] >= thi || acc[mt][tt][e] <= tlo) cand |= 1u << (4 * mt + e);
        }
        // the tile's x rows into LDS (bf16 [16][128])
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<uint4*>(xs + n_ * kHeadDim + 32 * ks + 8 * G) = bx[tt][ks];
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const uint64_t r = exact_tokens(xs, sm.rt, fbw, todo, cand, delta,
                                        static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16), cr, lv);
        s16 = static_cast<uint16_t>(r & 0xFFFFu);
        z16 = static_cast<uint16_t>((r >> 16) & 0xFFFFu);
        fbk = (r >> 32) & 1u;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      }

      // codes of this lane's 32 values into the stage (the x rows are no longer needed)
      const float sf = f16_to_f32(s16);
      const float zf = f16_to_f32(z16);
      const float inv_s = sf != 0.f ? 1.f / sf : 0.f;
      uint32_t cw[8];  // dims 16 mt + 4 G + e at byte e
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (CB) {
            // the nearest codebook level (a tie of the fp32 value lies inside the tolerated
            // band around the midpoint)
            w |= static_cast<uint32_t>(codebook_code((acc[mt][tt][e] - zf) * inv_s, lv)) << (8 * e);
          } else {
            // t + 1/2 clamped to [0, 3.5], truncated: the nearest level (a tie rounds up, and
            // a tie of the fp32 value lies inside the tolerated band around the boundary)
            const float t = __builtin_amdgcn_fmed3f(fmaf(acc[mt][tt][e] - zf, inv_s, 0.5f), 0.f, 3.5f);
            w |= static_cast<uint32_t>(t) << (8 * e);
          }
        }
        if (sf == 0.f) w = 0u;
        cw[mt] = w;
      }
      if (fbk) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const uint32_t f = (fbw[n_ * 8 + mt] >> (8 * G)) & 0xFFu;
          cw[mt] = (f & 3u) | (((f >> 2) & 3u) << 8) | (((f >> 4) & 3u) << 16) | ((f >> 6) << 24);
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (!is_v) {
        // K: bytes [token][dim]
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<uint32_t*>(cs + n_ * kHeadDim + 16 * mt + 4 * G) = cw[mt];
      } else {
        // V: bytes [dim][token]
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[(16 * mt + 4 * G + e) * 16 + n_] = static_cast<unsigned char>(cw[mt] >> (8 * e));
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);

      // scale and zero point of the token
      if (valid && G == 0) {
        uint8_t* blk = pool + (static_cast<size_t>(page) * n_kv + head) * kHeadBlock;
        *reinterpret_cast<uint32_t*>(blk + meta_off + 4 * slot) = static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16);
      }
      if (!is_v) {
        // K words: word q = lane + 64 r is (token q / 8 of the tile, dims 16 (q % 8) ..)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int q = lane + 64 * r;
          const int tk = q >> 3;
          const int w = q & 7;
          // page and slot of the word's token from lane tk, which loaded them (every lane
          // of the wave takes part in the shuffles)
          const int pg = __shfl(page, tk, 64);
          const int sl = __shfl(slot, tk, 64);
          if (t0 + tk < n) {
            const uint4 b = *reinterpret_cast<const uint4*>(cs + tk * kHeadDim + 16 * w);
            const uint32_t word = b.x | (b.y << 2) | (b.z << 4) | (b.w << 6);
            uint8_t* blk = pool + (static_cast<size_t>(pg) * n_kv + head) * kHeadBlock;
            *reinterpret_cast<uint32_t*>(blk + k_word_offset(sl, w)) = word;
          }
        }
      } else {
        // V: whole words when the tile fills slots 16u..16u+15 of one page in order
        const int page0 = __shfl(page, 0, 64);
        const int slot0 = __shfl(slot, 0, 64);
        const bool mine_ok = valid && page == page0 && slot == (slot0 & ~15) + n_;
        const bool aligned = (slot0 & 15) == 0 && __ballot(G == 0 && mine_ok) == 0xFFFFull;
        if (aligned) {
          uint8_t* blk = pool + (static_cast<size_t>(page0) * n_kv + head) * kHeadBlock;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int d = lane + 64 * r;
            const uint4 b = *reinterpret_cast<const uint4*>(cs + d * 16);
            const uint32_t word = b.x | (b.y << 2) | (b.z << 4) | (b.w << 6);
            *reinterpret_cast<uint32_t*>(blk + v_word_offset(d, slot0 >> 4)) = word;
          }
        } else if (valid) {
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
              atomicOr(w, ((cw[mt] >> (8 * e)) & 3u) << sh);
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
    hipLaunchKernelGGL(demote_bulk_kernel<true>, dim3(blocks, L.n_kv, 2), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), n, L.n_kv, dst_page,
                       dst_slot, static_cast<const uint16_t*>(rot_k), static_cast<const uint16_t*>(rot_v), clip_k,
                       clip_v, static_cast<uint8_t*>(pool), codebook);
  else
    hipLaunchKernelGGL(demote_bulk_kernel<false>, dim3(blocks, L.n_kv, 2), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src), n, L.n_kv, dst_page,
                       dst_slot, static_cast<const uint16_t*>(rot_k), static_cast<const uint16_t*>(rot_v), clip_k,
                       clip_v, static_cast<uint8_t*>(pool), nullptr);
  return hipGetLastError();
}

}  // namespace oscar
