// INT2 history pass of decode attention on the gfx950 matrix cores.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the INT2 kernel unpacks
// the 2-bit codes, dequantises with the per-group scale and zero point and accumulates
// in floating point; its result is joined with the BF16 sink/recent pass by an
// online-softmax merge.
//
// The dequantisation is folded so that both contractions run on raw codes:
//   score_t = s_t (q_rot . c_t) + z_t sum(q_rot)
//   acc     = sum_t (p_t s_t) c_t + sum_t p_t z_t
// Both contractions are small integer GEMMs on v_mfma_i32_16x16x64_i8:
//   K side: [query heads x 4 limbs] x [128 dims] x [16 tokens]: q_rot (fp64) is held as a
//           29-bit fixed-point integer split into four signed 8-bit limbs, so q_rot . c is
//           exact and the score is folded in fp64;
//   V side: [query heads x 4 limbs] x [64 tokens] x [16 dims]: p_t s_t of the page is held
//           as a 28-bit fixed-point integer relative to the page maximum, in four unsigned
//           7-bit limbs.
// A 16-row M tile holds 4 heads x 4 limbs; GQ <= 4 uses one tile (unused rows zero).
//
// Grid (split, kv_head x head group, request), 4 waves per workgroup, at most 8 query
// heads per workgroup (16 query heads per KV head run as two groups of 8); wave w walks pages
// split_begin + w, + 4, ... of its split, loading the next page while it processes the
// current one. In a page, MFMA column n of K tile nt is slot 4n + nt, so each lane's four
// scores belong to four consecutive slots and the P limbs reach the V operand layout (16
// consecutive slots per lane group) through one LDS dword write and one 16-byte read per
// tile. Reductions over the 16 lanes of a lane group use DPP row operations. Wave
// partials are merged through LDS and one (m, l, acc) partial per (request, query head,
// split) is written.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

constexpr int kWaves = 4;
typedef char i8x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i8x16 unpack16(uint32_t w) {
  // bytes of word m hold the codes at bits 2m..2m+1 of the packed word's four bytes
  uint4 u;
  u.x = w & 0x03030303u;
  u.y = (w >> 2) & 0x03030303u;
  u.z = (w >> 4) & 0x03030303u;
  u.w = (w >> 6) & 0x03030303u;
  return __builtin_bit_cast(i8x16, u);
}

__device__ __forceinline__ i32x4 mfma16(i8x16 a, i8x16 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 2^e with e in [-1022, 1023]
__device__ __forceinline__ double pow2(int e) { return __longlong_as_double(static_cast<long long>(e + 1023) << 52); }

// Fixed-point exponent: |x| <= amax < 2^k  ->  x * 2^(29 - k) has magnitude < 2^29.
__device__ __forceinline__ int fixed_shift(double amax) {
  if (!(amax > 0.0)) return 0;
  int k;
  frexp(amax, &k);  // amax = f * 2^k, 0.5 <= f < 1
  return 29 - k;
}

// Four signed 8-bit limbs of v (|v| < 2^29), least significant first, packed in a word.
__device__ __forceinline__ uint32_t limbs4(int v) {
  const int l0 = static_cast<signed char>(v & 0xFF);
  v = (v - l0) >> 8;
  const int l1 = static_cast<signed char>(v & 0xFF);
  v = (v - l1) >> 8;
  const int l2 = static_cast<signed char>(v & 0xFF);
  const int l3 = (v - l2) >> 8;
  return (static_cast<uint32_t>(l0) & 0xFF) | ((static_cast<uint32_t>(l1) & 0xFF) << 8) |
         ((static_cast<uint32_t>(l2) & 0xFF) << 16) | ((static_cast<uint32_t>(l3) & 0xFF) << 24);
}

__device__ __forceinline__ double combine_d(const i32x4& c) {
  // sum_j 2^(8j) c_j, exact: each (hi, lo) pair fits 32 bits, the total fits fp64
  const int lo = c[0] + c[1] * 256;
  const int hi = c[2] + c[3] * 256;
  return fma(static_cast<double>(hi), 65536.0, static_cast<double>(lo));
}

// sum_j 2^(7j) c_j for the V side's 7-bit limbs (fp32 result)
__device__ __forceinline__ float combine7_f(const i32x4& c) {
  const int lo = c[0] + c[1] * 128;
  const int hi = c[2] + c[3] * 128;
  return fmaf(static_cast<float>(hi), 16384.f, static_cast<float>(lo));
}

struct PageRegs {
  uint4 k[2];  // K words: slots 4n..4n+3 (two words each: dims 32G..32G+15, 32G+16..32G+31)
  uint4 km;    // K (scale, zero) of slots 4n..4n+3
  uint4 vm;    // V (scale, zero) of slots 4n..4n+3
  uint4 v[2];  // V words of dims 16dt + n, dt = 0..7, slots 16G..16G+15

  __device__ __forceinline__ uint32_t kword(int nt, int h) const {
    const uint4& c = k[nt >> 1];
    return (nt & 1) ? (h ? c.w : c.z) : (h ? c.y : c.x);
  }
  __device__ __forceinline__ uint32_t kmeta(int nt) const { return nt == 0 ? km.x : nt == 1 ? km.y : nt == 2 ? km.z : km.w; }
  __device__ __forceinline__ uint32_t vmeta(int nt) const { return nt == 0 ? vm.x : nt == 1 ? vm.y : nt == 2 ? vm.z : vm.w; }
  __device__ __forceinline__ uint32_t vword(int dt) const {
    const uint4& c = v[dt >> 2];
    const int i = dt & 3;
    return i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w;
  }
};

// Lane l = 16 G + n reads its page data as six 16-byte loads (the page layout keeps each
// lane's K and V words contiguous).
__device__ __forceinline__ void load_page(PageRegs& r, const uint8_t* __restrict__ blk, int lane, int n) {
  const uint4* kp = reinterpret_cast<const uint4*>(blk + kKCodes + 32 * lane);
  const uint4* vp = reinterpret_cast<const uint4*>(blk + kVCodes + 32 * lane);
  r.k[0] = kp[0];
  r.k[1] = kp[1];
  r.km = *reinterpret_cast<const uint4*>(blk + kKMeta + 16 * n);
  r.vm = *reinterpret_cast<const uint4*>(blk + kVMeta + 16 * n);
  r.v[0] = vp[0];
  r.v[1] = vp[1];
}

// Per-(wave, tile) state of the online softmax. V sums stay in int32 MFMA accumulators
// (fixed point relative to the reference maximum m and scale 2^-E) until the reference or
// the scale must change; then they are flushed into float sums.
template <int MT>
struct SoftmaxState {
  float m[MT];         // reference maximum (log2 units), -inf before the first token
  float l[MT];         // sum of 2^(s - m) over this lane's tokens
  float z[MT];         // sum of 2^(s - m) * z_v over this lane's tokens
  float vcap[MT];      // largest V scale the current fixed-point exponent can hold
  float down[MT];      // 2^-E of the current fixed point
  float up[MT];        // 2^E
  float accf[MT][8];   // flushed V sums, relative to m
  i32x4 acci[MT][8];   // pending V sums, 7-bit limbs, relative to m and 2^-E
};

template <int MT>
__device__ __forceinline__ void flush_tile(SoftmaxState<MT>& st, int mt) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    st.accf[mt][dt] = fmaf(combine7_f(st.acci[mt][dt]), st.down[mt], st.accf[mt][dt]);
    st.acci[mt][dt] = i32x4{0, 0, 0, 0};
  }
}

// The rotated query of one (request, query head), once per call: q_rot = q R_K in fp64
// (bf16 products are exact), its fixed-point limbs (|q_rot| * 2^sh < 2^29, four signed
// 8-bit limbs) and two doubles: the score scale 2^-sh * sm_scale * log2(e) and the scaled
// sum(q_rot). Thread t: wave rh sums rows 64 rh .. +63 at columns 2 lane, 2 lane + 1.
__global__ __launch_bounds__(128) void qprep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ rot_k,
                                                    int n_q, int gq, double scale_log2, char* __restrict__ qlimb,
                                                    double* __restrict__ qscal) {
  __shared__ double qd_s[kHeadDim];
  __shared__ double part_s[2][kHeadDim];
  __shared__ float amax_s[2];
  __shared__ double sum_s[2];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int kv = h / gq;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int rh = __builtin_amdgcn_readfirstlane(t >> 6);
  const size_t head = static_cast<size_t>(b) * n_q + h;

  const uint32_t* rcol = reinterpret_cast<const uint32_t*>(rot_k + static_cast<size_t>(kv) * kHeadDim * kHeadDim +
                                                           static_cast<size_t>(64 * rh) * kHeadDim) + lane;
  uint32_t rr[64];
#pragma unroll
  for (int u = 0; u < 64; ++u) rr[u] = rcol[u * (kHeadDim / 2)];
  qd_s[t] = static_cast<double>(bf16_to_f32(q[head * kHeadDim + t]));
  __syncthreads();
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    const double qv = qd_s[64 * rh + u];
    a0 = fma(qv, static_cast<double>(__uint_as_float(rr[u] << 16)), a0);
    a1 = fma(qv, static_cast<double>(__uint_as_float(rr[u] & 0xFFFF0000u)), a1);
  }
  part_s[rh][2 * lane] = a0;
  part_s[rh][2 * lane + 1] = a1;
  __syncthreads();
  const double x = part_s[0][t] + part_s[1][t];  // q_rot[t]
  const float am = wave_max_f32(static_cast<float>(fabs(x)));
  const double sm = wave_sum_f64(x);
  if (lane == 0) {
    amax_s[rh] = am;
    sum_s[rh] = sm;
  }
  __syncthreads();
  // amax rounded to float can only move up to the next power of two: the shift stays safe
  const int sh = fixed_shift(static_cast<double>(fmaxf(amax_s[0], amax_s[1])));
  const uint32_t w = limbs4(static_cast<int>(rint(x * pow2(sh))));
  char* dst = qlimb + head * 512;
#pragma unroll
  for (int l = 0; l < 4; ++l) dst[l * kHeadDim + t] = static_cast<char>((w >> (8 * l)) & 0xFF);
  if (t == 0) {
    qscal[2 * head] = pow2(-sh) * scale_log2;
    qscal[2 * head + 1] = (sum_s[0] + sum_s[1]) * scale_log2;
  }
}

// GQ is the number of query heads one workgroup serves (at most 8); a KV head whose group
// is larger is served by n_groups = (query heads per KV head) / GQ workgroups along y.
template <int GQ>
__global__ __launch_bounds__(256) void decode_int2_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rot_k, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ hist_len, int n_q,
    int n_kv, int n_groups, int n_splits, const char* __restrict__ qlimb, const double* __restrict__ qscal,
    float* __restrict__ out_m, float* __restrict__ out_l, float* __restrict__ out_acc) {
  constexpr int MT = (GQ + 3) / 4;  // 16-row M tiles
  constexpr int NH = 4 * MT;        // heads including padding rows
  constexpr int kWaccBytes = kWaves * GQ * kHeadDim * 4;
  constexpr int kPBytes = kWaves * NH * 4 * kPageTokens;
  constexpr int kScratch = kWaccBytes > kPBytes ? kWaccBytes : kPBytes;

  // page loop: P limbs of each wave; epilogue: wave partials
  __shared__ __align__(16) unsigned char scratch_s[kScratch];
  __shared__ float wm_s[kWaves][GQ];
  __shared__ float wl_s[kWaves][GQ];
  float (*wacc_s)[GQ][kHeadDim] = reinterpret_cast<float (*)[GQ][kHeadDim]>(scratch_s);

  const int split = blockIdx.x;
  const int kv = blockIdx.y / n_groups;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // MFMA column / row index
  const int G = lane >> 4;  // lane group
  const int h0 = blockIdx.y * GQ;  // first query head of this workgroup

  const int nh = hist_len[b];
  const int n_pages = (nh + kPageTokens - 1) / kPageTokens;
  const int pps = (n_pages + n_splits - 1) / n_splits;
  const int p_begin = split * pps;
  const int p_end = min(n_pages, p_begin + pps);
  const int32_t* table = block_table + static_cast<size_t>(b) * max_pages;
  const uint8_t* head_base = pool + static_cast<size_t>(kv) * kHeadBlock;
  const size_t page_stride = static_cast<size_t>(n_kv) * kHeadBlock;

  // the first page's loads go out together with the rotated query's
  PageRegs buf[2];
  int p = p_begin + wave;
  if (p < p_end) load_page(buf[0], head_base + table[p] * page_stride, lane, n);

  // K-side A operands: row n of tile mt is (head 4mt + n/4, limb n%4); lane group G owns
  // dims 32G + 16ks .. +15 of K step ks. Rows of heads beyond GQ are zero.
  const size_t head0 = static_cast<size_t>(b) * n_q + h0;
  i8x16 aK[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int g = 4 * mt + (n >> 2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i8x16 zero16 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      aK[mt][ks] = g < GQ ? *reinterpret_cast<const i8x16*>(qlimb + (head0 + g) * 512 + (n & 3) * kHeadDim +
                                                            32 * G + 16 * ks)
                          : zero16;
    }
  }
  double qsc[MT], sgm[MT];
  bool head_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int g = 4 * mt + G;
    head_ok[mt] = g < GQ;
    qsc[mt] = head_ok[mt] ? qscal[2 * (head0 + g)] : 0.0;
    sgm[mt] = head_ok[mt] ? qscal[2 * (head0 + g) + 1] : 0.0;
  }

  SoftmaxState<MT> st;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st.m[mt] = -INFINITY;
    st.l[mt] = st.z[mt] = 0.f;
    st.vcap[mt] = -1.f;
    st.down[mt] = st.up[mt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      st.accf[mt][dt] = 0.f;
      st.acci[mt][dt] = i32x4{0, 0, 0, 0};
    }
  }
  char (*pl)[kPageTokens] = reinterpret_cast<char (*)[kPageTokens]>(scratch_s + wave * NH * 4 * kPageTokens);

  auto process = [&](const PageRegs& cur, int ntok) {
    // K side: exact integer q_rot . c per (head, slot); all MFMAs first
    i32x4 ck[MT][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const i8x16 b0 = unpack16(cur.kword(nt, 0));
      const i8x16 b1 = unpack16(cur.kword(nt, 1));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x4 zero = {0, 0, 0, 0};
        ck[mt][nt] = mfma16(aK[mt][1], b1, mfma16(aK[mt][0], b0, zero));
      }
    }
    // the page's largest V scale (shared by all heads)
    float sv[4], zv[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sv[nt] = f16_to_f32(cur.vmeta(nt));
      zv[nt] = f16_to_f32(cur.vmeta(nt) >> 16);
    }
    const float vmax = row16_max(__builtin_fmaxf(__builtin_fmaxf(sv[0], sv[1]), __builtin_fmaxf(sv[2], sv[3])));

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // scores in log2 units, folded in fp64
      double sc[4];
      float smax = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bool valid = head_ok[mt] && (4 * n + nt < ntok);
        const double sk = static_cast<double>(f16_to_f32(cur.kmeta(nt)));
        const double zk = static_cast<double>(f16_to_f32(cur.kmeta(nt) >> 16));
        sc[nt] = valid ? fma(sk, combine_d(ck[mt][nt]) * qsc[mt], zk * sgm[mt]) : -INFINITY;
        smax = __builtin_fmaxf(smax, static_cast<float>(sc[nt]));
      }
      smax = row16_max(smax);
      const float m_new = __builtin_fmaxf(st.m[mt], smax);
      if (m_new > st.m[mt] || vmax > st.vcap[mt]) {
        // new reference or scale: fold the pending integer sums into the float sums, rescale
        flush_tile(st, mt);
        if (m_new > st.m[mt]) {
          const float alpha = exp2f(st.m[mt] - m_new);
          st.l[mt] *= alpha;
          st.z[mt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) st.accf[mt][dt] *= alpha;
          st.m[mt] = m_new;
        }
        if (vmax > st.vcap[mt]) {
          // P = p s_v <= s_v < 2^k with one bit of headroom: P 2^(27 - k) < 2^27 fits four 7-bit limbs
          int k = 0;
          frexpf(vmax, &k);
          const int e = 27 - k;
          st.up[mt] = __int_as_float((e + 127) << 23);
          st.down[mt] = __int_as_float((127 - e) << 23);
          st.vcap[mt] = __int_as_float((k + 127) << 23);  // 2^k: room for V scales up to 2x vmax
        }
      }
      uint32_t pi[4];
      float psum = 0.f, zsum = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float pt = (m_new == -INFINITY) ? 0.f : exp2f(static_cast<float>(sc[nt] - static_cast<double>(m_new)));
        psum += pt;
        zsum = fmaf(pt, zv[nt], zsum);
        pi[nt] = static_cast<uint32_t>(rintf(pt * sv[nt] * st.up[mt]));
      }
      st.l[mt] += psum;
      st.z[mt] += zsum;
      // limb l of slots 4n..4n+3 -> one dword of row (head, limb)
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const uint32_t word = __builtin_amdgcn_ubfe(pi[0], 7 * l, 7) | (__builtin_amdgcn_ubfe(pi[1], 7 * l, 7) << 8) |
                              (__builtin_amdgcn_ubfe(pi[2], 7 * l, 7) << 16) |
                              (__builtin_amdgcn_ubfe(pi[3], 7 * l, 7) << 24);
        *reinterpret_cast<uint32_t*>(&pl[(4 * mt + G) * 4 + l][4 * n]) = word;
      }
    }
    // the wave's own LDS writes must land before its lanes read each other's
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    i8x16 aP[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      aP[mt] = *reinterpret_cast<const i8x16*>(&pl[(4 * mt + (n >> 2)) * 4 + (n & 3)][16 * G]);
    // V side: rows (head, limb) x 64 slots x 16 dims per dim tile, accumulated in int32
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const i8x16 bv = unpack16(cur.vword(dt));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) st.acci[mt][dt] = mfma16(aP[mt], bv, st.acci[mt][dt]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // two page buffers in turn: the wave's next page loads while the current one is processed
  for (; p < p_end; p += 2 * kWaves) {
    const int p1 = p + kWaves;
    if (p1 < p_end) load_page(buf[1], head_base + table[p1] * page_stride, lane, n);
    process(buf[0], min(kPageTokens, nh - p * kPageTokens));
    if (p1 >= p_end) break;
    const int p2 = p1 + kWaves;
    if (p2 < p_end) load_page(buf[0], head_base + table[p2] * page_stride, lane, n);
    process(buf[1], min(kPageTokens, nh - p1 * kPageTokens));
  }

  // ---- wave partials: lane (G, n) holds head 4mt + G, dims 16dt + n (the buffer is the
  // one the P limbs used, so every wave must be done with its pages first)
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    flush_tile(st, mt);
    const int g = 4 * mt + G;
    const float l = row16_sum(st.l[mt]);
    const float zs = row16_sum(st.z[mt]);
    if (g < GQ) {
      if (n == 0) {
        wm_s[wave][g] = st.m[mt];
        wl_s[wave][g] = l;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) wacc_s[wave][g][16 * dt + n] = st.accf[mt][dt] + zs;
    }
  }
  __syncthreads();

  for (int idx = tid; idx < GQ * kHeadDim; idx += 256) {
    const int g = idx >> 7;
    const int d = idx & 127;
    float big = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) big = __builtin_fmaxf(big, wm_s[w][g]);
    float l = 0.f, a = 0.f;
    if (big != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float s = exp2f(wm_s[w][g] - big);
        l = fmaf(s, wl_s[w][g], l);
        a = fmaf(s, wacc_s[w][g][d], a);
      }
    }
    const size_t o = (static_cast<size_t>(b) * n_q + h0 + g) * n_splits + split;
    out_acc[o * kHeadDim + d] = a;
    if (d == 0) {
      out_m[o] = big;
      out_l[o] = l;
    }
  }
}

template <int GQ>
hipError_t launch(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                  const int32_t* block_table, int max_pages, const int32_t* hist_len, int batch,
                  float sm_scale, int n_splits, const PartialsView& out, hipStream_t stream) {
  const int n_groups = L.gq / GQ;
  const double scale_log2 = static_cast<double>(sm_scale) * 1.4426950408889634;
  hipLaunchKernelGGL(qprep_kernel, dim3(L.n_q, batch), dim3(128), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(rot_k), L.n_q, L.gq, scale_log2, out.qlimb, out.qscal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_int2_kernel<GQ>, dim3(n_splits, L.n_kv * n_groups, batch), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(rot_k),
                     static_cast<const uint8_t*>(pool), block_table, max_pages, hist_len, L.n_q, L.n_kv, n_groups,
                     n_splits, out.qlimb, out.qscal, out.m, out.l, out.acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_int2(const LayerShape& L, const void* q, const void* rot_k, const void* pool,
                              const int32_t* block_table, int max_pages, const int32_t* hist_len,
                              int batch, float sm_scale, int n_splits, const PartialsView& out,
                              hipStream_t stream) {
  switch (L.gq) {
    case 1: return launch<1>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 2: return launch<2>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 4: return launch<4>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 8: return launch<8>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    case 16: return launch<8>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
