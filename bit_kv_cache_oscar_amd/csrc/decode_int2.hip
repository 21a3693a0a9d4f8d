// INT2 history pass of decode attention.
//
// Method: OSCAR; QbitAI article on OSCAR, serving-path section: the INT2 kernel unpacks
// the 2-bit codes, dequantises with the per-group scale and zero point and accumulates
// in floating point; its result is joined with the BF16 sink/recent pass by an
// online-softmax merge.
//
// Grid (split, kv_head, request); 4 waves per workgroup, each wave walking every 4th
// page of the split. Within a page the 64 lanes own the 64 tokens for the scores and
// the 128 dims (two per lane) for the value sum. The dequantisation is folded:
//   q_rot . (c s + z) = s (q_rot . c) + z sum(q_rot)
//   sum_t p_t (c_t s_t + z_t) = sum_t (p_t s_t) c_t + sum_t p_t z_t
// so the inner loops multiply raw codes. Wave partials are merged through LDS and one
// (m, l, acc) partial per (request, query head, split) is written.

#include "device_common.h"
#include "launch.h"

namespace oscar {
namespace {

constexpr int kWaves = 4;

template <int GQ>
__global__ __launch_bounds__(256) void decode_int2_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rot_k, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ hist_len, int n_q,
    int n_kv, int n_splits, float scale_log2, float* __restrict__ out_m, float* __restrict__ out_l,
    float* __restrict__ out_acc) {
  __shared__ float q_s[GQ][kHeadDim];
  __shared__ float qr_s[GQ][kHeadDim];
  __shared__ float sig_s[GQ];
  __shared__ float wm_s[kWaves][GQ];
  __shared__ float wl_s[kWaves][GQ];
  __shared__ float wacc_s[kWaves][GQ][kHeadDim];

  const int split = blockIdx.x;
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h0 = kv * GQ;

  for (int i = tid; i < GQ * kHeadDim; i += 256)
    q_s[i >> 7][i & 127] = bf16_to_f32(q[(static_cast<size_t>(b) * n_q + h0) * kHeadDim + i]);
  __syncthreads();

  // q_rot[g][j] = sum_i q[g][i] R_K[i][j]; thread (half, j) takes heads half, half+2, ...
  {
    constexpr int kPer = (GQ + 1) / 2;
    const int j = tid & 127;
    const int half = tid >> 7;
    const uint16_t* rot = rot_k + static_cast<size_t>(kv) * kHeadDim * kHeadDim;
    float a[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) a[k] = 0.f;
    for (int i = 0; i < kHeadDim; ++i) {
      const float r = bf16_to_f32(rot[i * kHeadDim + j]);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int g = half + 2 * k;
        if (g < GQ) a[k] = fmaf(q_s[g][i], r, a[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int g = half + 2 * k;
      if (g < GQ) qr_s[g][j] = a[k];
    }
  }
  __syncthreads();
  for (int g = wave; g < GQ; g += kWaves) {
    const float v = wave_sum(qr_s[g][lane] + qr_s[g][lane + 64]);
    if (lane == 0) sig_s[g] = v;
  }
  __syncthreads();

  const int nh = hist_len[b];
  const int n_pages = (nh + kPageTokens - 1) / kPageTokens;
  const int pps = (n_pages + n_splits - 1) / n_splits;
  const int p_begin = split * pps;
  const int p_end = min(n_pages, p_begin + pps);

  float m_run[GQ], l_lane[GQ], z_lane[GQ], acc0[GQ], acc1[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = z_lane[g] = acc0[g] = acc1[g] = 0.f;
  }

  for (int p = p_begin + wave; p < p_end; p += kWaves) {
    const int phys = block_table[static_cast<size_t>(b) * max_pages + p];
    const uint8_t* blk = pool + (static_cast<size_t>(phys) * n_kv + kv) * kHeadBlock;
    const int ntok = min(kPageTokens, nh - p * kPageTokens);
    const bool valid = lane < ntok;

    const uint4 k0 = *reinterpret_cast<const uint4*>(blk + kKCodes + 32 * lane);
    const uint4 k1 = *reinterpret_cast<const uint4*>(blk + kKCodes + 32 * lane + 16);
    const uint32_t km = *reinterpret_cast<const uint32_t*>(blk + kKMeta + 4 * lane);
    const uint32_t vm = *reinterpret_cast<const uint32_t*>(blk + kVMeta + 4 * lane);
    const uint4 v0 = *reinterpret_cast<const uint4*>(blk + kVCodes + 16 * lane);
    const uint4 v1 = *reinterpret_cast<const uint4*>(blk + kVCodes + 16 * (lane + 64));

    // scores: lane = token. The half loop stays rolled so the q_rot reads from LDS are
    // re-issued per page instead of being hoisted into registers.
    float dot[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) dot[g] = 0.f;
#pragma unroll 1
    for (int hh = 0; hh < 2; ++hh) {
      const uint4 kk = hh ? k1 : k0;
      const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t bytes = (kw[w] >> (2 * m)) & 0x03030303u;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float c = static_cast<float>((bytes >> (8 * jj)) & 0xFFu);
            const int d = 64 * hh + 16 * w + 4 * m + jj;
#pragma unroll
            for (int g = 0; g < GQ; ++g) dot[g] = fmaf(c, qr_s[g][d], dot[g]);
          }
        }
      }
    }
    const float sk = f16_to_f32(km);
    const float zk = f16_to_f32(km >> 16);
    const float sv = f16_to_f32(vm);
    const float zv = f16_to_f32(vm >> 16);

    float pw[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float sc = valid ? fmaf(sk, dot[g], zk * sig_s[g]) * scale_log2 : -INFINITY;
      const float mn = fmaxf(m_run[g], wave_max(sc));
      const float alpha = exp2f(m_run[g] - mn);
      const float pt = valid ? exp2f(sc - mn) : 0.f;
      l_lane[g] = fmaf(l_lane[g], alpha, pt);
      z_lane[g] = fmaf(z_lane[g], alpha, valid ? pt * zv : 0.f);
      acc0[g] *= alpha;
      acc1[g] *= alpha;
      m_run[g] = mn;
      pw[g] = valid ? pt * sv : 0.f;
    }

    // value sum: lane = dims lane and lane + 64
    const uint32_t vw0[4] = {v0.x, v0.y, v0.z, v0.w};
    const uint32_t vw1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t b0 = (vw0[u] >> (2 * m)) & 0x03030303u;
        const uint32_t b1 = (vw1[u] >> (2 * m)) & 0x03030303u;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = 16 * u + 4 * m + jj;
          const float c0 = static_cast<float>((b0 >> (8 * jj)) & 0xFFu);
          const float c1 = static_cast<float>((b1 >> (8 * jj)) & 0xFFu);
#pragma unroll
          for (int g = 0; g < GQ; ++g) {
            const float pt = lane_value(pw[g], t);
            acc0[g] = fmaf(c0, pt, acc0[g]);
            acc1[g] = fmaf(c1, pt, acc1[g]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const float l = wave_sum(l_lane[g]);
    const float zs = wave_sum(z_lane[g]);
    if (lane == 0) {
      wm_s[wave][g] = m_run[g];
      wl_s[wave][g] = l;
    }
    wacc_s[wave][g][lane] = acc0[g] + zs;
    wacc_s[wave][g][lane + 64] = acc1[g] + zs;
  }
  __syncthreads();

  for (int idx = tid; idx < GQ * kHeadDim; idx += 256) {
    const int g = idx >> 7;
    const int d = idx & 127;
    float big = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) big = fmaxf(big, wm_s[w][g]);
    float l = 0.f, a = 0.f;
    if (big != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = exp2f(wm_s[w][g] - big);
        l = fmaf(sc, wl_s[w][g], l);
        a = fmaf(sc, wacc_s[w][g][d], a);
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
  hipLaunchKernelGGL(decode_int2_kernel<GQ>, dim3(n_splits, L.n_kv, batch), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(rot_k),
                     static_cast<const uint8_t*>(pool), block_table, max_pages, hist_len, L.n_q, L.n_kv,
                     n_splits, sm_scale * kLog2e, out.m, out.l, out.acc);
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
    case 16: return launch<16>(L, q, rot_k, pool, block_table, max_pages, hist_len, batch, sm_scale, n_splits, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
