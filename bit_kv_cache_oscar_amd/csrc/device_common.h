// Device helpers shared by the liboscar_kv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kPageTokens = 64;
constexpr int kHeadBlock = 4608;  // bytes of one page for one KV head
constexpr int kKCodes = 0;
constexpr int kVCodes = 2048;
constexpr int kKMeta = 4096;
constexpr int kVMeta = 4352;
// Bytes of one page for one KV head with NG quantisation groups per vector (groups of
// 128 / NG rotated dims): the K and V codes (4096 bytes), then the K (scale, zero) pairs,
// NG per slot (slot t, group g at 4 (NG t + g)), then the V pairs the same way. NG = 1 is
// the one-group layout above.
template <int NG>
constexpr int head_block_bytes() {
  return kKMeta + 512 * NG;
}
static_assert(head_block_bytes<1>() == kHeadBlock && kVMeta - kKMeta == 256, "one-group layout");
constexpr float kLog2e = 1.4426950408889634f;

// Byte offsets inside a head's page block of the word holding K slot t, dims 16w..16w+15
// and of the word holding V dim d, slots 16u..16u+15.
__host__ __device__ constexpr int k_word_offset(int t, int w) {
  return kKCodes + 32 * (16 * (w >> 1) + (t >> 2)) + 8 * (t & 3) + 4 * (w & 1);
}
__host__ __device__ constexpr int v_word_offset(int d, int u) { return kVCodes + 32 * (16 * u + (d & 15)) + 4 * (d >> 4); }

// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit float data format, no swizzle.
// A load whose offset lies past the descriptor's byte count returns 0 and touches no memory.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// Codebook word of the Lloyd-Max variant, one per (KV head, K or V): byte c holds level c
// of the four in sixteenths of the group's scale above its zero point (increasing, within
// [0, 48]; the uniform INT2 levels are 0, 16, 32, 48). Integer centre of the level range:
// every level lies within 24 of it.
__host__ __device__ inline int codebook_mid(uint32_t lv) {
  return static_cast<int>(((lv & 0xFFu) + (lv >> 24)) >> 1);
}

// Code of t = (y - z16) / s16 under a codebook word: the nearest level, a midpoint between
// two levels going to the even index. The midpoints are multiples of 1/32, exact in fp64
// and fp32.
template <typename T>
__device__ __forceinline__ int codebook_code(T t, uint32_t lv) {
  const T th0 = static_cast<T>(static_cast<int>((lv & 0xFFu) + ((lv >> 8) & 0xFFu))) * static_cast<T>(0.03125);
  const T th1 = static_cast<T>(static_cast<int>(((lv >> 8) & 0xFFu) + ((lv >> 16) & 0xFFu))) * static_cast<T>(0.03125);
  const T th2 = static_cast<T>(static_cast<int>(((lv >> 16) & 0xFFu) + (lv >> 24))) * static_cast<T>(0.03125);
  return static_cast<int>(t > th0) + static_cast<int>(t >= th1) + static_cast<int>(t > th2);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
  return static_cast<double>(bf16_to_f32(b));
}

// fp16 bits -> float (exact for every fp16 value, subnormals included).
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xFFFFu));
  return static_cast<float>(v);
}

// Nearest fp16 of a double (ties to even), as if rounded once from the fp64 value: the
// double is first rounded to fp32 with rounding to odd (to nearest, then, when inexact,
// stepped back toward zero if it went away from it and given an odd last bit), which keeps
// 24 >= 11 + 2 significand bits, so the hardware's fp32 -> fp16 rounding to nearest even
// then yields the fp64 value's nearest fp16 (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", IEEE Trans. Computers
// 57(4), 2008). Overflow gives +-inf, magnitudes below half the smallest subnormal +-0.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  const float r = static_cast<float>(x);
  const double back = static_cast<double>(r);
  uint32_t bits = __float_as_uint(r);
  if (back != x) bits = (bits - (fabs(back) > fabs(x) ? 1u : 0u)) | 1u;
  const _Float16 h = static_cast<_Float16>(__uint_as_float(bits));
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return static_cast<double>(f16_to_f32(h));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmin(v, __shfl_xor(v, o, 64));
  return v;
}

// DPP row operations (16-lane rows): quad xor 1, quad xor 2, half-row mirror, row mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// max / sum over each 16-lane row; every lane of the row receives the result
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}

// fp32 sum over the whole wave without LDS traffic: row butterflies, then the four rows
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = row16_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// two bf16 values in one dword (low half first), the operand type of the bf16 pair dot product
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

__device__ __forceinline__ double lane_value_f64(double v, int src) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), src);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), src);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// fp64 sum over the whole wave without LDS traffic: row butterflies, then the four rows
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return (lane_value_f64(v, 0) + lane_value_f64(v, 16)) + (lane_value_f64(v, 32) + lane_value_f64(v, 48));
}

// Value of lane `src` (wave-uniform) of v, broadcast to every lane.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// fp64 max / min over the whole wave (row butterflies, then the four rows)
template <int SEL>  // 0: max, 1: min
__device__ __forceinline__ double wave_ext_f64(double v) {
  auto op = [](double a, double b) { return SEL == 0 ? fmax(a, b) : fmin(a, b); };
  v = op(v, dpp_f64<kDppQuadXor1>(v));
  v = op(v, dpp_f64<kDppQuadXor2>(v));
  v = op(v, dpp_f64<kDppHalfMirror>(v));
  v = op(v, dpp_f64<kDppMirror>(v));
  return op(op(lane_value_f64(v, 0), lane_value_f64(v, 16)), op(lane_value_f64(v, 32), lane_value_f64(v, 48)));
}
__device__ __forceinline__ double wave_max_f64(double v) { return wave_ext_f64<0>(v); }
__device__ __forceinline__ double wave_min_f64(double v) { return wave_ext_f64<1>(v); }

__device__ __forceinline__ float wave_max_f32(float v) {
  v = row16_max(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

}  // namespace oscar
