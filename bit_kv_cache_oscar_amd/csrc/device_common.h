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
constexpr float kLog2e = 1.4426950408889634f;

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

// Nearest fp16 of a double (ties to even), in one rounding step from the fp64 value.
// Overflow gives +-inf, NaN gives a quiet NaN, magnitudes below half the smallest
// subnormal give +-0.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) return static_cast<uint16_t>(sign | (a > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u));
  const int e = static_cast<int>(a >> 52);
  if (e == 0) return static_cast<uint16_t>(sign);
  const uint64_t m = (a & 0xFFFFFFFFFFFFFull) | 0x10000000000000ull;  // value = m * 2^(e-1075)
  int he = e - 1008;                                                  // fp16 biased exponent
  int shift = 42;                                                     // keep 11 bits when normal
  if (he < 1) {
    shift = 43 - he;  // subnormal: units of 2^-24
    he = 0;
  }
  if (shift >= 54) return static_cast<uint16_t>(sign);
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1))) ++q;
  if (he == 0) return static_cast<uint16_t>(sign | static_cast<uint32_t>(q));  // q == 1024 is the min normal
  if (q == 2048) {
    q = 1024;
    ++he;
  }
  if (he >= 31) return static_cast<uint16_t>(sign | 0x7C00u);
  return static_cast<uint16_t>(sign | (static_cast<uint32_t>(he) << 10) | static_cast<uint32_t>(q - 1024));
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

// Value of lane `src` (wave-uniform) of v, broadcast to every lane.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// 2^x with 2^(-inf) = 0.
__device__ __forceinline__ float exp2_safe(float x) { return exp2f(x); }

}  // namespace oscar
