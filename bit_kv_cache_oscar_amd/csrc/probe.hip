// Read-bandwidth probe (oscar_read_probe): the measured streaming ceiling that the decode
// kernels' achieved HBM bandwidth is compared with. Not part of the method.
//
// 2048 workgroups of 256 threads sweep the buffer in 16-byte loads, eight independent loads
// in flight per thread and a grid-wide stride; each workgroup writes the XOR of what it read
// (so no load can be dropped) to out[workgroup].

#include "launch.h"

namespace oscar {
namespace {

constexpr int kProbeBlocks = 2048;
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                                   uint32_t* __restrict__ out) {
  __shared__ uint32_t part[kProbeThreads / 64];
  const size_t stride = static_cast<size_t>(kProbeBlocks) * kProbeThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  u32x4 acc[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc[u] ^= v[u];
  }
  for (; i < n16; i += stride) acc[0] ^= buf[i];
  uint32_t x = 0u;
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) x ^= acc[u].x ^ acc[u].y ^ acc[u].z ^ acc[u].w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

int read_probe_blocks() { return kProbeBlocks; }

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace oscar
