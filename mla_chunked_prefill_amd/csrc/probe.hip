// Measurement helper: a plain streaming read of a device buffer, the
// practical HBM read ceiling that the decode and gather rates are set
// against. Not part of the attention path.
#include "kernels.hpp"

namespace mla {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane

// Workgroup w reads the 16-byte words w * kProbeThreads + t, stepping by the
// whole grid, eight loads in flight per lane, and folds them with XOR; one
// word per workgroup is stored so that no load can be dropped.
__global__ void __launch_bounds__(kProbeThreads) hbm_read_kernel(const u32x4* __restrict__ src,
                                                                 size_t n16,
                                                                 uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t s[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* out, int groups,
                           hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(groups), dim3(kProbeThreads), 0, stream,
                     (const u32x4*)src, bytes / 16, out);
  return hipGetLastError();
}

}  // namespace mla
