// Chunk planner ("mla_prefill_plan" page, description and Args).
//
// One workgroup per chunk row. Each thread owns one sequence of the current
// 256-sequence slab; the per-chunk row lengths are prefix-summed with a
// wavefront scan (shuffle-up within each 64-lane wave, then a scan of the four
// wave totals through LDS) and the slab total is carried to the next slab.
// All arithmetic is integer, so the result is exact.
#include "kernels.hpp"

namespace mla {

constexpr int kPlanThreads = 256;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(uint32_t* __restrict__ bro, uint32_t* __restrict__ co, int32_t* __restrict__ bl,
            uint32_t* __restrict__ chunks_needed, const uint32_t* __restrict__ offs,
            const uint32_t* __restrict__ clen, int B, uint32_t T) {
  __shared__ uint32_t wave_tot[kPlanThreads / 64];
  __shared__ uint32_t red_max[kPlanThreads / 64];
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const uint64_t start_pos = (uint64_t)c * T;
  uint32_t carry = 0;
  uint64_t lmax = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + tid;
    uint32_t n = 0;
    uint64_t L = 0;
    if (b < B) {
      L = (uint64_t)(offs[b + 1] - offs[b]) + clen[b];
      const uint64_t s = start_pos < L ? start_pos : L;
      const uint64_t rem = L - s;
      n = (uint32_t)(rem < T ? rem : T);
      co[(size_t)c * B + b] = (uint32_t)s;
    }
    lmax = L > lmax ? L : lmax;
    const uint32_t incl = wave_incl_scan(n);
    if ((tid & 63) == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (b < B) bro[(size_t)c * (B + 1) + b] = before + incl - n;
    uint32_t slab = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) slab += wave_tot[w];
    carry += slab;
    __syncthreads();
  }
  if (tid == 0) {
    bro[(size_t)c * (B + 1) + B] = carry;
    bl[c] = carry > 0 ? (int32_t)carry : -1;
  }
  if (c == 0 && chunks_needed != nullptr) {
    // max over the batch of L_b, then ceil(max / T)
    uint64_t m = lmax;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t x = __shfl_xor(m, o, 64);
      m = x > m ? x : m;
    }
    if ((tid & 63) == 0) red_max[wave] = (uint32_t)m;
    __syncthreads();
    if (tid == 0) {
      uint32_t mm = 0;
      for (int w = 0; w < kPlanThreads / 64; ++w) mm = red_max[w] > mm ? red_max[w] : mm;
      chunks_needed[0] = (uint32_t)(((uint64_t)mm + T - 1) / T);
    }
  }
}

hipError_t launch_plan(uint32_t* bro, uint32_t* co, int32_t* bl, uint32_t* chunks_needed,
                       const uint32_t* offs, const uint32_t* clen, int B, int C, uint32_t T,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(C), dim3(kPlanThreads), 0, stream, bro, co, bl,
                     chunks_needed, offs, clen, B, T);
  return hipGetLastError();
}

}  // namespace mla
