// Latent gather from the paged pool fused with RMSNorm and RoPE
// ("mla_prefill_decode_graph_bf16" page: Parameters "kv_input_fn" (a cache
// row is 512 latent + 64 rope values); Args "kv_norm_gamma", "epsilon",
// "freqs_cis", "buffer_row_offsets", "cache_offsets").
//
// One 64-lane wave per buffer row, four rows per workgroup. Every lane issues
// one 16-byte load of the latent (8 bf16, or 8 e4m3 in 8 bytes), lanes 0-7
// also load the rope part and the matching 16 bytes of freqs_cis, so a row is
// read with fully coalesced vector loads. The sum of squares is reduced across
// the wave, then every lane writes its 8 normalised values with one store.
#include "kernels.hpp"

namespace mla {

constexpr int kGatherRowsPerBlock = 4;


// Largest b in [0, B) with bro[b] <= row (sequences with no rows in the chunk
// share their offset with the next one and are skipped over).
__device__ __forceinline__ int find_seq(const uint32_t* __restrict__ bro, int B, uint32_t row) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bro[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// 8 rope values of a buffer row, lanes 0-7: e4m3 (saturating) or bf16
template <bool kFp8Rope>
__device__ __forceinline__ void store_rope(void* krope, int row, int lane, const float* r) {
  if (kFp8Rope) {
    u32x2 w;
    w[0] = f32_to_e4m3_sat(r[0]) | (f32_to_e4m3_sat(r[1]) << 8) |
           (f32_to_e4m3_sat(r[2]) << 16) | (f32_to_e4m3_sat(r[3]) << 24);
    w[1] = f32_to_e4m3_sat(r[4]) | (f32_to_e4m3_sat(r[5]) << 8) |
           (f32_to_e4m3_sat(r[6]) << 16) | (f32_to_e4m3_sat(r[7]) << 24);
    *(u32x2*)((uint8_t*)krope + (size_t)row * kRope + lane * 8) = w;
  } else {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(r[2 * i], r[2 * i + 1]);
    *(u32x4*)((uint16_t*)krope + (size_t)row * kRope + lane * 8) = w;
  }
}

// kProcessed: the pool holds rows already normalised and rotated (as the KV
// write path stores them); they are copied into the buffers unchanged.
template <bool kFp8Cache, bool kFp8Rope, bool kProcessed>
__global__ void __launch_bounds__(64 * kGatherRowsPerBlock)
gather_norm_rope_kernel(GatherArgs a) {
  const int nrows = *a.bl_c;
  const int row = blockIdx.x * kGatherRowsPerBlock + (threadIdx.x >> 6);
  if (nrows <= 0 || row >= nrows || row >= a.max_rows) return;
  const int lane = lane_id();
  const int b = find_seq(a.bro_c, a.B, (uint32_t)row);
  const uint32_t p = a.co_c[b] + ((uint32_t)row - a.bro_c[b]);
  const uint32_t lp = p / (uint32_t)a.ps;
  int page = -1;
  if (lp < (uint32_t)a.maxp) page = a.page_table[(size_t)b * a.maxp + lp];
  const bool ok = page >= 0 && page < a.num_pages && (kProcessed || p < (uint32_t)a.max_seq_len);
  const size_t slot = ok ? (size_t)page * a.ps + (p % (uint32_t)a.ps) : 0;

  float x[8];
  float y[8];
  if (kFp8Cache) {
    const uint8_t* rowp = (const uint8_t*)a.cache + slot * kCache;
    u32x2 v = ok ? *(const u32x2*)(rowp + lane * 8) : u32x2{0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = e4m3_to_f32((v[0] >> (8 * i)) & 0xFF);
      x[4 + i] = e4m3_to_f32((v[1] >> (8 * i)) & 0xFF);
    }
    if (lane < 8) {
      u32x2 r = ok ? *(const u32x2*)(rowp + kLora + lane * 8) : u32x2{0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = e4m3_to_f32((r[0] >> (8 * i)) & 0xFF);
        y[4 + i] = e4m3_to_f32((r[1] >> (8 * i)) & 0xFF);
      }
    }
  } else {
    const uint16_t* rowp = (const uint16_t*)a.cache + slot * kCache;
    u32x4 v = ok ? *(const u32x4*)(rowp + lane * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(v[i]);
      x[2 * i + 1] = bf16_hi(v[i]);
    }
    if (lane < 8) {
      u32x4 r = ok ? *(const u32x4*)(rowp + kLora + lane * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = bf16_lo(r[i]);
        y[2 * i + 1] = bf16_hi(r[i]);
      }
    }
  }

  if (kProcessed) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *(u32x4*)(a.latn + (size_t)row * kLora + lane * 8) = o;
    if (lane < 8) store_rope<kFp8Rope>(a.krope, row, lane, y);
    return;
  }

  // RMSNorm of the latent
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss * (1.0f / kLora) + a.eps);
  const u32x4 g = *(const u32x4*)(a.gamma + lane * 8);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = x[2 * i] * inv * bf16_lo(g[i]);
    const float hi = x[2 * i + 1] * inv * bf16_hi(g[i]);
    o[i] = pack_bf16x2(lo, hi);
  }
  *(u32x4*)(a.latn + (size_t)row * kLora + lane * 8) = o;

  // RoPE of the rope part: adjacent pairs rotated by (cos, sin) from freqs_cis
  if (lane < 8) {
    const u32x4 f = ok ? *(const u32x4*)(a.freqs + (size_t)p * kRope + lane * 8)
                       : u32x4{0, 0, 0, 0};
    float r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float c = bf16_lo(f[i]);
      const float s = bf16_hi(f[i]);
      r[2 * i] = y[2 * i] * c - y[2 * i + 1] * s;
      r[2 * i + 1] = y[2 * i] * s + y[2 * i + 1] * c;
    }
    store_rope<kFp8Rope>(a.krope, row, lane, r);
  }
}

// KV write path ("mla_prefill_decode_graph_bf16" page: Parameters
// "kv_input_fn", the new tokens' raw latent rows [tot_seq_len, 576]; Args
// "kv_norm_gamma", "epsilon", "freqs_cis", "input_row_offsets" and the paged
// KV cache). Token t of sequence b (input_row_offsets[b] <= t <
// input_row_offsets[b+1]) sits at position p = cache_lengths[b] + t -
// input_row_offsets[b]; its row is normalised and rotated exactly as the
// gather above does for a cache row, then stored in the pool slot of p. One
// wave per token, the same 16-byte loads and stores; tokens whose page or
// position is out of range are skipped.
template <bool kFp8Cache>
__global__ void __launch_bounds__(64 * kGatherRowsPerBlock) kv_write_kernel(KvWriteArgs a) {
  const int t = blockIdx.x * kGatherRowsPerBlock + (threadIdx.x >> 6);
  if (t >= a.total || (uint32_t)t >= a.offs[a.B]) return;
  const int lane = lane_id();
  const int b = find_seq(a.offs, a.B, (uint32_t)t);
  const uint32_t p = a.clen[b] + ((uint32_t)t - a.offs[b]);
  const uint32_t lp = p / (uint32_t)a.ps;
  const int page = lp < (uint32_t)a.maxp ? a.page_table[(size_t)b * a.maxp + lp] : -1;
  if (page < 0 || page >= a.num_pages || p >= (uint32_t)a.max_seq_len) return;  // wave-uniform
  const size_t slot = (size_t)page * a.ps + (p % (uint32_t)a.ps);

  const uint16_t* in = a.input + (size_t)t * kCache;
  const u32x4 v = *(const u32x4*)(in + lane * 8);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(v[i]);
    x[2 * i + 1] = bf16_hi(v[i]);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss * (1.0f / kLora) + a.eps);
  const u32x4 g = *(const u32x4*)(a.gamma + lane * 8);
  float o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = x[2 * i] * inv * bf16_lo(g[i]);
    o[2 * i + 1] = x[2 * i + 1] * inv * bf16_hi(g[i]);
  }
  float r[8];
  if (lane < 8) {
    const u32x4 y = *(const u32x4*)(in + kLora + lane * 8);
    const u32x4 f = *(const u32x4*)(a.freqs + (size_t)p * kRope + lane * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y0 = bf16_lo(y[i]), y1 = bf16_hi(y[i]);
      const float c = bf16_lo(f[i]), s = bf16_hi(f[i]);
      r[2 * i] = y0 * c - y1 * s;
      r[2 * i + 1] = y0 * s + y1 * c;
    }
  }
  auto e4m3x8 = [](const float (&z)[8]) {
    u32x2 w;
    w[0] = f32_to_e4m3_sat(z[0]) | (f32_to_e4m3_sat(z[1]) << 8) | (f32_to_e4m3_sat(z[2]) << 16) |
           (f32_to_e4m3_sat(z[3]) << 24);
    w[1] = f32_to_e4m3_sat(z[4]) | (f32_to_e4m3_sat(z[5]) << 8) | (f32_to_e4m3_sat(z[6]) << 16) |
           (f32_to_e4m3_sat(z[7]) << 24);
    return w;
  };
  auto bf16x8_of = [](const float (&z)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(z[2 * i], z[2 * i + 1]);
    return w;
  };
  if (kFp8Cache) {
    uint8_t* rowp = (uint8_t*)a.cache + slot * kCache;
    *(u32x2*)(rowp + lane * 8) = e4m3x8(o);
    if (lane < 8) *(u32x2*)(rowp + kLora + lane * 8) = e4m3x8(r);
  } else {
    uint16_t* rowp = (uint16_t*)a.cache + slot * kCache;
    *(u32x4*)(rowp + lane * 8) = bf16x8_of(o);
    if (lane < 8) *(u32x4*)(rowp + kLora + lane * 8) = bf16x8_of(r);
  }
}

hipError_t launch_kv_write(const KvWriteArgs& a, bool fp8_cache, hipStream_t stream) {
  const dim3 grid((a.total + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock);
  const dim3 block(64 * kGatherRowsPerBlock);
  if (fp8_cache) hipLaunchKernelGGL(kv_write_kernel<true>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(kv_write_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

template <bool kProcessed>
void launch_gather_t(const GatherArgs& a, bool fp8_cache, bool fp8_rope, dim3 grid, dim3 block,
                     hipStream_t stream) {
  if (fp8_cache) {
    if (fp8_rope) hipLaunchKernelGGL((gather_norm_rope_kernel<true, true, kProcessed>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gather_norm_rope_kernel<true, false, kProcessed>), grid, block, 0, stream, a);
  } else {
    if (fp8_rope) hipLaunchKernelGGL((gather_norm_rope_kernel<false, true, kProcessed>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gather_norm_rope_kernel<false, false, kProcessed>), grid, block, 0, stream, a);
  }
}

hipError_t launch_gather(const GatherArgs& a, bool fp8_cache, bool fp8_rope, bool processed,
                         hipStream_t stream) {
  const dim3 grid((a.max_rows + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock);
  const dim3 block(64 * kGatherRowsPerBlock);
  if (processed) launch_gather_t<true>(a, fp8_cache, fp8_rope, grid, block, stream);
  else launch_gather_t<false>(a, fp8_cache, fp8_rope, grid, block, stream);
  return hipGetLastError();
}

}  // namespace mla
