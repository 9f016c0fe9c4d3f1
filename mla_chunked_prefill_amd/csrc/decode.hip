// Absorbed MLA decode ("mla_prefill_decode_graph_bf16" page: decode branch,
// Args "w_uk" [H, 512, 128] and "w_uv" [H, 128, 512], num_partitions;
// "flare_mla_prefill_dispatch" page: kv_num_heads 1, cache_depth 576).
//
// Four kernels:
//  1. absorb:   q_abs[b, h] = [w_uk[h] q_nope[b, h] | q_rope[b, h]] (576 wide),
//               bf16 MFMA, one wave per 32x32 output tile, operands read
//               straight from global memory (both are contiguous along the
//               128-long reduction).
//  2. split-KV: one workgroup per (sequence, partition) streams the
//               partition's 576-wide cache rows once for all heads. Each of the
//               four waves keeps the absorbed queries of 32 heads in registers
//               and computes S^T = Z Q^T (keys x heads) on mfma 32x32x16, so
//               softmax statistics are per-lane. The tile is staged in LDS
//               twice: row-major for the score product and transposed
//               (512 x keys, built with an in-register 8x8 transpose) for the
//               value product O^T += Z^T P^T, whose B operand is the
//               bf16-converted score registers (K rows fed in the same
//               bit-2/3-swapped order as the prefill kernel).
//  3. combine:  log-sum-exp merge of the partitions' (max, sum, O) states.
//  4. project:  out[b, h] = w_uv[h] o_lat[b, h], bf16 MFMA like the absorb.
#include "kernels.hpp"

namespace mla {

typedef long fp8x8_d;

// ---------------------------------------------------------------------------
// 1/4. per-head small GEMMs: C[b, n] = sum_k X[b, k] W[n, k]
// ---------------------------------------------------------------------------
// X rows: x + b*x_stride (K contiguous, bf16); W rows: w + n*K (K contiguous).
// Output: y[b*y_stride + n] as bf16 (or e4m3 when kFp8Out). One wave computes a
// 32 (b) x 32 (n) tile; K is a multiple of 16.
template <int K, bool kFp8Out>
__global__ void __launch_bounds__(256) head_gemm_kernel(
    void* __restrict__ y, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    int B, int N, long x_stride_b, long x_stride_h, long w_stride_h, long y_stride_b,
    long y_stride_h, int n_tiles_n) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int h = blockIdx.y;
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles_b = (B + 31) / 32;
  if (tile >= n_tiles_b * n_tiles_n) return;
  const int tb = tile / n_tiles_n;
  const int tn = tile - tb * n_tiles_n;
  const int brow = tb * 32 + l32;
  const int nrow = tn * 32 + l32;
  const uint16_t* xp = x + (long)h * x_stride_h + (long)min(brow, B - 1) * x_stride_b + hf * 8;
  const uint16_t* wp = w + (long)h * w_stride_h + (long)nrow * K + hf * 8;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 16) {
    u32x4 xa = *(const u32x4*)(xp + k0);
    if (brow >= B) xa = u32x4{0, 0, 0, 0};
    const u32x4 wb = *(const u32x4*)(wp + k0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa),
                                                  __builtin_bit_cast(bf16x8, wb), acc, 0, 0, 0);
  }
  // lane holds column n = nrow, rows b = tb*32 + 8*(i/4) + 4*hf + i%4
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int bb = tb * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
    if (bb < B) {
      const long o = (long)bb * y_stride_b + (long)h * y_stride_h + nrow;
      if (kFp8Out) ((uint8_t*)y)[o] = (uint8_t)f32_to_e4m3_sat(acc[i]);
      else ((uint16_t*)y)[o] = (uint16_t)f32_to_bf16_rne(acc[i]);
    }
  }
}

// copy q_rope into the last 64 columns of q_abs (bf16, or e4m3 for an fp8 cache)
template <bool kFp8Out>
__global__ void copy_rope_kernel(void* __restrict__ q_abs, const uint16_t* __restrict__ q,
                                 int B, int H) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // over B*H*64
  if (i >= (long)B * H * kRope) return;
  const long bh = i / kRope;
  const int e = (int)(i - bh * kRope);
  const uint16_t v = q[bh * kQDepth + kNope + e];
  if (kFp8Out) ((uint8_t*)q_abs)[bh * kCache + kLora + e] = (uint8_t)f32_to_e4m3_sat(bf16_to_f32(v));
  else ((uint16_t*)q_abs)[bh * kCache + kLora + e] = v;
}

// ---------------------------------------------------------------------------
// 2. split-KV attention over the latent cache (bf16 cache)
// ---------------------------------------------------------------------------
constexpr int kDecBN = 32;                 // keys per tile
constexpr int kZRow = kCache + 8;          // LDS row of Z (bf16 elements, 1168 B)
constexpr int kZtRow = kDecBN + 8;         // LDS row of Z^T (bf16 elements, 80 B)


__device__ __forceinline__ uint32_t sel_lo16(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t sel_hi16(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

__global__ void __launch_bounds__(256, 1) decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sZ[kDecBN * kZRow];
  __shared__ __attribute__((aligned(16))) uint16_t sZt[kLora * kZtRow];

  const int b = blockIdx.x / a.P;
  const int part = blockIdx.x - b * a.P;
  const int ctx = (int)a.ctx[b];
  const int k_begin = part * a.keys_per_part;
  if (k_begin >= ctx) return;
  const int k_end = min(ctx, k_begin + a.keys_per_part);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int head = wave * 32 + l32;  // this lane's query column
  const bool hvalid = head < a.H;

  bf16x8 qf[36];
  {
    const uint16_t* qp = a.q_abs + ((long)b * a.H + min(head, a.H - 1)) * kCache + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      u32x4 v = hvalid ? *(const u32x4*)(qp + ks * 16) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 o[16];
#pragma unroll
  for (int md = 0; md < 16; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[md][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int kappa = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const uint16_t* cache = (const uint16_t*)a.cache;

  // loader roles: latent: dim chunk dc (0..63) x key group kg (0..3) of 8 keys
  const int dc = tid & 63;
  const int kg = tid >> 6;
  for (int kt = k_begin; kt < k_end; kt += kDecBN) {
    __syncthreads();
    {
      u32x4 r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = kt + kg * 8 + j;
        bool ok = p < k_end;
        long slot = 0;
        if (ok) {
          const int lp = p / a.ps;
          const int pg = lp < a.maxp ? a.page_table[(long)b * a.maxp + lp] : -1;
          ok = pg >= 0 && pg < a.num_pages;
          slot = (long)pg * a.ps + (p - lp * a.ps);
        }
        r[j] = ok ? *(const u32x4*)(cache + slot * kCache + dc * 8) : u32x4{0, 0, 0, 0};
        *(u32x4*)(sZ + (kg * 8 + j) * kZRow + dc * 8) = r[j];
      }
      // 8x8 transpose: Z^T[8*dc + d][8*kg + j]
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        u32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t a0 = r[2 * i][d >> 1];
          const uint32_t a1 = r[2 * i + 1][d >> 1];
          t[i] = (d & 1) ? sel_hi16(a0, a1) : sel_lo16(a0, a1);
        }
        *(u32x4*)(sZt + (dc * 8 + d) * kZtRow + kg * 8) = t;
      }
      // rope columns: 32 keys x 8 chunks
      {
        const int kk = tid >> 3, ch = tid & 7;
        const int p = kt + kk;
        bool ok = p < k_end;
        long slot = 0;
        if (ok) {
          const int lp = p / a.ps;
          const int pg = lp < a.maxp ? a.page_table[(long)b * a.maxp + lp] : -1;
          ok = pg >= 0 && pg < a.num_pages;
          slot = (long)pg * a.ps + (p - lp * a.ps);
        }
        const u32x4 v = ok ? *(const u32x4*)(cache + slot * kCache + kLora + ch * 8)
                           : u32x4{0, 0, 0, 0};
        *(u32x4*)(sZ + kk * kZRow + kLora + ch * 8) = v;
      }
    }
    __syncthreads();

    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const bf16x8 za = *(const bf16x8*)(sZ + kappa * kZRow + ks * 16 + hf * 8);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za, qf[ks], s, 0, 0, 0);
    }
    // register i holds key kt + 16*(i/8) + 8*hf + i%8
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = s[i] * a.scale_log2;
      const int kk = kt + (i >> 3) * 16 + hf * 8 + (i & 7);
      if (kk >= k_end) v = -INFINITY;
      s[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[i] - m_new);
      s[i] = p;
      psum += p;
    }
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(s[ks * 8 + 2 * j], s[ks * 8 + 2 * j + 1]);
      pb[ks] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int md = 0; md < 16; ++md) {
#pragma unroll
      for (int i = 0; i < 16; ++i) o[md][i] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 za = *(const bf16x8*)(sZt + (md * 32 + l32) * kZtRow + ks * 16 + hf * 8);
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za, pb[ks], o[md], 0, 0, 0);
      }
    }
  }
  if (!hvalid) return;
  // O^T register i of block md: dim 32*md + 8*(i/4) + 4*hf + i%4
  const long base = (((long)b * a.P + part) * a.H + head);
  float* op = a.part_o + base * kLora;
#pragma unroll
  for (int md = 0; md < 16; ++md)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = o[md][g * 4 + j];
      *(f32x4*)(op + md * 32 + g * 8 + hf * 4) = v;
    }
  if (hf == 0) {
    a.part_ml[base * 2 + 0] = m_run;
    a.part_ml[base * 2 + 1] = l_run;
  }
}

// ---------------------------------------------------------------------------
// 3. combine partitions: o_lat[b, h, :] (bf16)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_combine_kernel(
    uint16_t* __restrict__ o_lat, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const uint32_t* __restrict__ ctx, int H, int P,
    int keys_per_part) {
  // one workgroup per (b, h); 256 threads x 2 dims
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int h = bh - b * H;
  const int np = min(P, (int)((ctx[b] + keys_per_part - 1) / keys_per_part));
  float M = -INFINITY;
  for (int s = 0; s < np; ++s) M = fmaxf(M, part_ml[(((long)b * P + s) * H + h) * 2]);
  float lsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int d = threadIdx.x * 2;
  for (int s = 0; s < np; ++s) {
    const long base = ((long)b * P + s) * H + h;
    const float w = __builtin_amdgcn_exp2f(part_ml[base * 2] - M);
    lsum += w * part_ml[base * 2 + 1];
    acc0 += w * part_o[base * kLora + d];
    acc1 += w * part_o[base * kLora + d + 1];
  }
  const float inv = 1.f / lsum;
  *(uint32_t*)(o_lat + ((long)b * H + h) * kLora + d) = pack_bf16x2(acc0 * inv, acc1 * inv);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode_absorb(void* q_abs, const uint16_t* q, const uint16_t* w_uk, int B,
                                int H, bool fp8_out, hipStream_t stream) {
  // q_lat[b, h, l] = sum_d q[b, h, d] w_uk[h, l, d]: X = q (stride 192 per h),
  // W = w_uk[h] rows (l), K = 128, N = 512
  const int ntn = kLora / 32;
  const int tiles = ((B + 31) / 32) * ntn;
  const dim3 grid((tiles + 3) / 4, H);
  if (fp8_out)
    hipLaunchKernelGGL((head_gemm_kernel<kNope, true>), grid, dim3(256), 0, stream, q_abs, q,
                       w_uk, B, kLora, (long)H * kQDepth, (long)kQDepth, (long)kLora * kNope,
                       (long)H * kCache, (long)kCache, ntn);
  else
    hipLaunchKernelGGL((head_gemm_kernel<kNope, false>), grid, dim3(256), 0, stream, q_abs, q,
                       w_uk, B, kLora, (long)H * kQDepth, (long)kQDepth, (long)kLora * kNope,
                       (long)H * kCache, (long)kCache, ntn);
  const long n = (long)B * H * kRope;
  if (fp8_out)
    hipLaunchKernelGGL(copy_rope_kernel<true>, dim3((n + 255) / 256), dim3(256), 0, stream,
                       q_abs, q, B, H);
  else
    hipLaunchKernelGGL(copy_rope_kernel<false>, dim3((n + 255) / 256), dim3(256), 0, stream,
                       q_abs, q, B, H);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.B * a.P), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_combine(uint16_t* o_lat, const float* part_o, const float* part_ml,
                                 const uint32_t* ctx, int B, int H, int P, int keys_per_part,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * H), dim3(256), 0, stream, o_lat, part_o,
                     part_ml, ctx, H, P, keys_per_part);
  return hipGetLastError();
}

hipError_t launch_decode_project(uint16_t* out, const uint16_t* o_lat, const uint16_t* w_uv,
                                 int B, int H, hipStream_t stream) {
  // out[b, h, d] = sum_l o_lat[b, h, l] w_uv[h, d, l]: K = 512, N = 128
  const int ntn = kV / 32;
  const int tiles = ((B + 31) / 32) * ntn;
  const dim3 grid((tiles + 3) / 4, H);
  hipLaunchKernelGGL((head_gemm_kernel<kLora, false>), grid, dim3(256), 0, stream, out, o_lat,
                     w_uv, B, kV, (long)H * kLora, (long)kLora, (long)kV * kLora,
                     (long)H * kV, (long)kV, ntn);
  return hipGetLastError();
}

}  // namespace mla
