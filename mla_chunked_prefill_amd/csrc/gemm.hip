// Up-projection of the normalised latent to K_nope and V
// ("mla_prefill_decode_graph_bf16" page, Args "w_k" [H*128, 512] and "w_uv"
// [H, 128, 512]).
//
// One NT GEMM: C[r, n] = sum_l latent[r, l] W[n, l] with W = [w_k ; w_uv] viewed
// as [2*H*128, 512]; both operands are contiguous along the 512-long reduction.
// A 256-thread workgroup computes a 128-row x 128-column tile (one head of
// K_nope or of V) on bf16 MFMA 32x32x16 with fp32 accumulation; each of the four
// waves owns a 64x64 quadrant. The reduction is staged through LDS in 64-wide
// slices with one 16-byte global load per thread per operand quarter.
//
// The epilogue writes the layouts the attention kernel streams:
//   K_nope [H][rows][128]  (lanes run along d: contiguous 64-byte segments)
//   V^T    [H][128][rows]  (the tile is computed transposed, C^T = W latent^T,
//                           so lanes run along rows: contiguous segments)
#include "kernels.hpp"

namespace mla {

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmBK = 64;
constexpr int kGemmLdsRow = kGemmBK + 8;  // bf16 elements per LDS row (144 B: conflict-free)


template <bool kFp8K>
__global__ void __launch_bounds__(256, 2) up_project_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kGemmBM * kGemmLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kGemmBN * kGemmLdsRow];

  const int nrows = *g.bl_c;
  const int m0 = blockIdx.y * kGemmBM;
  if (nrows <= 0 || m0 >= nrows) return;
  const int ntile = blockIdx.x;            // 0 .. 2H-1
  const bool vpart = ntile >= g.H;
  const int h = vpart ? ntile - g.H : ntile;
  const uint16_t* W = (vpart ? g.wuv : g.wk) + (size_t)h * kNope * kLora;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * 64;  // quadrant row offset (rows of latent)
  const int wn = (wave & 1) * 64;   // quadrant column offset (d)
  const int l32 = lane & 31;
  const int khalf = (lane >> 5) * 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // each thread loads 4 x 16 B of A and 4 x 16 B of B per K slice
  for (int k0 = 0; k0 < kLora; k0 += kGemmBK) {
    u32x4 ra[4], rb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + it * 256;  // 0..1023: row = idx/8, chunk = idx%8
      const int r = idx >> 3;
      const int ch = idx & 7;
      const int grow = m0 + r;
      ra[it] = (grow < nrows && grow < g.max_rows)
                   ? *(const u32x4*)(g.a + (size_t)grow * kLora + k0 + ch * 8)
                   : u32x4{0, 0, 0, 0};
      rb[it] = *(const u32x4*)(W + (size_t)r * kLora + k0 + ch * 8);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + it * 256;
      const int r = idx >> 3;
      const int ch = idx & 7;
      *(u32x4*)(sA + r * kGemmLdsRow + ch * 8) = ra[it];
      *(u32x4*)(sB + r * kGemmLdsRow + ch * 8) = rb[it];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *(const bf16x8*)(sA + (wm + i * 32 + l32) * kGemmLdsRow + ks * 16 + khalf);
        fb[i] = *(const bf16x8*)(sB + (wn + i * 32 + l32) * kGemmLdsRow + ks * 16 + khalf);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (vpart)  // C^T tile: rows = d (from W), columns = latent rows
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
          else        // C tile: rows = latent rows, columns = d
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  // epilogue. acc[i][j] covers latent rows wm+32i.. and d = wn+32j..
  // MFMA output: lane holds column (lane%32) and rows (e/4)*8 + (lane/32)*4 + e%4.
  const int hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = (e >> 2) * 8 + hi4 + (e & 3);
        if (vpart) {
          // rows = d, column = latent row
          const int d = wn + 32 * j + rr;
          const int grow = m0 + wm + 32 * i + l32;
          if (grow < g.max_rows)
            g.vt_out[((size_t)h * kV + d) * g.max_rows + grow] =
                (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
        } else {
          const int grow = m0 + wm + 32 * i + rr;
          const int d = wn + 32 * j + l32;
          if (grow < g.max_rows) {
            const size_t o = ((size_t)h * g.max_rows + grow) * kNope + d;
            if (kFp8K) ((uint8_t*)g.k_out)[o] = (uint8_t)f32_to_e4m3_sat(acc[i][j][e]);
            else ((uint16_t*)g.k_out)[o] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
          }
        }
      }
}

hipError_t launch_up_project(const GemmArgs& g, bool fp8_k, hipStream_t stream) {
  const dim3 grid(2 * g.H, (g.max_rows + kGemmBM - 1) / kGemmBM);
  if (fp8_k) hipLaunchKernelGGL(up_project_kernel<true>, grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL(up_project_kernel<false>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace mla
