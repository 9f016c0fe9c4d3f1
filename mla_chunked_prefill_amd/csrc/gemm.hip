// Up-projection of the normalised latent to K_nope and V
// ("mla_prefill_decode_graph_bf16" page, Args "w_k" [H*128, 512] and "w_uv"
// [H, 128, 512]).
//
// One NT GEMM: C[r, n] = sum_l latent[r, l] W[n, l] with W = [w_k ; w_uv] viewed
// as [2*H*128, 512]; both operands are contiguous along the 512-long reduction.
// A 256-thread workgroup computes a 256-row x 256-column tile (two heads of
// K_nope or of V) on bf16 MFMA 32x32x16 with fp32 accumulation; each of the
// four waves owns a 128 x 128 quadrant (one head), 4 x 4 MFMA blocks whose
// accumulators live in the accumulation registers, so every operand fragment
// read from LDS feeds four MFMAs.
//
// The 512-long reduction runs in 64-wide slices that go from global memory
// straight into LDS stages with 16-byte direct loads (global_load_lds_dwordx4);
// 128-byte LDS rows keep their eight 16-byte chunks XORed by (row / 2) % 8 so
// that the fragment reads (32 rows at one chunk) are conflict-free. The one
// workgroup barrier per slice sits before the slice's last 16-deep k-step:
// before it a wave has read all of the slice's fragments and waited for its
// own loads of the next slice; after it, the next slice's first fragments and
// a new slice's loads go out while the last k-step's MFMAs run. (32-wide
// slices, one barrier per two k-steps, measured 6% slower.)
//
// Epilogue: each wave stages its quadrant in LDS in the destination's layout
// and writes it with 16-byte stores, 1 KB of contiguous memory per
// instruction:
//   K_nope [H][rows][128]  (bf16 or e4m3)
//   V^T    [H][128][rows]  (bf16)
// For that the stored dimension is put on the MFMA rows, where a lane holds
// four consecutive elements: K takes C^T = W latent^T, V^T takes C.
#include <type_traits>

#include "kernels.hpp"

namespace mla {

constexpr int kGemmBM = 256;                   // latent rows per workgroup
constexpr int kGemmBK = 64;                    // reduction slice
constexpr int kGemmSlices = kLora / kGemmBK;   // 16
constexpr int kGemmRowB = kGemmBK * 2;         // 128 bytes per LDS row
constexpr int kGemmOpB = kGemmBM * kGemmRowB;  // 32 KB per operand and stage
constexpr int kGemmStageB = 2 * kGemmOpB;      // latent slice, then W slice
constexpr int kGemmStages = 2;                 // LDS stages (three measured no faster)
constexpr int kGemmEpiB = 32768;               // per wave in the epilogue
constexpr int kGemmLdsB =
    kGemmStages * kGemmStageB > 4 * kGemmEpiB ? kGemmStages * kGemmStageB : 4 * kGemmEpiB;
static_assert(kGemmStages >= 2 && kGemmStages <= 4, "LDS stages");
static_assert(kGemmLdsB <= 160 * 1024, "LDS of one CU");

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

// direct global -> LDS load of 16 bytes per lane from sbase + voff (sbase
// wave-uniform) to lds + 16 lane; ordered by s_waitcnt vmcnt and barriers
__device__ __forceinline__ void gdma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ const void* g_uniform(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
// one 256 x 256 tile: latent rows m0 .., heads h0, h0 + 1 of the K part
// (kVPart false) or of the V part
template <bool kFp8K, bool kVPart>
__device__ __forceinline__ void up_project_tile(const GemmArgs& g, uint8_t* smem, int m0, int h0,
                                                int nvalid) {
  const int n_h = min(2, g.H - h0);  // heads of this tile (1 for an odd last pair)
  // 256 rows of W: heads h0, h0 + 1 (a lone last head serves both halves)
  const uint16_t* W = (kVPart ? g.wuv : g.wk) + (size_t)h0 * kNope * kLora;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * 128;  // quadrant row offset (rows of latent)
  const int wn = (wave & 1) * 128;   // quadrant column offset (d of head h0 + (wave & 1))
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // direct loads: load p (of 32) of an operand slice fills LDS rows 8 p ..
  // 8 p + 7, lane -> row 8 p + lane / 8, LDS chunk lane % 8 holding source
  // chunk (lane % 8) ^ gswz(row); this wave issues loads p = wave + 4 k
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)smem);
  uint32_t offA[8], offB[8];  // bytes from the operand bases
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int p = wave + 4 * k;
    const int r = 8 * p + (lane >> 3);
    const int ch = (lane & 7) ^ gswz(r);
    const int arow = min(m0 + r, nvalid - 1);      // past the chunk: a valid row, output zeroed
    const int wrow = r < 128 * n_h ? r : r - 128;  // a lone last head: its own rows again
    offA[k] = (uint32_t)(arow * kLora * 2 + ch * 16);
    offB[k] = (uint32_t)(wrow * kLora * 2 + ch * 16);
  }
  auto issue = [&](int s) __attribute__((always_inline)) {  // slice s -> stage s % stages
    const uint32_t base = lds0 + (s % kGemmStages) * kGemmStageB;
    const void* sa = g_uniform(g.a + s * kGemmBK);
    const void* sb = g_uniform(W + s * kGemmBK);
#pragma unroll
    for (int k = 0; k < 8; ++k) gdma16(sa, offA[k], base + (wave + 4 * k) * 1024);
#pragma unroll
    for (int k = 0; k < 8; ++k) gdma16(sb, offB[k], base + kGemmOpB + (wave + 4 * k) * 1024);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragments of one k-step: f[0..3] latent rows wm + 32 i + l32, f[4..7] W
  // rows wn + 32 j + l32, each the 16-byte chunk 2 ks + hf of its LDS row
  auto read = [&](int s, int ks, bf16x8* f) __attribute__((always_inline)) {
    const uint8_t* sA = smem + (s % kGemmStages) * kGemmStageB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm + 32 * i + l32;
      f[i] = *(const bf16x8*)(sA + r * kGemmRowB + (((2 * ks + hf) ^ gswz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn + 32 * j + l32;
      f[4 + j] = *(const bf16x8*)(sA + kGemmOpB + r * kGemmRowB + (((2 * ks + hf) ^ gswz(r)) * 16));
    }
  };
  auto mfmas = [&](const bf16x8* f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kVPart)  // C block: rows = latent rows, columns = d
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], f[4 + j], acc[i][j], 0, 0, 0);
        else  // C^T block: rows = d, columns = latent rows
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[4 + j], f[i], acc[i][j], 0, 0, 0);
      }
  };

  // prologue: every stage loading, slice 0 landed everywhere, its first
  // fragments read
#pragma unroll
  for (int s = 0; s < kGemmStages; ++s) issue(s);
  static_assert(kGemmStages == 2, "wait counts");
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // slice 0 landed, slice 1 may not have
  __syncthreads();
  bf16x8 f0[8], f1[8];
  read(0, 0, f0);

  // Slice s lives in stage s % stages and takes four 16-deep k-steps. At the
  // barrier before its last k-step every wave has all of slice s in
  // registers and its own loads of slice s + 1 landed: slice s + 1 can be
  // read, and stage s % stages takes slice s + 2. sched_barrier fences keep
  // each k-step's MFMAs between the waits and barriers that bound them
  // (MFMAs touch no memory, so the scheduler would otherwise move them).
#pragma unroll 1
  for (int s = 0; s < kGemmSlices; ++s) {
    read(s, 1, f1);
    mfmas(f0);  // k-step 0 of slice s
    __builtin_amdgcn_sched_barrier(0);
    read(s, 2, f0);
    mfmas(f1);  // k-step 1
    __builtin_amdgcn_sched_barrier(0);
    read(s, 3, f1);
    mfmas(f0);  // k-step 2
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < kGemmSlices) {
      // slice s + 1 is the last one issued: wait for all of this wave's loads
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slice s fully in registers
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if (s + kGemmStages < kGemmSlices) issue(s + kGemmStages);
      read(s + 1, 0, f0);
    }
    mfmas(f1);  // k-step 3 of slice s
    __builtin_amdgcn_sched_barrier(0);
  }

  // Epilogue: each wave stages its 128 x 128 quadrant (one head: latent rows
  // wm .. wm + 127 of the tile, all 128 d) in its own 32 KB of LDS, laid out
  // as the destination (K: [row][d], V^T: [d][row]), then writes it with
  // 16-byte stores that cover 1 KB of contiguous memory per instruction.
  // MFMA output: lane holds column l32 and rows 8q + 4hf + (0..3) in
  // registers 4q .. 4q + 3, i.e. four consecutive elements of the stored
  // dimension: one 8-byte LDS write (4 bytes for K in e4m3). 16-byte LDS
  // chunks are XORed by the line index so that writes and reads spread over
  // the banks. Rows of the chunk past nvalid are written as zeros, rows past
  // max_rows are not written.
  const int h = h0 + (wave & 1);
  __syncthreads();  // every wave is done with the operand stages
  if (h >= g.H) return;  // the second half of a lone last head
  uint8_t* st = smem + wave * kGemmEpiB;
  const int row0 = m0 + wm;  // first latent row of the quadrant
  // rows of the chunk past nvalid are zeroed only where the quadrant reaches them
  auto stage_out = [&](auto masked) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        asm volatile("" : "+a"(acc[i][j]));  // one block in ordinary registers at a time
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = acc[i][j][4 * q + e];
          if (kVPart) {
            // line = d (32 j + l32), 256 bytes of rows; elements at rows 32 i + 8 q + 4 hf + e
            const int line = 32 * j + l32;
            const int r = 32 * i + 8 * q + 4 * hf;
            if (kMasked) {
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = row0 + r + e < nvalid ? x[e] : 0.f;
            }
            const int chunk = (4 * i + q) ^ (line & 15);
            *(uint2*)(st + line * 256 + chunk * 16 + 8 * hf) =
                make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
          } else {
            // line = latent row 32 i + l32; elements at d = 32 j + 8 q + 4 hf + e
            const int line = 32 * i + l32;
            if (kMasked) {
              const bool ok = row0 + line < nvalid;
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = ok ? x[e] : 0.f;
            }
            if (kFp8K) {  // 128-byte lines
              const int chunk = (2 * j + (q >> 1)) ^ ((line >> 1) & 7);
              *(uint32_t*)(st + line * 128 + chunk * 16 + 8 * (q & 1) + 4 * hf) =
                  f32_to_e4m3_sat(x[0]) | (f32_to_e4m3_sat(x[1]) << 8) |
                  (f32_to_e4m3_sat(x[2]) << 16) | (f32_to_e4m3_sat(x[3]) << 24);
            } else {
              const int chunk = (4 * j + q) ^ (line & 15);
              *(uint2*)(st + line * 256 + chunk * 16 + 8 * hf) =
                  make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
            }
          }
        }
      }
  };
  if (row0 + 128 <= nvalid) stage_out(std::false_type{});
  else stage_out(std::true_type{});
  // the wave reads lines other lanes wrote: complete the writes first
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (kVPart) {
    // 128 lines of 256 bytes; an instruction covers lines 4 it .. 4 it + 3
    const int cg = lane & 15;
    if (row0 + 8 * cg < g.max_rows) {  // max_rows is a multiple of 64: whole chunks
#pragma unroll 4
      for (int it = 0; it < 32; ++it) {
        const int line = 4 * it + (lane >> 4);
        const uint4 v = *(const uint4*)(st + line * 256 + ((cg ^ (line & 15)) * 16));
        *(uint4*)((uint8_t*)g.vt_out + (((size_t)h * kV + line) * g.max_rows + row0) * 2 + cg * 16) = v;
      }
    }
  } else if (kFp8K) {
    // 128 lines of 128 bytes; an instruction covers lines 8 it .. 8 it + 7
    const int cg = lane & 7;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int line = 8 * it + (lane >> 3);
      const uint4 v = *(const uint4*)(st + line * 128 + ((cg ^ ((line >> 1) & 7)) * 16));
      if (row0 + line < g.max_rows)
        *(uint4*)((uint8_t*)g.k_out + ((size_t)h * g.max_rows + row0 + line) * kNope + cg * 16) = v;
    }
  } else {
    // 128 lines of 256 bytes; an instruction covers lines 4 it .. 4 it + 3
    const int cg = lane & 15;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int line = 4 * it + (lane >> 4);
      const uint4 v = *(const uint4*)(st + line * 256 + ((cg ^ (line & 15)) * 16));
      if (row0 + line < g.max_rows)
        *(uint4*)((uint8_t*)g.k_out + ((size_t)h * g.max_rows + row0 + line) * kNope * 2 + cg * 16) = v;
    }
  }
}

template <bool kFp8K>
__global__ void __launch_bounds__(256, 1) up_project_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmLdsB];
  const int nvalid = min(*g.bl_c, g.max_rows);
  const int m0 = blockIdx.y * kGemmBM;
  if (nvalid <= 0 || m0 >= nvalid) return;
  const int npairs = (g.H + 1) / 2;
  const int ntile = blockIdx.x;  // 0 .. 2 npairs - 1: pairs of heads, K part then V part
  if (ntile < npairs) up_project_tile<kFp8K, false>(g, smem, m0, 2 * ntile, nvalid);
  else up_project_tile<kFp8K, true>(g, smem, m0, 2 * (ntile - npairs), nvalid);
}

hipError_t launch_up_project(const GemmArgs& g, bool fp8_k, hipStream_t stream) {
  const dim3 grid(2 * ((g.H + 1) / 2), (g.max_rows + kGemmBM - 1) / kGemmBM);
  if (fp8_k) hipLaunchKernelGGL(up_project_kernel<true>, grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL(up_project_kernel<false>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace mla
