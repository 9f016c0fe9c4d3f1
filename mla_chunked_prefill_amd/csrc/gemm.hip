// Up-projection of the normalised latent to K_nope and V
// ("mla_prefill_decode_graph_bf16" page, Args "w_k" [H*128, 512] and "w_uv"
// [H, 128, 512]).
//
// One NT GEMM: C[r, n] = sum_l latent[r, l] W[n, l] with W = [w_k ; w_uv] viewed
// as [2*H*128, 512]; both operands are contiguous along the 512-long reduction.
// A 256-thread workgroup computes a 256-row x 128-column tile (one head of
// K_nope or of V) on bf16 MFMA 32x32x16 with fp32 accumulation; each of the
// four waves owns a 128 x 64 block, 4 x 2 MFMA blocks whose 128 accumulators
// leave room for two workgroups per CU: one's barriers, load waits and
// epilogue overlap the other's MFMAs.
//
// The 512-long reduction runs in 32-wide slices that go from global memory
// straight into three LDS stages with 16-byte direct loads
// (global_load_lds_dwordx4); 64-byte LDS rows keep their four 16-byte chunks
// XORed by (row / 4) % 4, so that the fragment reads (16 rows at one chunk per
// read phase) are conflict-free. One workgroup barrier per slice: slice s has
// landed everywhere and slice s - 1 is consumed, so its stage takes slice s + 2.
//
// Tile order: consecutive workgroups of one XCD (the hardware deals
// workgroups to the 8 XCDs in turn) take 8 heads' columns for one 256-row tile
// of the latent, then the next row tile, so that the 64 workgroups resident on
// an XCD share 8 heads of W (1 MB) and 8 row tiles of the latent (2 MB) in its
// L2.
//
// Epilogue: each wave stages its block in LDS in the destination's layout and
// writes it with 16-byte stores, whole 128- or 256-byte runs of contiguous
// memory:
//   K_nope [H][rows][128]  (bf16 or e4m3)
//   V^T    [H][128][rows]  (bf16)
// For that the stored dimension is put on the MFMA rows, where a lane holds
// four consecutive elements: K takes C^T = W latent^T, V^T takes C.
#include <type_traits>

#include "kernels.hpp"

namespace mla {

constexpr int kGemmBM = 256;                    // latent rows per workgroup
constexpr int kGemmBN = 128;                    // columns per workgroup: one head
constexpr int kGemmBK = 32;                     // reduction slice
constexpr int kGemmSlices = kLora / kGemmBK;    // 16
constexpr int kGemmRowB = kGemmBK * 2;          // 64 bytes per LDS row
constexpr int kGemmAB = kGemmBM * kGemmRowB;    // 16 KB of latent per stage
constexpr int kGemmWB = kGemmBN * kGemmRowB;    // 8 KB of W per stage
constexpr int kGemmStageB = kGemmAB + kGemmWB;  // 24 KB
constexpr int kGemmStages = 3;
constexpr int kGemmALoads = kGemmAB / 4096;     // direct loads per wave and slice: 4
constexpr int kGemmWLoads = kGemmWB / 4096;     // 2
constexpr int kGemmLoads = kGemmALoads + kGemmWLoads;
constexpr int kGemmEpiB = 16384;                // per wave in the epilogue
constexpr int kGemmColGroup = 8;                // heads' columns sharing a row tile in L2
constexpr int kGemmLdsB =
    kGemmStages * kGemmStageB > 4 * kGemmEpiB ? kGemmStages * kGemmStageB : 4 * kGemmEpiB;
static_assert(2 * kGemmLdsB <= 160 * 1024, "two workgroups per CU");
static_assert(kGemmSlices >= kGemmStages, "pipeline depth");

// the two 8-byte halves of a 16-byte chunk, exchanged when `swap`
__device__ __forceinline__ uint4 half_swap(uint4 v, int swap) {
  return swap ? make_uint4(v.z, v.w, v.x, v.y) : v;
}
// the two 4-byte words of each 8-byte half, exchanged when `swap`
__device__ __forceinline__ uint4 word_swap(uint4 v, int swap) {
  return swap ? make_uint4(v.y, v.x, v.w, v.z) : v;
}

// chunk permutation of a 64-byte operand row
__device__ __forceinline__ int gswz(int r) { return (r >> 2) & 3; }

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

// one 256 x 128 tile: latent rows m0 .., head h of the K part (kVPart false)
// or of the V part
template <bool kFp8K, bool kVPart>
__device__ __forceinline__ void up_project_tile(const GemmArgs& g, uint8_t* smem, int m0, int h,
                                                int nvalid) {
  const uint16_t* W = (kVPart ? g.wuv : g.wk) + (size_t)h * kNope * kLora;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * 128;  // block row offset (rows of latent)
  const int wn = (wave & 1) * 64;    // block column offset (d)
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // direct loads: load p of an operand slice fills LDS rows 16 p .. 16 p + 15,
  // lane -> row 16 p + lane / 4, LDS chunk lane % 4 holding source chunk
  // (lane % 4) ^ gswz(row); this wave issues loads p = wave + 4 k
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)smem);
  uint32_t offA[kGemmALoads], offW[kGemmWLoads];  // bytes from the operand bases
#pragma unroll
  for (int k = 0; k < kGemmALoads; ++k) {
    const int r = 16 * (wave + 4 * k) + (lane >> 2);
    const int ch = (lane & 3) ^ gswz(r);
    const int arow = min(m0 + r, nvalid - 1);  // past the chunk: a valid row, output zeroed
    offA[k] = (uint32_t)(arow * kLora * 2 + ch * 16);
  }
#pragma unroll
  for (int k = 0; k < kGemmWLoads; ++k) {
    const int r = 16 * (wave + 4 * k) + (lane >> 2);
    const int ch = (lane & 3) ^ gswz(r);
    offW[k] = (uint32_t)(r * kLora * 2 + ch * 16);
  }
  auto issue = [&](int s) __attribute__((always_inline)) {  // slice s -> stage s % stages
    const uint32_t base = lds0 + (s % kGemmStages) * kGemmStageB;
    const void* sa = g_uniform(g.a + s * kGemmBK);
    const void* sw = g_uniform(W + s * kGemmBK);
#pragma unroll
    for (int k = 0; k < kGemmALoads; ++k) gdma16(sa, offA[k], base + (wave + 4 * k) * 1024);
#pragma unroll
    for (int k = 0; k < kGemmWLoads; ++k) gdma16(sw, offW[k], base + kGemmAB + (wave + 4 * k) * 1024);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragments of one k-step: f[0..3] latent rows wm + 32 i + l32, f[4..5] W
  // rows wn + 32 j + l32, each the 16-byte chunk 2 ks + hf of its LDS row
  auto read = [&](int s, int ks, bf16x8* f) __attribute__((always_inline)) {
    const uint8_t* sA = smem + (s % kGemmStages) * kGemmStageB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm + 32 * i + l32;
      f[i] = *(const bf16x8*)(sA + r * kGemmRowB + (((2 * ks + hf) ^ gswz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn + 32 * j + l32;
      f[4 + j] = *(const bf16x8*)(sA + kGemmAB + r * kGemmRowB + (((2 * ks + hf) ^ gswz(r)) * 16));
    }
  };
  auto mfmas = [&](const bf16x8* f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (kVPart)  // C block: rows = latent rows, columns = d
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], f[4 + j], acc[i][j], 0, 0, 0);
        else  // C^T block: rows = d, columns = latent rows
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[4 + j], f[i], acc[i][j], 0, 0, 0);
      }
  };

  // Slice s lives in stage s % 3. At the barrier of slice s it has landed for
  // every wave and every wave has consumed slice s - 1, whose stage then
  // takes slice s + 2. Loads complete in order: waiting for slice s leaves
  // slice s + 1 in flight.
  issue(0);
  issue(1);
  bf16x8 f0[6], f1[6];
#pragma unroll 1
  for (int s = 0; s < kGemmSlices; ++s) {
    if (s + 1 < kGemmSlices) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kGemmLoads) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (s + 2 < kGemmSlices) issue(s + 2);
    read(s, 0, f0);
    read(s, 1, f1);
    mfmas(f0);
    mfmas(f1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Epilogue: each wave stages its 128 x 64 block (latent rows wm .. wm + 127
  // of the tile, d = wn .. wn + 63) in its own 16 KB of LDS, laid out as the
  // destination (K: [row][d], V^T: [d][row]), then writes it with 16-byte
  // stores. MFMA output: lane holds column l32 and rows 8q + 4hf + (0..3) in
  // registers 4q .. 4q + 3, i.e. four consecutive elements of the stored
  // dimension: one 8-byte LDS write (4 bytes for K in e4m3). 16-byte LDS
  // chunks are XORed by the line index so that the writes of 16 lines and the
  // reads of one line spread over the banks; in addition a line bit picks
  // which 8-byte half of a chunk (and, for e4m3, which 4-byte word of a half)
  // a lane writes, so that the 16 lanes an 8-byte write serves per cycle (32
  // for 4-byte writes) hit distinct banks of the 128-byte bank cycle; the
  // halves and words are put back in order after the 16-byte reads.
  // Rows of the chunk past nvalid are written as zeros, rows past max_rows
  // are not written.
  __syncthreads();  // every wave is done with the operand stages
  uint8_t* st = smem + wave * kGemmEpiB;
  const int row0 = m0 + wm;  // first latent row of the block
  // rows of the chunk past nvalid are zeroed only where the block reaches them
  auto stage_out = [&](auto masked) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
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
            *(uint2*)(st + line * 256 + chunk * 16 + 8 * (hf ^ ((line >> 3) & 1))) =
                make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
          } else {
            // line = latent row 32 i + l32; elements at d = 32 j + 8 q + 4 hf + e of the block
            const int line = 32 * i + l32;
            if (kMasked) {
              const bool ok = row0 + line < nvalid;
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = ok ? x[e] : 0.f;
            }
            if (kFp8K) {  // 64-byte lines
              const int chunk = (2 * j + (q >> 1)) ^ ((line >> 2) & 3);
              *(uint32_t*)(st + line * 64 + chunk * 16 + 8 * ((q & 1) ^ ((line >> 4) & 1)) +
                           4 * (hf ^ ((line >> 1) & 1))) =
                  f32_to_e4m3_sat(x[0]) | (f32_to_e4m3_sat(x[1]) << 8) |
                  (f32_to_e4m3_sat(x[2]) << 16) | (f32_to_e4m3_sat(x[3]) << 24);
            } else {  // 128-byte lines
              const int chunk = (4 * j + q) ^ ((line >> 1) & 7);
              *(uint2*)(st + line * 128 + chunk * 16 + 8 * (hf ^ (line & 1))) =
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
    // 64 lines (d) of 256 bytes (128 rows); an instruction covers lines 4 it .. 4 it + 3
    const int cg = lane & 15;
    if (row0 + 8 * cg < g.max_rows) {  // max_rows is a multiple of 64: whole chunks
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int line = 4 * it + (lane >> 4);
        const uint4 v = half_swap(*(const uint4*)(st + line * 256 + ((cg ^ (line & 15)) * 16)), (line >> 3) & 1);
        *(uint4*)((uint8_t*)g.vt_out + (((size_t)h * kV + wn + line) * g.max_rows + row0) * 2 + cg * 16) = v;
      }
    }
  } else if (kFp8K) {
    // 128 lines (rows) of 64 bytes; an instruction covers lines 16 it .. 16 it + 15
    const int cg = lane & 3;
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const int line = 16 * it + (lane >> 2);
      const uint4 v = word_swap(half_swap(*(const uint4*)(st + line * 64 + ((cg ^ ((line >> 2) & 3)) * 16)),
                                          (line >> 4) & 1),
                                (line >> 1) & 1);
      if (row0 + line < g.max_rows)
        *(uint4*)((uint8_t*)g.k_out + ((size_t)h * g.max_rows + row0 + line) * kNope + wn + cg * 16) = v;
    }
  } else {
    // 128 lines (rows) of 128 bytes; an instruction covers lines 8 it .. 8 it + 7
    const int cg = lane & 7;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int line = 8 * it + (lane >> 3);
      const uint4 v = half_swap(*(const uint4*)(st + line * 128 + ((cg ^ ((line >> 1) & 7)) * 16)), line & 1);
      if (row0 + line < g.max_rows)
        *(uint4*)((uint8_t*)g.k_out + (((size_t)h * g.max_rows + row0 + line) * kNope + wn) * 2 + cg * 16) = v;
    }
  }
}

// Tiles: 2 H columns (K of heads 0 .. H-1, then V) x R row tiles. Linear
// index L = (cg * R + rt) * 8 + c for column group cg, row tile rt and column
// cg * 8 + c; workgroup b takes L = (b % 8) * per_xcd + b / 8, so that every
// XCD runs a contiguous range of L.
template <bool kFp8K>
__global__ void __launch_bounds__(256, 2) up_project_kernel(GemmArgs g, int row_tiles, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmLdsB];
  const int nvalid = min(*g.bl_c, g.max_rows);
  const int L = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int c = L % kGemmColGroup;
  const int rt = (L / kGemmColGroup) % row_tiles;
  const int col = (L / (kGemmColGroup * row_tiles)) * kGemmColGroup + c;
  const int m0 = rt * kGemmBM;
  if (col >= 2 * g.H || nvalid <= 0 || m0 >= nvalid) return;
  if (col < g.H) up_project_tile<kFp8K, false>(g, smem, m0, col, nvalid);
  else up_project_tile<kFp8K, true>(g, smem, m0, col - g.H, nvalid);
}

hipError_t launch_up_project(const GemmArgs& g, bool fp8_k, hipStream_t stream) {
  const int row_tiles = (g.max_rows + kGemmBM - 1) / kGemmBM;
  const int groups = (2 * g.H + kGemmColGroup - 1) / kGemmColGroup;
  const long tiles = (long)groups * kGemmColGroup * row_tiles;
  const long per_xcd = (tiles + 7) / 8;
  if (8 * per_xcd > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(8 * per_xcd));
  if (fp8_k) hipLaunchKernelGGL(up_project_kernel<true>, grid, dim3(256), 0, stream, g, row_tiles, (int)per_xcd);
  else hipLaunchKernelGGL(up_project_kernel<false>, grid, dim3(256), 0, stream, g, row_tiles, (int)per_xcd);
  return hipGetLastError();
}

}  // namespace mla
