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
template <int K, bool kFp8Out, bool kTwoTerm = false>
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
    if (kTwoTerm) {  // x = hi + lo, lo stored K elements after hi
      u32x4 xl = *(const u32x4*)(xp + K + k0);
      if (brow >= B) xl = u32x4{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xl),
                                                    __builtin_bit_cast(bf16x8, wb), acc, 0, 0, 0);
    }
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
// 2. balanced split-KV attention over the latent cache (bf16 cache)
// ---------------------------------------------------------------------------
// The batch's contexts are laid end to end (N keys in all) and key range w of G
// covers keys [w*N/G, (w+1)*N/G): every range streams the same number of rows
// whatever the mix of context lengths. A range writes one partial state per
// sequence it touches, into slot w + b (injective over the touching pairs, at
// most G + B slots).
//
// Two workgroups share a range, one per half of the heads (64 each); they are
// numbered so that both land on the same XCD back to back and the second read
// of every tile hits that XCD's L2. A workgroup has four waves, one per SIMD:
// head group hg = wave & 1 (32 heads) and half dh = wave >> 1. For the scores
// S^T = Z Q^T (keys x heads, mfma 32x32x16: per-lane softmax statistics) a wave
// reduces its 288 of the 576 depths and the two waves of a head group add their
// partial score tiles through LDS; for the values O^T += Z^T P^T a wave keeps
// its 256 of the 512 latent dims, reading Z^T straight from the row-major tile
// with transposed LDS reads.
//
// The accumulator is never rescaled: each lane takes its first tile's maximum
// as the reference and later probabilities are formed against it (exact in
// bf16 and fp32 while below 2^64). A wave whose scores would exceed that
// marks its partials invalid (with the exact maximum of the segment, which it
// keeps tracking) and the combine step recomputes them.
//
// Tiles of 32 rows are triple-buffered in LDS by direct global->LDS loads. A
// row keeps its 72 16-byte chunks with the chunk index's low three bits XORed
// by zswz(row), which makes both the score-operand reads (16 rows at one
// column) and the transposed reads (4 rows x 64 bytes) bank-conflict free.
// Every LDS address the loop uses is a per-lane base plus an immediate.
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecHeads = 64;                     // heads per workgroup
constexpr int kDecBN = 32;                        // rows per tile
constexpr int kZRowChunks = 72;                   // 16-byte chunks per row
constexpr int kZRowB = kZRowChunks * 16;          // 1152 bytes
constexpr int kZLoads = kDecBN * kZRowChunks / 64;  // 36 wave loads of 1 KB
constexpr int kZStageB = kZLoads * 1024;          // 36864 bytes
constexpr int kZStages = 3;
constexpr int kDmaPerWave = kZLoads / kDecWaves;  // 9
static_assert(kZLoads % kDecWaves == 0, "every wave issues the same loads");

// XOR applied to the low three bits of a row's 16-byte chunk index
__device__ __forceinline__ int zswz(int row) { return 4 * ((row >> 1) & 1) + ((row >> 2) & 3); }
__device__ __forceinline__ int zchunk(int row, int chunk) { return (chunk & ~7) | ((chunk & 7) ^ zswz(row)); }
constexpr int kPTWindow = 2048;                   // page-table entries staged per segment

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// transposed 4 x 16-bit read: lane i of each 16-lane group receives element
// i % 4 of the 8 bytes addressed by lane 4k + i / 4, for k = 0..3
__device__ __forceinline__ bf16x4 ds_read_tr16(const uint8_t* lds_byte_ptr) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_byte_ptr)));
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds_dst + 16 l (lds_dst is wave-uniform). Issued as inline assembly so that
// the compiler does not treat later LDS reads of other stages as dependent on
// it (it would wait for every load in flight); the kernel orders these loads
// itself with s_waitcnt vmcnt, counting in issue order, and barriers. The
// asm sets m0 itself on every call; the compiler keeps no value of its own in
// m0 in these kernels (checked in their assembly), so the clobber is safe.
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_dst) {
  const uint32_t lds_addr = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "memory", "m0");
}

__global__ void __launch_bounds__(kDecThreads, 1) decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sZ[kZStages * kZStageB];
  __shared__ __attribute__((aligned(16))) float sX[kDecWaves * 16 * 64];
  __shared__ int sPT[kPTWindow];

  // workgroup -> (key range, head half); the two halves of a range share an XCD
  const int L = blockIdx.x;
  const int w = a.halves == 2 ? (L >> 4) * 8 + (L & 7) : L;
  const int half = a.halves == 2 ? (L >> 3) & 1 : 0;
  if (w >= a.G) return;
  const uint32_t N = a.cum[a.B];
  const uint32_t s_lo = (uint32_t)(((uint64_t)w * N) / a.G);
  const uint32_t s_hi = (uint32_t)(((uint64_t)(w + 1) * N) / a.G);
  if (s_lo >= s_hi) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 1;
  const int dh = wave >> 1;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int head = half * kDecHeads + hg * 32 + l32;
  const bool hvalid = head < a.H;
  const float sl2 = a.scale_log2;
  const uint16_t* cache = (const uint16_t*)a.cache;

  // per-lane LDS byte offsets (within a stage). Scores: row kappa (bits 2 and 3
  // of l32 swapped), chunk 36*dh + hf + 2*ks; ks = 4a + r -> s_base[r] + 128 a.
  const int kappa = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  int s_base[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s_base[r] = kappa * kZRowB + zchunk(kappa, 36 * dh + hf + 2 * r) * 16;
  // transposed reads for (ks, t): row 16*ks + 8*(g16/2) + 4*t + L16/4, bytes
  // 512*dh + 64*md + 32*(g16&1) + 8*(L16&3); md = 2a + pm -> tr_base[ks][t][pm] + 128 a
  const int g16 = lane >> 4, L16 = lane & 15;
  int tr_base[2][2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int pm = 0; pm < 2; ++pm) {
        const int row = 16 * ks + 8 * (g16 >> 1) + 4 * t + (L16 >> 2);
        const int chunk = 32 * dh + 4 * pm + 2 * (g16 & 1) + ((L16 >> 1) & 1);
        tr_base[ks][t][pm] = row * kZRowB + zchunk(row, chunk) * 16 + (L16 & 1) * 8;
      }
  // the DMA loads of this wave: j = wave + 4 i (i < 9) fills LDS chunks
  // 64 j + lane; keep (tile row << 8 | source chunk) per load, two per register
  int dma_rc[(kDmaPerWave + 1) / 2];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int pch = (wave + kDecWaves * i) * 64 + lane;
    const int row = pch / kZRowChunks;
    const int rc = (row << 8) | zchunk(row, pch - row * kZRowChunks);  // XOR is its own inverse
    if (i & 1) dma_rc[i >> 1] |= rc << 16; else dma_rc[i >> 1] = rc;
  }

  // first sequence touched: largest b with cum[b] <= s_lo
  int b;
  {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cum[mid] <= s_lo) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  uint32_t pos = s_lo;
  while (pos < s_hi) {
    const uint32_t seg_end = min(s_hi, a.cum[b + 1]);
    if (seg_end <= pos) { ++b; continue; }
    const int k0 = (int)(pos - a.cum[b]);
    const int k1 = (int)(seg_end - a.cum[b]);
    const int ntiles = (k1 - k0 + kDecBN - 1) / kDecBN;
    // the segment's page-table entries, staged in LDS once: the DMA queue then
    // holds only tile loads, so waits on it never stall for a table lookup
    const int lp0 = k0 / a.ps;
    const int npg = (k1 - 1) / a.ps - lp0 + 1;
    __syncthreads();  // the previous segment is done with the page window and the stages
    for (int i = tid; i < min(npg, kPTWindow); i += kDecThreads) {
      const int lp = lp0 + i;
      int pg = lp < a.maxp ? a.page_table[(size_t)b * a.maxp + lp] : 0;
      sPT[i] = (pg < 0 || pg >= a.num_pages) ? 0 : pg;
    }
    __syncthreads();

    auto issue = [&](int tile, int stage) {
      uint8_t* base = sZ + stage * kZStageB;
      const int kt = k0 + tile * kDecBN;
      // pool row of tile row (lane & 31); rows past the segment read a valid row
      const int key = min(kt + (lane & 31), k1 - 1);
      const int lp = key / a.ps;
      const int slot = sPT[min(lp - lp0, kPTWindow - 1)] * a.ps + (key - lp * a.ps);
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const int rc = (dma_rc[i >> 1] >> (16 * (i & 1))) & 0xFFFF;
        const int rs = __shfl(slot, rc >> 8, 64);
        dma16(cache + ((size_t)rs * kCache + (rc & 255) * 8), base + (wave + kDecWaves * i) * 1024);
      }
    };

    // absorbed queries of this wave's heads and depth half: 18 steps of 16
    bf16x8 qf[18];
    {
      const uint16_t* qp =
          a.q_abs + ((size_t)b * a.H + min(head, a.H - 1)) * kCache + 288 * dh + hf * 8;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        u32x4 v = hvalid ? *(const u32x4*)(qp + ks * 16) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // wait for q here, before any tile load is in flight: the compiler cannot
    // count the tile loads, so a wait it placed for q inside the tile loop
    // would drain them every tile (gfx9 encoding: vmcnt 0, others unlimited)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    float m_ref = -INFINITY;   // reference maximum (log2 domain)
    float m_seen = -INFINITY;  // largest scaled score of the segment (exact at the end)
    f32x16 o[8];
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[md][i] = 0.f;
    float l_run = 0.f;
    bool halted = false;  // wave-uniform: the partial is marked for recomputation

    issue(0, 0);
    if (ntiles > 1) issue(1, 1);

    for (int t = 0; t < ntiles; ++t) {
      // wait for this wave's loads of tile t (tile t+1's may stay in flight)
      if (t + 1 < ntiles) {
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // = kDmaPerWave
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      if (t + 2 < ntiles) issue(t + 2, (t + 2) % kZStages);
      const uint8_t* Z = sZ + (t % kZStages) * kZStageB;
      const int kt = k0 + t * kDecBN;

      // partial scores over this wave's depth half, in two independent chains
      f32x16 s, s2;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.f; s2[i] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < 18; ks += 2) {
        const bf16x8 za = *(const bf16x8*)(Z + s_base[ks & 3] + 128 * (ks >> 2));
        const bf16x8 zb = *(const bf16x8*)(Z + s_base[(ks + 1) & 3] + 128 * ((ks + 1) >> 2));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za, qf[ks], s, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zb, qf[ks + 1], s2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] += s2[i];
      float* xw = sX + wave * 1024;
#pragma unroll
      for (int i = 0; i < 16; ++i) xw[i * 64 + lane] = s[i];
      __syncthreads();
      const float* xp = sX + (wave ^ 2) * 1024;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] += xp[i * 64 + lane];

      // register i holds tile row 16*(i/8) + 8*hf + i%8
      if (kt + kDecBN > k1) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt + (i >> 3) * 16 + hf * 8 + (i & 7) >= k1) s[i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
      tmax = max_with_lane32(tmax);
      const float mt = tmax * sl2;  // finite: every tile holds a valid row
      m_seen = fmaxf(m_seen, mt);
      if (m_ref == -INFINITY) m_ref = mt;
      halted = halted || (__ballot(mt > m_ref + 64.0f) != 0);
      const float neg_m = -m_ref;
      float psum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 wv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[ks * 8 + 2 * j], sl2, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[ks * 8 + 2 * j + 1], sl2, neg_m));
          psum += p0 + p1;
          wv[j] = pack_bf16x2(p0, p1);
        }
        pb[ks] = __builtin_bit_cast(bf16x8, wv);
      }
      psum = sum_with_lane32(psum);
      l_run += psum;

      // O^T[256 dims x 32 heads] += Z^T P^T, Z^T read transposed from the row tile
#pragma unroll
      for (int md = 0; md < 8; ++md)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x4 a0 = ds_read_tr16(Z + tr_base[ks][0][md & 1] + 128 * (md >> 1));
          const bf16x4 a1 = ds_read_tr16(Z + tr_base[ks][1][md & 1] + 128 * (md >> 1));
          const bf16x8 va = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[md], 0, 0, 0);
        }
    }

    // partial state of (w, b): slot w + b
    if (hvalid) {
      const size_t base = ((size_t)(w + b) * a.H + head);
      float* op = a.part_o + base * kLora + 256 * dh;
      // O^T register i of block md: dim 32*md + 8*(i/4) + 4*hf + i%4 (within the half)
#pragma unroll
      for (int md = 0; md < 8; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = o[md][g * 4 + j];
          *(f32x4*)(op + md * 32 + g * 8 + hf * 4) = v;
        }
      if (hf == 0 && dh == 0) {
        // an overflowing head group hands (exact maximum, -1) to the combine
        // step, which recomputes this partial against that maximum
        // (both waves of a head group hold the same summed scores and flags)
        a.part_ml[base * 2 + 0] = halted ? m_seen : m_ref;
        a.part_ml[base * 2 + 1] = halted ? -1.0f : l_run;
      }
    }
    pos = seg_end;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// prefix sums of the context lengths (one workgroup)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_prefix_kernel(uint32_t* cum, const uint32_t* ctx,
                                                            int B) {
  __shared__ uint32_t s_scan[256];
  __shared__ uint32_t s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    const uint32_t v = b < B ? ctx[b] : 0u;
    s_scan[tid] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const uint32_t x = tid >= d ? s_scan[tid - d] : 0u;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    if (b < B) cum[b + 1] = s_carry + s_scan[tid];
    __syncthreads();
    if (tid == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  if (tid == 0) cum[0] = 0;
}

// ---------------------------------------------------------------------------
// 3. combine partial states: o_lat[b, h, :] (bf16)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t split_start(int w, uint32_t N, int G) {
  return (uint32_t)(((uint64_t)w * N) / G);
}

// Recompute the partial of (range w, sequence b, head h) against the exact
// maximum m (log2 domain) the split kernel recorded. Plain fp32 arithmetic,
// one key per thread for the scores; only reached for extreme score ranges.
__device__ void recompute_partial(const CombineArgs& c, int w, int b, int h, float m,
                                  float* sh_q, float* sh_p) {
  const int tid = threadIdx.x;
  const uint32_t N = c.cum[c.B];
  const uint32_t lo = max(split_start(w, N, c.G), c.cum[b]);
  const uint32_t hi = min(split_start(w + 1, N, c.G), c.cum[b + 1]);
  const int k0 = (int)(lo - c.cum[b]), k1 = (int)(hi - c.cum[b]);
  const uint16_t* qa = c.q_abs + ((size_t)b * c.H + h) * kCache;
  for (int e = tid; e < kCache; e += 256) sh_q[e] = bf16_to_f32(qa[e]);
  __syncthreads();
  const uint16_t* cache = (const uint16_t*)c.cache;
  auto row_of = [&](int key) -> const uint16_t* {
    const int lp = key / c.ps;
    int pg = lp < c.maxp ? c.page_table[(size_t)b * c.maxp + lp] : 0;
    if (pg < 0 || pg >= c.num_pages) pg = 0;
    return cache + ((size_t)pg * c.ps + (key - lp * c.ps)) * kCache;
  };
  float acc0 = 0.f, acc1 = 0.f, lsum = 0.f;
  const int d = 2 * tid;
  for (int kc = k0; kc < k1; kc += 256) {
    const int key = kc + tid;
    float p = 0.f;
    if (key < k1) {
      const uint16_t* z = row_of(key);
      float sc = 0.f;
      for (int e = 0; e < kCache; ++e) sc = fmaf(sh_q[e], bf16_to_f32(z[e]), sc);
      p = __builtin_amdgcn_exp2f(sc * c.scale_log2 - m);
    }
    sh_p[tid] = p;
    __syncthreads();
    const int n = min(256, k1 - kc);
    for (int k = 0; k < n; ++k) {
      const float pk = sh_p[k];
      const uint16_t* z = row_of(kc + k);
      acc0 = fmaf(pk, bf16_to_f32(z[d]), acc0);
      acc1 = fmaf(pk, bf16_to_f32(z[d + 1]), acc1);
      lsum += pk;
    }
    __syncthreads();
  }
  const size_t base = (size_t)(w + b) * c.H + h;
  c.part_o[base * kLora + d] = acc0;
  c.part_o[base * kLora + d + 1] = acc1;
  __syncthreads();
  if (tid == 0) {
    c.part_ml[base * 2 + 0] = m;
    c.part_ml[base * 2 + 1] = lsum;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) decode_combine_kernel(CombineArgs c) {
  __shared__ float sh_q[kCache];
  __shared__ float sh_p[256];
  // one workgroup per (b, h); 256 threads x 2 dims
  const int bh = blockIdx.x;
  const int b = bh / c.H;
  const int h = bh - b * c.H;
  const uint32_t N = c.cum[c.B];
  const uint32_t lo_key = c.cum[b], hi_key = c.cum[b + 1];  // keys [lo_key, hi_key)
  if (hi_key <= lo_key) return;
  // ranges touching the sequence: w_lo holds lo_key, w_hi holds hi_key - 1
  int w_lo, w_hi;
  {
    int lo = 0, hi = c.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (split_start(mid, N, c.G) <= lo_key) lo = mid; else hi = mid - 1;
    }
    w_lo = lo;
    lo = w_lo; hi = c.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (split_start(mid, N, c.G) < hi_key) lo = mid; else hi = mid - 1;
    }
    w_hi = lo;
  }
  float M = -INFINITY;
  for (int w = w_lo; w <= w_hi; ++w) {
    if (split_start(w, N, c.G) >= split_start(w + 1, N, c.G)) continue;  // empty range
    const size_t base = (size_t)(w + b) * c.H + h;
    const float m = c.part_ml[base * 2];
    if (c.part_ml[base * 2 + 1] < 0.f) recompute_partial(c, w, b, h, m, sh_q, sh_p);
    M = fmaxf(M, m);
  }
  float lsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int d = threadIdx.x * 2;
  for (int w = w_lo; w <= w_hi; ++w) {
    if (split_start(w, N, c.G) >= split_start(w + 1, N, c.G)) continue;
    const size_t base = (size_t)(w + b) * c.H + h;
    const float wt = __builtin_amdgcn_exp2f(c.part_ml[base * 2] - M);
    lsum += wt * c.part_ml[base * 2 + 1];
    const float2 v = *(const float2*)(c.part_o + base * kLora + d);
    acc0 += wt * v.x;
    acc1 += wt * v.y;
  }
  const float inv = 1.f / lsum;
  // o_lat as a bf16 pair (hi + lo): the output projection runs on bf16 MFMA
  // and takes both terms, so o_lat is not rounded to 8 bits on the way
  const float v0 = acc0 * inv, v1 = acc1 * inv;
  const uint32_t hi = pack_bf16x2(v0, v1);
  const uint32_t lo = pack_bf16x2(v0 - bf16_lo(hi), v1 - bf16_hi(hi));
  uint16_t* orow = c.o_lat + ((size_t)b * c.H + h) * (2 * kLora);
  *(uint32_t*)(orow + d) = hi;
  *(uint32_t*)(orow + kLora + d) = lo;
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

hipError_t launch_decode_prefix(uint32_t* cum, const uint32_t* ctx, int B, hipStream_t stream) {
  hipLaunchKernelGGL(decode_prefix_kernel, dim3(1), dim3(256), 0, stream, cum, ctx, B);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.halves == 2 ? 16 * ((a.G + 7) / 8) : a.G;
  hipLaunchKernelGGL(decode_split_kernel, dim3(grid), dim3(kDecThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const CombineArgs& c, hipStream_t stream) {
  hipLaunchKernelGGL(decode_combine_kernel, dim3(c.B * c.H), dim3(256), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_decode_project(uint16_t* out, const uint16_t* o_lat, const uint16_t* w_uv,
                                 int B, int H, hipStream_t stream) {
  // out[b, h, d] = sum_l o_lat[b, h, l] w_uv[h, d, l]: K = 512, N = 128; o_lat
  // rows hold hi then lo (2 x 512 bf16)
  const int ntn = kV / 32;
  const int tiles = ((B + 31) / 32) * ntn;
  const dim3 grid((tiles + 3) / 4, H);
  hipLaunchKernelGGL((head_gemm_kernel<kLora, false, true>), grid, dim3(256), 0, stream, out,
                     o_lat, w_uv, B, kV, (long)H * 2 * kLora, (long)2 * kLora,
                     (long)kV * kLora, (long)H * kV, (long)kV, ntn);
  return hipGetLastError();
}

}  // namespace mla
