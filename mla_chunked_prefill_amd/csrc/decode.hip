// Absorbed MLA decode ("mla_prefill_decode_graph_bf16" page: decode branch,
// Args "w_uk" [H, 512, 128] and "w_uv" [H, 128, 512], num_partitions;
// "flare_mla_prefill_dispatch" page: kv_num_heads 1, cache_depth 576).
//
// Four steps:
//  1. absorb:   q_abs[b, h] = [w_uk[h] q_nope[b, h] | q_rope[b, h]] (576 wide),
//               bf16 MFMA, operands read straight from global memory (both
//               are contiguous along the 128-long reduction).
//  2. split-KV: the batch's contexts laid end to end are cut into G equal key
//               ranges; one workgroup per range streams its 576-wide cache
//               rows once for all 128 heads and keeps an unnormalised
//               softmax state (max, sum, O_lat) per sequence it touches.
//  3. combine:  per (sequence, head), the states of the key ranges that
//               touched the sequence are merged by log-sum-exp into o_lat.
//  4. project:  out[b, h] = w_uv[h] o_lat[b, h], bf16 MFMA, one wave per
//               32 x 32 output tile.
#include <array>
#include <type_traits>

#include "kernels.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// 1, 4. per-head small GEMMs (bf16 MFMA 32x32x16, fp32 accumulation)
// ---------------------------------------------------------------------------
// Both are latency-bound (about 1 GFLOP and 17 MB of weights each at 64
// sequences and 128 heads): every wave issues all of its operand loads
// straight from global memory at once (both operands are contiguous along
// the reduction), then runs its MFMAs. A lane's 16-byte operand fragment is
// row l32 of a 32-row block, reduction elements 16 k + 8 hf .. + 7.

// ---------------------------------------------------------------------------
// prefix sums of the context lengths (one workgroup)
// ---------------------------------------------------------------------------
// The context length of sequence b is ctx[b] + add (add is 1 when ctx holds
// cache lengths that exclude the new token). Lengths above max_ctx (the
// host's bound, which sized the ranges) are taken as max_ctx, so the prefix
// sums stay below 2^31 whatever the device holds; the results of such
// sequences are unspecified, their reads in bounds.
// Run by one workgroup of 256 threads (the extra column of the absorb grid).
__device__ void decode_prefix(const PrefixArgs& pa) {
  uint32_t* cum = pa.cum;
  const uint32_t* ctx = pa.ctx;
  const uint32_t add = pa.add;
  const int B = pa.B;
  const uint32_t max_ctx = pa.max_ctx;
  uint32_t* wstart = pa.wstart;
  int2* wspan = pa.wspan;
  int32_t* wfirst = pa.wfirst;
  const int G = pa.G;
  __shared__ uint32_t s_scan[256];
  __shared__ uint32_t s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    const uint32_t v = b < B ? (uint32_t)min((uint64_t)ctx[b] + add, (uint64_t)max_ctx) : 0u;
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
  // key range w covers keys [wstart[w], wstart[w+1])
  const uint32_t N = s_carry;
  for (int w = tid; w <= G; w += 256) wstart[w] = (uint32_t)(((uint64_t)w * N) / G);
  __threadfence();  // other threads of the workgroup read these entries below
  __syncthreads();
  // first sequence of every key range: largest b with cum[b] <= wstart[w]
  for (int w = tid; w < G; w += 256) {
    const uint32_t key = wstart[w];
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= key) lo = mid; else hi = mid - 1;
    }
    wfirst[w] = lo;
  }
  // ranges holding sequence b's first and last keys (empty sequences: (0, -1))
  for (int b = tid; b < B; b += 256) {
    const uint32_t lo_key = cum[b], hi_key = cum[b + 1];
    if (hi_key <= lo_key) { wspan[b] = make_int2(0, -1); continue; }
    int lo = 0, hi = G - 1;  // largest w with wstart[w] <= lo_key
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wstart[mid] <= lo_key) lo = mid; else hi = mid - 1;
    }
    const int w_lo = lo;
    hi = G - 1;              // largest w with wstart[w] < hi_key
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wstart[mid] < hi_key) lo = mid; else hi = mid - 1;
    }
    wspan[b] = make_int2(w_lo, lo);
  }
}

// q_abs[b, h, 0:512] = w_uk[h] q_nope[b, h]; q_abs[b, h, 512:576] = q_rope[b, h].
// Grid (H + 1, ceil(B / 64)): workgroup (h, z) handles head h for sequences
// 64 z .. 64 z + 63. Their q_nope rows (16 KB) are staged in LDS once, 16-byte
// chunks XORed by (row % 16) so that 32 rows read at one chunk hit distinct
// banks; wave v computes latent dims 128 v .. 128 v + 127 (four 32-dim blocks,
// all w_uk loads issued up front) as D = W Q^T, so that a lane holds four runs
// of four consecutive dims of one sequence; an exchange with the lane 32 away
// turns them into two runs of eight, each stored with one 16-byte store. The
// workgroup also copies the rope part of its sequences. Workgroup (H, 0)
// computes the split-KV prefix sums; the rest of column H exits.
__global__ void __launch_bounds__(256) absorb_kernel(uint16_t* __restrict__ q_abs,
                                                     const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ w_uk, int B,
                                                     int H, PrefixArgs pa) {
  if ((int)blockIdx.x == H) {
    if (blockIdx.y == 0) decode_prefix(pa);
    return;
  }
  __shared__ __attribute__((aligned(16))) uint8_t sq[64 * 256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * 64;
  constexpr int kSteps = kNope / 16;  // 8
  // this wave's w_uk rows: four blocks of 32 dims, all loads up front
  u32x4 wf[4][kSteps];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const uint16_t* wp = w_uk + ((size_t)h * kLora + wave * 128 + nb * 32 + l32) * kNope + hf * 8;
#pragma unroll
    for (int k = 0; k < kSteps; ++k) wf[nb][k] = *(const u32x4*)(wp + 16 * k);
  }
  // q_nope rows of the 64 sequences: thread t loads row t / 4, chunks 4 (t % 4) ..
  {
    const int r = tid >> 2;
    const int b = min(b0 + r, B - 1);
    const uint16_t* qp = q + ((size_t)b * H + h) * kQDepth;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = (tid & 3) * 4 + j;
      u32x4 v = *(const u32x4*)(qp + c * 8);
      if (b0 + r >= B) v = u32x4{0, 0, 0, 0};
      *(u32x4*)(sq + r * 256 + ((c ^ (r & 15)) * 16)) = v;
    }
    // the rope part of the same rows: 64 rows x 8 chunks, two per thread
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int piece = j * 256 + tid;
      const int rr = piece >> 3, c = (piece & 7) * 8;
      if (b0 + rr < B)
        *(u32x4*)(q_abs + ((size_t)(b0 + rr) * H + h) * kCache + kLora + c) =
            *(const u32x4*)(q + ((size_t)(b0 + rr) * H + h) * kQDepth + kNope + c);
    }
  }
  __syncthreads();
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    bf16x8 xf[kSteps];
    const int r = bt * 32 + l32;
#pragma unroll
    for (int k = 0; k < kSteps; ++k)
      xf[k] = *(const bf16x8*)(sq + r * 256 + (((2 * k + hf) ^ (r & 15)) * 16));
    const int b = b0 + r;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int k = 0; k < kSteps; ++k)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wf[nb][k]),
                                                      xf[k], acc, 0, 0, 0);
      // lane holds sequence b, dims n0 + 8 (i / 4) + 4 hf + i % 4
      const int n0 = wave * 128 + nb * 32;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          uint32_t x[2][2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            // lanes 0-31 keep odd-group values and take the upper lanes' ones;
            // lanes 32-63 take the lower lanes' even-group values
            const auto rr2 = __builtin_amdgcn_permlane32_swap(
                __float_as_uint(acc[(2 * pr + 1) * 4 + e + u]),
                __float_as_uint(acc[(2 * pr) * 4 + e + u]), false, false);
            x[u][0] = rr2[0];
            x[u][1] = rr2[1];
          }
          o[e / 2] = pack_bf16x2(__uint_as_float(x[0][0]), __uint_as_float(x[1][0]));
          o[2 + e / 2] = pack_bf16x2(__uint_as_float(x[0][1]), __uint_as_float(x[1][1]));
        }
        const int dim0 = n0 + 8 * (2 * pr + (hf ^ 1));
        if (b < B) *(u32x4*)(q_abs + ((size_t)b * H + h) * kCache + dim0) = o;
      }
    }
  }
}

// Projection: C[b, n] = sum_k X[b, k] W[n, k] per head.
// X rows: x + b*x_stride (K contiguous, bf16); W rows: w + n*K (K contiguous).
// Output: y[b*y_stride + n] as bf16. One wave computes a 32 (b) x 32 (n) tile;
// K is a multiple of 16. kTwoTerm: X = hi + lo, with lo stored K elements
// after hi.
template <int K, bool kTwoTerm = false>
__global__ void __launch_bounds__(256) head_gemm_kernel(
    uint16_t* __restrict__ y, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
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
    if (kTwoTerm) {
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
      y[o] = (uint16_t)f32_to_bf16_rne(acc[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. split-KV attention over the latent cache
// ---------------------------------------------------------------------------
// Key ranges. The contexts laid end to end hold N keys; range w of G covers
// keys [w*N/G, (w+1)*N/G), so every range streams the same number of rows
// whatever the mix of context lengths. A range writes one partial state per
// sequence it touches, into slot w + b (injective over the touching pairs, at
// most G + B slots).
//
// One workgroup per range, four waves, one per SIMD; wave w owns heads
// 32w .. 32w+31 completely: its absorbed queries (576 deep, 144 registers)
// and its unnormalised output O^T (512 dims x 32 heads fp32, held in the
// accumulation registers) stay resident, so no score or output crosses
// between waves and each cache row is read from memory once for all heads.
// Per tile of 32 keys a wave computes S^T = Z Q^T (keys x heads, 36 MFMA
// steps of mfma 32x32x16 in two accumulation chains; each lane owns one head,
// its softmax statistics are in-lane plus one exchange with the lane 32
// away) and accumulates O^T += Z^T P^T (16 dim blocks x 2 key steps), reading
// Z^T straight from the row-major tile with transposed LDS reads. Key rows
// are fed to the score MFMA in the order kappa (bits 2 and 3 of the row index
// swapped), which makes the bf16 probabilities directly the B operand of the
// value product. LDS operands are read four MFMAs ahead into rotating
// registers.
//
// The softmax reference maximum of a segment is its first tile's maximum and
// never moves, so the output accumulator is never rescaled. Probabilities
// stay below 2^kDecSlack (far inside fp32 and bf16 range) unless a later
// score exceeds the reference by more than kDecSlack log2 units; a wave that
// sees one marks its partial states, and the combine step recomputes them
// against their exact maximum.
//
// Tiles are aligned to 32 keys of the sequence (keys of the first tile before
// the range start are masked), one barrier per tile. A wave computes tile
// t's scores, then tile t-1's value product with tile t's softmax placed
// between its MFMAs (those MFMAs wait on LDS reads, which leaves room for the
// vector work); the loads of tile t+2 go out while tile t's scores are
// computed. Four stages hold tiles t-1 .. t+2. When the page size is a
// multiple of 32 a tile is 32 consecutive pool rows (36 KB in one piece) and
// its direct loads are spread between the score MFMAs; otherwise every row's
// pool slot is looked up and the loads go out in one burst. A row keeps its
// 72 16-byte chunks with the chunk index's low three bits XORed by zswz(row),
// so the score reads (16 rows at one column) and the transposed reads (4 rows
// x 64 bytes) touch distinct LDS banks.
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecBN = 32;                          // keys per tile
constexpr int kZRowChunks = 72;                     // 16-byte chunks per row
constexpr int kZRowB = kZRowChunks * 16;            // 1152 bytes
constexpr int kZStageB = kDecBN * kZRowB;           // 36864 bytes
constexpr int kZStages = 4;
constexpr int kZLoads = kZStageB / 1024;            // 36 wave loads of 1 KB
constexpr int kZLoadsPerWave = kZLoads / kDecWaves; // 9
constexpr int kPTWindow = kDecPageWindow;           // page-table entries staged per segment
constexpr int kQSteps = kCache / 16;                // 36 score steps
constexpr float kDecSlack = 64.0f;
static_assert(kZLoads % kDecWaves == 0, "even bf16 loads per wave");
static_assert(kPTWindow % kDecThreads == 0, "even page-table staging per thread");

// XOR applied to the low three bits of a row's 16-byte chunk index
__device__ __forceinline__ int zswz(int row) { return 4 * ((row >> 1) & 1) + ((row >> 2) & 3); }
__device__ __forceinline__ int zchunk(int row, int chunk) { return (chunk & ~7) | ((chunk & 7) ^ zswz(row)); }

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// transposed 4 x 16-bit read: lane i of each 16-lane group receives element
// i % 4 of the 8 bytes addressed by lane 4k + i / 4, for k = 0..3
__device__ __forceinline__ bf16x4 ds_read_tr16(const uint8_t* lds_byte_ptr) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_byte_ptr)));
}

// Direct global -> LDS loads: lane l's 16 bytes land at lds + 16 l; lds is
// wave-uniform. Inline assembly keeps the compiler from
// treating later LDS reads of other stages as dependent on them (it would
// wait for every load in flight); the kernel orders these loads itself with
// s_waitcnt vmcnt, counting in issue order, and barriers. The asm sets m0 on
// every call; the kernels keep no value of their own in m0. The variants
// without a compiler memory barrier are issued between the score MFMAs of
// another stage, where the kernel never touches the target stage.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_s_nb(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "m0");
}
__device__ __forceinline__ const void* uniform_ptr_d(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

__global__ void __launch_bounds__(kDecThreads, 1) decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sZ[kZStages * kZStageB];
  __shared__ int sPT[kPTWindow];

  const int w = blockIdx.x;
  if (w >= a.G) return;
  const uint32_t s_lo = a.wstart[w];
  const uint32_t s_hi = a.wstart[w + 1];
  if (s_lo >= s_hi) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int head = wave * 32 + l32;
  const bool hvalid = head < a.H;
  const float sl2 = a.scale_log2;
  const uint8_t* cache = (const uint8_t*)a.cache;
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)sZ);

  // ---- per-lane LDS read offsets (bytes inside a stage) ----
  // scores: row kappa, step ks = 4c + r reads chunk 2 ks + hf at s_base[r] + 128 c
  const int kappa = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  int s_base[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s_base[r] = kappa * kZRowB + zchunk(kappa, 2 * r + hf) * 16;
  // transposed reads for key step ks, half t, dim block md = 2 c + pm: row
  // 16 ks + 8 (g16 / 2) + 4 t + L16 / 4, bytes 64 md + 32 (g16 & 1) +
  // 8 (L16 & 3) -> tr_base[t][pm] + 18432 ks + 128 c (the swizzle ignores
  // row bit 4)
  const int g16 = lane >> 4, L16 = lane & 15;
  int tr_base[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int pm = 0; pm < 2; ++pm) {
      const int row = 8 * (g16 >> 1) + 4 * t + (L16 >> 2);
      const int chunk = 4 * pm + 2 * (g16 & 1) + ((L16 >> 1) & 1);
      tr_base[t][pm] = row * kZRowB + zchunk(row, chunk) * 16 + (L16 & 1) * 8;
    }
  // direct loads of a contiguous tile: load j of this wave (p = wave + 4 j)
  // fills LDS chunks 64 p + lane, i.e. tile row rr, source chunk zchunk(rr,
  // cc) (the XOR is its own inverse); byte offsets below 36 KB, two per
  // register
  uint32_t dma_pk[(kZLoadsPerWave + 1) / 2];
#pragma unroll
  for (int j = 0; j < kZLoadsPerWave; ++j) {
    const int pch = (wave + kDecWaves * j) * 64 + lane;
    const int rr = pch / kZRowChunks;
    const uint32_t off = (uint32_t)(rr * kZRowB + zchunk(rr, pch - rr * kZRowChunks) * 16);
    if (j & 1) dma_pk[j >> 1] |= off << 16; else dma_pk[j >> 1] = off;
  }
  auto dma_off = [&](int j) __attribute__((always_inline)) {
    return (dma_pk[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
  };
  const bool contiguous = (a.ps % kDecBN) == 0;

  int b = a.wfirst[w];  // first sequence the range touches
  uint32_t pos = s_lo;
  while (pos < s_hi) {
    const uint32_t seg_end = min(s_hi, a.cum[b + 1]);
    if (seg_end <= pos) { ++b; continue; }
    const int k0 = (int)(pos - a.cum[b]);
    const int k1 = (int)(seg_end - a.cum[b]);
    const int kt0 = k0 & ~(kDecBN - 1);
    const int ntiles = (k1 - kt0 + kDecBN - 1) / kDecBN;
    const int ctx_b = (int)(a.cum[b + 1] - a.cum[b]);
    const int lp0 = kt0 / a.ps;
    const int npg = (k1 - 1) / a.ps - lp0 + 1;
    // absorbed queries of this wave's heads, all 36 score steps; their loads
    // go out together with the page-table loads below
    bf16x8 qf[kQSteps];
    {
      const uint16_t* qrow = a.q_abs + ((size_t)b * a.H + min(head, a.H - 1)) * kCache + hf * 8;
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks) {
        u32x4 v = hvalid ? *(const u32x4*)(qrow + ks * 16) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // the segment's page-table entries, staged in LDS once: the first two per
    // thread are loaded before the barrier, the rest after it (registers)
    auto pt_entry = [&](int e) __attribute__((always_inline)) {
      const int lp = lp0 + e;
      const int v = (e < npg && lp < a.maxp) ? a.page_table[(size_t)b * a.maxp + lp] : 0;
      return (v < 0 || v >= a.num_pages) ? 0 : v;
    };
    int pg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) pg[i] = pt_entry(tid + kDecThreads * i);
    __syncthreads();  // the previous segment is done with the page window and the stages
#pragma unroll
    for (int i = 0; i < 2; ++i) sPT[tid + kDecThreads * i] = pg[i];
#pragma unroll
    for (int i = 2; i < kPTWindow / kDecThreads; ++i)
      sPT[tid + kDecThreads * i] = pt_entry(tid + kDecThreads * i);
    __syncthreads();  // page window written
    // wait for q here, before any tile load is in flight: the compiler cannot
    // count the tile loads, so a wait it placed for q inside the tile loop
    // would drain them (gfx9 encoding: vmcnt 0, others unlimited)
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // pool slot of key (lp0 is the window's first page)
    auto slot_of = [&](int key) __attribute__((always_inline)) {
      const int lp = key / a.ps;
      return sPT[min(lp - lp0, kPTWindow - 1)] * a.ps + (key - lp * a.ps);
    };
    // tile t (keys kt0 + 32 t ..) can be loaded in one piece when the page
    // holds the whole tile and every row of it is a context row
    auto one_piece = [&](int t) __attribute__((always_inline)) {
      return contiguous && kt0 + (t + 1) * kDecBN <= ctx_b;
    };
    // all loads of tile t into stage t % 4, in one burst
    auto issue = [&](int t) __attribute__((always_inline)) {
      const int kt = kt0 + t * kDecBN;
      const uint32_t base = lds0 + (t % kZStages) * kZStageB;
      if (one_piece(t)) {
        const void* sb = uniform_ptr_d(cache + (size_t)slot_of(kt) * kZRowB);
#pragma unroll
        for (int j = 0; j < kZLoadsPerWave; ++j)
          dma16_s_nb(sb, dma_off(j), base + (wave + kDecWaves * j) * 1024);
        asm volatile("" ::: "memory");
      } else {
        // pool slot of tile row (lane & 31); rows past the segment read its last
        // row (a context row whose page is inside the staged window). One load
        // at a time keeps this rarely taken path's registers few.
        const int slot = slot_of(min(kt + (lane & 31), k1 - 1));
#pragma unroll 1
        for (int p = wave; p < kZLoads; p += kDecWaves) {
          const int pch = p * 64 + lane;
          const int rr = pch / kZRowChunks;
          const int rs = __shfl(slot, rr, 64);
          dma16(cache + (size_t)rs * kZRowB + zchunk(rr, pch - rr * kZRowChunks) * 16,
                base + p * 1024);
        }
      }
    };

    f32x16 o[16];
#pragma unroll
    for (int md = 0; md < 16; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[md][i] = 0.f;
    float m_ref = -INFINITY;   // reference maximum (log2 domain): the first tile's
    float m_seen = -INFINITY;  // largest scaled score of the segment
    float l_run = 0.f;
    bool halted = false;       // wave-uniform: the partial is marked for recomputation

    // tile t's scores, then tile t-1's value product with tile t's softmax
    // interleaved between its MFMAs (the value MFMAs wait on LDS reads; the
    // softmax fills those gaps). The stages hold tiles t-1 (value product),
    // t (scores), t+1 and t+2 (loads in flight): the loads of tile t+2 go
    // out once the barrier of tile t shows every wave done with tile t-2.
    for (int t = 0; t < min(2, ntiles); ++t) issue(t);
    auto scores_t = [&](const uint8_t* Zs, const void* sbn, uint32_t nbase, auto with_dma)
        __attribute__((always_inline)) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      constexpr int kAhead = 4;
      bf16x8 zb[kAhead];
      auto zload = [&](int ks) __attribute__((always_inline)) {
        return *(const bf16x8*)(Zs + s_base[ks & 3] + 128 * (ks >> 2));
      };
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) zb[ks] = zload(ks);
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zb[ks % kAhead], qf[ks], acc, 0, 0, 0);
        if (ks + kAhead < kQSteps) zb[ks % kAhead] = zload(ks + kAhead);
        if constexpr (decltype(with_dma)::value) {
          if (ks % 4 == 0 && ks / 4 < kZLoadsPerWave)
            dma16_s_nb(sbn, dma_off(ks / 4), nbase + (wave + kDecWaves * (ks / 4)) * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return acc;
    };
    // O^T[512 dims x 32 heads] += Z^T P^T, transposed fragments four MFMAs
    // ahead in rotating registers; piece(i) runs after MFMA i
    auto value_product = [&](const uint8_t* Zv, const bf16x8* pb, auto piece)
        __attribute__((always_inline)) {
      constexpr int kAhead = 4;
      bf16x8 vb[kAhead];
      auto vload = [&](int i) __attribute__((always_inline)) {
        const int md = i >> 1, ks = i & 1;
        const bf16x4 a0 = ds_read_tr16(Zv + tr_base[0][md & 1] + 18432 * ks + 128 * (md >> 1));
        const bf16x4 a1 = ds_read_tr16(Zv + tr_base[1][md & 1] + 18432 * ks + 128 * (md >> 1));
        return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
#pragma unroll
      for (int i = 0; i < kAhead; ++i) vb[i] = vload(i);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        o[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % kAhead], pb[i & 1], o[i >> 1], 0, 0, 0);
        if (i + kAhead < 32) vb[i % kAhead] = vload(i + kAhead);
        piece(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // softmax of one tile's scores in pieces: 0, 1 the tile maximum, 2 the
    // reference, 4, 6, .., 18 two probabilities each, 20 the row sum
    float tmax = -INFINITY, neg_m = 0.f, psum = 0.f;
    uint32_t pw[8];
    auto softmax_piece = [&](const f32x16& sc, int i, bool first) __attribute__((always_inline)) {
      if (i == 0) {
        tmax = sc[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) tmax = fmaxf(tmax, sc[k]);
      } else if (i == 1) {
#pragma unroll
        for (int k = 8; k < 16; ++k) tmax = fmaxf(tmax, sc[k]);
      } else if (i == 2) {
        const float mt = max_with_lane32(tmax) * sl2;  // finite: every tile holds a valid key
        m_seen = fmaxf(m_seen, mt);
        if (first) m_ref = mt;  // the segment's first tile
        halted = halted || (__ballot(mt > m_ref + kDecSlack) != 0);
        neg_m = -m_ref;
        psum = 0.f;
      } else if (i >= 4 && i <= 18 && (i & 1) == 0) {
        const int j = (i - 4) >> 1;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[2 * j], sl2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[2 * j + 1], sl2, neg_m));
        psum += p0 + p1;
        pw[j] = pack_bf16x2(p0, p1);
      } else if (i == 20) {
        l_run += sum_with_lane32(psum);
      }
    };
    // the probabilities of the tile whose softmax ran last, as the B operand
    bf16x8 pprev[2];
    auto take_probs = [&]() __attribute__((always_inline)) {
      pprev[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      pprev[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
    };

    // wait for tile t, publish it, send tile t+2's loads, compute and mask
    // tile t's scores
    auto front = [&](int t) __attribute__((always_inline)) {
      // this wave's loads of tile t are done (those of tile t+1 may not be)
      if (t + 1 < ntiles) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      static_assert(kZLoadsPerWave == 9, "wait counts");
      // tile t is in place for every wave; every wave is done with tile
      // t-2, whose stage receives tile t+2
      __syncthreads();
      const bool spread = t + 2 < ntiles && one_piece(t + 2);
      const void* sbn = cache;
      if (spread) sbn = uniform_ptr_d(cache + (size_t)slot_of(kt0 + (t + 2) * kDecBN) * kZRowB);
      else if (t + 2 < ntiles) issue(t + 2);
      const uint32_t nbase = lds0 + ((t + 2) % 4) * kZStageB;
      const uint8_t* Z = sZ + (t % kZStages) * kZStageB;
      const int kt = kt0 + t * kDecBN;
      f32x16 s = spread ? scores_t(Z, sbn, nbase, std::integral_constant<bool, true>())
                        : scores_t(Z, sbn, nbase, std::integral_constant<bool, false>());
      // register i holds tile row 16*(i/8) + 8*hf + i%8
      if (kt < k0 || kt + kDecBN > k1) {
        const int lo = k0 - kt - hf * 8, hi = k1 - kt - hf * 8;  // valid: lo <= c < hi
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = (i >> 3) * 16 + (i & 7);
          if (c < lo || c >= hi) s[i] = -INFINITY;
        }
      }
      return s;
    };
    {
      const f32x16 s = front(0);
#pragma unroll
      for (int i = 0; i <= 20; ++i) softmax_piece(s, i, true);
      take_probs();
    }
    for (int t = 1; t < ntiles; ++t) {
      const f32x16 s = front(t);
      value_product(sZ + ((t - 1) % kZStages) * kZStageB, pprev,
                    [&](int i) __attribute__((always_inline)) { softmax_piece(s, i, false); });
      take_probs();
    }
    value_product(sZ + ((ntiles - 1) % kZStages) * kZStageB, pprev,
                  [&](int) __attribute__((always_inline)) {});
    // partial state of (w, b): slot w + b. The output is stored in bf16 by
    // groups of eight dims, [slot][dim / 8][head][dim % 8], so that every
    // store instruction writes 512 bytes in one piece (32 heads x 16 bytes).
    if (hvalid) {
      const size_t base = ((size_t)(w + b) * a.H + head);
      // O^T register i of block md: dim 32 md + 8 (i / 4) + 4 hf + i % 4
      uint16_t* op = a.part_o + ((size_t)(w + b) * (kLora / 8) * a.H + head) * 8 + hf * 4;
#pragma unroll
      for (int md = 0; md < 16; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v;
          v[0] = pack_bf16x2(o[md][g * 4 + 0], o[md][g * 4 + 1]);
          v[1] = pack_bf16x2(o[md][g * 4 + 2], o[md][g * 4 + 3]);
          *(u32x2*)(op + (size_t)(4 * md + g) * a.H * 8) = v;
        }
      if (hf == 0) {
        // a wave whose scores outgrew the reference hands (exact maximum, -1)
        // to the combine step, which recomputes this partial against it
        a.part_ml[base * 2 + 0] = halted ? m_seen : m_ref;
        a.part_ml[base * 2 + 1] = halted ? -1.0f : l_run;
      }
    }
    pos = seg_end;
    ++b;
  }
}


// ---------------------------------------------------------------------------
// 2'. split-KV attention over an e4m3 cache: both products on fp8 MFMA
// ---------------------------------------------------------------------------
// The same key ranges and partial states as the bf16 kernel; tiles of 64 keys
// (36 KB of e4m3 rows, as stored) and v_mfma_f32_32x32x64_f8f6f4 for both
// products, which runs at twice the rate of the bf16 instructions, so a byte
// of cache costs the same matrix time as in the bf16 kernel. Wave w owns heads
// 32 w .. 32 w + 31: per tile S^T = Z Q^T (2 key blocks x 9 depth steps of
// 64) and O^T += Z^T P^T (16 dim blocks, one 64-key step).
//  - q_abs is quantised per (sequence, head) to e4m3 when the segment starts:
//    q / 2^e with 2^e the power of two that puts the head's largest |q| in
//    (128, 256]; 2^e is folded into the score scale, so the scores are the
//    e4m3 products accumulated in fp32 and rescaled exactly.
//  - A lane's 32 fp8 values of an operand are depth (or key) 32 h + 0 .. 31 of
//    its step, h = lane / 32, in both operands; the instruction sums over k
//    in any order both operands share.
//  - Key rows go to the score MFMA in the order kappa64 (block mb, row r ->
//    key 32 ((r >> 2) & 1) + 16 mb + 4 (r >> 3) + (r & 3)), which makes a
//    lane's 32 scores the keys 32 h .. 32 h + 31, in the order the value
//    product's B operand (P^T) takes them.
//  - Z^T is read with ds_read_b64_tr_b8: in each 16-lane group, lane i gets
//    byte i % 8 of the 8 bytes that lanes i / 8, i / 8 + 2, .., i / 8 + 14
//    address, so four reads give a lane 32 keys of one dim.
//  - Probabilities are e4m3 as well: P = 2^(s - m + 7) against a reference
//    maximum m per head that is raised (and O and the row sum rescaled) when a
//    tile's maximum exceeds it by more than kF8Slack, so P stays below
//    2^(7 + kF8Slack) < 448 and a weight 2^-16 of the maximum's is still
//    represented.
//  - Rows keep their 16-byte chunks with the low two index bits XORed by
//    zf8swz(row) (bit 0: row bit 5, bit 1: row bit 2): the 16 lanes a score
//    read serves per cycle (rows with 4 values of row % 4, bits 2 and 5
//    varying) and the 32 lanes a transposed 8-byte read serves per cycle
//    (8 rows, two chunks, both 8-byte halves) land on distinct banks.
constexpr int kF8BN = 64;                              // keys per tile
constexpr int kF8TileB = kF8BN * kCache;               // 36864 bytes
constexpr int kF8TStages = 4;
constexpr int kF8TLoads = kF8TileB / 1024;             // 36 wave loads of 1 KB
constexpr int kF8TLoadsPerWave = kF8TLoads / kDecWaves;  // 9
constexpr int kF8RowChunks = kCache / 16;              // 36
constexpr int kF8DSteps = kCache / 64;                 // 9 score steps
constexpr float kF8Slack = 1.5f;
constexpr float kF8Bias = 7.0f;
static_assert(kF8TLoads % kDecWaves == 0, "even e4m3 loads per wave");
static_assert(kF8TStages * kF8TileB <= kZStages * kZStageB, "staging fits");

typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));
typedef int i32x2 __attribute__((__vector_size__(2 * sizeof(int))));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ int zf8swz(int row) { return ((row >> 5) & 1) | (((row >> 2) & 1) << 1); }
__device__ __forceinline__ int zf8chunk(int row, int chunk) { return (chunk & ~3) | ((chunk & 3) ^ zf8swz(row)); }

__device__ __forceinline__ u32x2 ds_read_tr8(const uint8_t* lds_byte_ptr) {
  const auto v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_byte_ptr));
  return __builtin_bit_cast(u32x2, v);
}

__global__ void __launch_bounds__(kDecThreads, 1) decode_split_f8_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sZ[kF8TStages * kF8TileB];
  __shared__ int sPT[kPTWindow];

  const int w = blockIdx.x;
  if (w >= a.G) return;
  const uint32_t s_lo = a.wstart[w];
  const uint32_t s_hi = a.wstart[w + 1];
  if (s_lo >= s_hi) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int head = wave * 32 + l32;
  const bool hvalid = head < a.H;
  const uint8_t* cache = (const uint8_t*)a.cache;
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)sZ);

  // ---- per-lane LDS read offsets (bytes inside a stage) ----
  // scores, block mb, step ks: row kappa64(mb, l32), chunks 4 ks + 2 hf and
  // 4 ks + 2 hf + 1 -> s_base[mb][0 or 1] + 64 ks
  int s_base[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = 32 * ((l32 >> 2) & 1) + 16 * mb + 4 * (l32 >> 3) + (l32 & 3);
#pragma unroll
    for (int c = 0; c < 2; ++c) s_base[mb][c] = row * kCache + zf8chunk(row, 2 * hf + c) * 16;
  }
  // transposed reads: dim block md, read q (keys 32 h + 8 q .. + 7), lane i
  // of group G = lane / 16 (h = G / 2): source row 32 h + 8 q + i / 2, chunk
  // 2 md + (G & 1), byte 8 (i & 1) -> tr_base[q][md & 1] + 64 (md >> 1)
  uint32_t tr_pk[4];
  {
    const int G = lane >> 4, i = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int m1 = 0; m1 < 2; ++m1) {
        const int row = 32 * (G >> 1) + 8 * q + (i >> 1);
        const uint32_t off = (uint32_t)(row * kCache + zf8chunk(row, 2 * m1 + (G & 1)) * 16 + 8 * (i & 1));
        const int idx = q * 2 + m1;
        if (idx & 1) tr_pk[idx >> 1] |= off << 16; else tr_pk[idx >> 1] = off;
      }
  }
  auto tr_off = [&](int q, int md) __attribute__((always_inline)) {
    const int idx = q * 2 + (md & 1);
    return (int)((tr_pk[idx >> 1] >> (16 * (idx & 1))) & 0xFFFFu) + 64 * (md >> 1);
  };
  // direct loads of a contiguous tile: load j of this wave (p = wave + 4 j)
  // fills LDS chunks 64 p + lane: tile row rr, source chunk zf8chunk(rr, cc)
  uint32_t dma_pk[(kF8TLoadsPerWave + 1) / 2];
#pragma unroll
  for (int j = 0; j < kF8TLoadsPerWave; ++j) {
    const int pch = (wave + kDecWaves * j) * 64 + lane;
    const int rr = pch / kF8RowChunks;
    const uint32_t off = (uint32_t)(rr * kCache + zf8chunk(rr, pch - rr * kF8RowChunks) * 16);
    if (j & 1) dma_pk[j >> 1] |= off << 16; else dma_pk[j >> 1] = off;
  }
  auto dma_off = [&](int j) __attribute__((always_inline)) {
    return (dma_pk[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
  };
  const bool contiguous = (a.ps % kF8BN) == 0;

  int b = a.wfirst[w];
  uint32_t pos = s_lo;
  while (pos < s_hi) {
    const uint32_t seg_end = min(s_hi, a.cum[b + 1]);
    if (seg_end <= pos) { ++b; continue; }
    const int k0 = (int)(pos - a.cum[b]);
    const int k1 = (int)(seg_end - a.cum[b]);
    const int kt0 = k0 & ~(kF8BN - 1);
    const int ntiles = (k1 - kt0 + kF8BN - 1) / kF8BN;
    const int ctx_b = (int)(a.cum[b + 1] - a.cum[b]);
    const int lp0 = kt0 / a.ps;
    const int npg = (k1 - 1) / a.ps - lp0 + 1;
    // this lane's half of its head's absorbed query: depth 64 ks + 32 hf + 0..31
    u32x4 qraw[kF8DSteps][4];
    {
      const uint16_t* qrow = a.q_abs + ((size_t)b * a.H + min(head, a.H - 1)) * kCache + hf * 32;
#pragma unroll
      for (int ks = 0; ks < kF8DSteps; ++ks)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          qraw[ks][c] = hvalid ? *(const u32x4*)(qrow + ks * 64 + c * 8) : u32x4{0, 0, 0, 0};
    }
    auto pt_entry = [&](int e) __attribute__((always_inline)) {
      const int lp = lp0 + e;
      const int v = (e < npg && lp < a.maxp) ? a.page_table[(size_t)b * a.maxp + lp] : 0;
      return (v < 0 || v >= a.num_pages) ? 0 : v;
    };
    int pg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) pg[i] = pt_entry(tid + kDecThreads * i);
    __syncthreads();  // the previous segment is done with the page window and the stages
#pragma unroll
    for (int i = 0; i < 2; ++i) sPT[tid + kDecThreads * i] = pg[i];
#pragma unroll
    for (int i = 2; i < kPTWindow / kDecThreads; ++i)
      sPT[tid + kDecThreads * i] = pt_entry(tid + kDecThreads * i);
    __syncthreads();  // page window written
    __builtin_amdgcn_s_waitcnt(0x0F70);  // q and the page table in registers (vmcnt 0)

    // quantise the head's query to e4m3 with a power-of-two scale 2^qe
    i32x8 qf[kF8DSteps];
    float sl2;  // scale * log2(e) * 2^qe: converts q8 . z8 to log2 units
    {
      float amax = 0.f;
#pragma unroll
      for (int ks = 0; ks < kF8DSteps; ++ks)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(qraw[ks][c][e])), fabsf(bf16_hi(qraw[ks][c][e]))));
      amax = max_with_lane32(amax);
      // amax * 2^-qe in (128, 256]; a zero query keeps qe = 0
      const int qe = amax > 0.f ? (int)ceilf(__builtin_amdgcn_logf(amax)) - 8 : 0;
      const float inv = __builtin_amdgcn_ldexpf(1.0f, -qe);
      sl2 = a.scale_log2 * __builtin_amdgcn_ldexpf(1.0f, qe);
#pragma unroll
      for (int ks = 0; ks < kF8DSteps; ++ks)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t w0 = 0, w1 = 0;
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(qraw[ks][c][0]) * inv, bf16_hi(qraw[ks][c][0]) * inv, w0, false);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(qraw[ks][c][1]) * inv, bf16_hi(qraw[ks][c][1]) * inv, w0, true);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(qraw[ks][c][2]) * inv, bf16_hi(qraw[ks][c][2]) * inv, w1, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(qraw[ks][c][3]) * inv, bf16_hi(qraw[ks][c][3]) * inv, w1, true);
          qf[ks][2 * c] = (int)w0;
          qf[ks][2 * c + 1] = (int)w1;
        }
    }

    auto slot_of = [&](int key) __attribute__((always_inline)) {
      const int lp = key / a.ps;
      return sPT[min(lp - lp0, kPTWindow - 1)] * a.ps + (key - lp * a.ps);
    };
    auto one_piece = [&](int t) __attribute__((always_inline)) {
      return contiguous && kt0 + (t + 1) * kF8BN <= ctx_b;
    };
    auto issue = [&](int t) __attribute__((always_inline)) {
      const int kt = kt0 + t * kF8BN;
      const uint32_t base = lds0 + (t % kF8TStages) * kF8TileB;
      if (one_piece(t)) {
        const void* sb = uniform_ptr_d(cache + (size_t)slot_of(kt) * kCache);
#pragma unroll
        for (int j = 0; j < kF8TLoadsPerWave; ++j)
          dma16_s_nb(sb, dma_off(j), base + (wave + kDecWaves * j) * 1024);
        asm volatile("" ::: "memory");
      } else {
        // pool slot of tile row `lane`; rows past the segment read its last row
        const int slot = slot_of(min(kt + lane, k1 - 1));
#pragma unroll 1
        for (int p = wave; p < kF8TLoads; p += kDecWaves) {
          const int pch = p * 64 + lane;
          const int rr = pch / kF8RowChunks;
          const int rs = __shfl(slot, rr, 64);
          dma16(cache + (size_t)rs * kCache + zf8chunk(rr, pch - rr * kF8RowChunks) * 16,
                base + p * 1024);
        }
      }
    };

    f32x16 o[16];
#pragma unroll
    for (int md = 0; md < 16; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[md][i] = 0.f;
    float m_ref = -INFINITY;  // reference maximum of this head (log2 domain)
    float l_run = 0.f;        // this lane's share of the row sum, in units of 2^(m_ref - 7)

    for (int t = 0; t < min(2, ntiles); ++t) issue(t);

    auto scores_t = [&](const uint8_t* Zs, const void* sbn, uint32_t nbase, auto with_dma)
        __attribute__((always_inline)) {
      std::array<f32x16, 2> acc;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
      constexpr int kAhead = 2;
      constexpr int kSteps = 2 * kF8DSteps;  // 18: (ks, mb) pairs
      i32x8 zb[kAhead];
      auto zload = [&](int i) __attribute__((always_inline)) {
        const int ks = i >> 1, mb = i & 1;
        const u32x4 lo = *(const u32x4*)(Zs + s_base[mb][0] + 64 * ks);
        const u32x4 hi = *(const u32x4*)(Zs + s_base[mb][1] + 64 * ks);
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int i = 0; i < kAhead; ++i) zb[i] = zload(i);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        acc[i & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(zb[i % kAhead], qf[i >> 1],
                                                                     acc[i & 1], 0, 0, 0, 0, 0, 0);
        if (i + kAhead < kSteps) zb[i % kAhead] = zload(i + kAhead);
        if constexpr (decltype(with_dma)::value) {
          if ((i & 1) == 0 && i / 2 < kF8TLoadsPerWave)
            dma16_s_nb(sbn, dma_off(i / 2), nbase + (wave + kDecWaves * (i / 2)) * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return acc;
    };
    // O^T[512 dims x 32 heads] += Z^T P^T, fragments two MFMAs ahead; piece(i)
    // runs after MFMA i
    auto value_product = [&](const uint8_t* Zv, const i32x8& pb, auto piece)
        __attribute__((always_inline)) {
      constexpr int kAhead = 2;
      i32x8 vb[kAhead];
      auto vload = [&](int md) __attribute__((always_inline)) {
        const u32x2 r0 = ds_read_tr8(Zv + tr_off(0, md));
        const u32x2 r1 = ds_read_tr8(Zv + tr_off(1, md));
        const u32x2 r2 = ds_read_tr8(Zv + tr_off(2, md));
        const u32x2 r3 = ds_read_tr8(Zv + tr_off(3, md));
        return i32x8{(int)r0[0], (int)r0[1], (int)r1[0], (int)r1[1],
                     (int)r2[0], (int)r2[1], (int)r3[0], (int)r3[1]};
      };
#pragma unroll
      for (int i = 0; i < kAhead; ++i) vb[i] = vload(i);
#pragma unroll
      for (int md = 0; md < 16; ++md) {
        o[md] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb[md % kAhead], pb, o[md], 0, 0,
                                                                0, 0, 0, 0);
        if (md + kAhead < 16) vb[md % kAhead] = vload(md + kAhead);
        piece(md);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // softmax pieces of one tile: 0, 1 the tile maximum; 2 the head's maximum
    // and the growth test; 4, 5, .., 11 four probabilities each
    float tmax = -INFINITY, mt = -INFINITY, neg_m = 0.f, psum = 0.f;
    bool grow = false;
    uint32_t pw[8];
    auto prob4 = [&](const std::array<f32x16, 2>& sc, int j) __attribute__((always_inline)) {
      // bytes 4 j .. 4 j + 3 of the lane's 32: block j / 4, registers 4 (j % 4) ..
      const f32x16& v = sc[j >> 2];
      const int r = 4 * (j & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(v[r], sl2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(v[r + 1], sl2, neg_m));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(v[r + 2], sl2, neg_m));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(v[r + 3], sl2, neg_m));
      uint32_t x = 0;
      x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, x, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
      pw[j] = x;
      psum += (p0 + p1) + (p2 + p3);
    };
    auto softmax_piece = [&](const std::array<f32x16, 2>& sc, int i, bool first)
        __attribute__((always_inline)) {
      if (i == 0) {
        tmax = sc[0][0];
#pragma unroll
        for (int k = 1; k < 16; ++k) tmax = fmaxf(tmax, sc[0][k]);
      } else if (i == 1) {
#pragma unroll
        for (int k = 0; k < 16; ++k) tmax = fmaxf(tmax, sc[1][k]);
      } else if (i == 2) {
        mt = max_with_lane32(tmax * sl2);  // the head's tile maximum; -inf if all masked
        if (first) m_ref = mt;             // finite: the first tile holds a valid key
        grow = __ballot(mt > m_ref + kF8Slack) != 0;
        neg_m = kF8Bias - m_ref;
        psum = 0.f;
      } else if (i >= 4 && i < 12) {
        if (!grow) prob4(sc, i - 4);
      }
    };
    // after the value product that used the previous reference: raise the
    // reference to the tile maximum where it grew, rescale, recompute P
    auto settle = [&](const std::array<f32x16, 2>& sc) __attribute__((always_inline)) {
      if (grow) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
        // in place in the accumulation registers, one value at a time (the
        // compiler would otherwise move the 256 accumulators through vector
        // registers and spill)
#pragma unroll
        for (int md = 0; md < 16; ++md)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(o[md][i]), "=&v"(tmp)
                : "v"(alpha));
          }
        m_ref = m_new;
        neg_m = kF8Bias - m_ref;
        psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) prob4(sc, j);
        grow = false;
      }
      l_run += psum;
    };
    i32x8 pprev;
    auto take_probs = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pprev[j] = (int)pw[j];
    };

    auto front = [&](int t) __attribute__((always_inline)) {
      if (t + 1 < ntiles) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      static_assert(kF8TLoadsPerWave == 9, "wait counts");
      // the packed offsets stay packed (unpacked per use, not kept unpacked
      // across the loop, where they would not fit the registers)
#pragma unroll
      for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(tr_pk[k]));
#pragma unroll
      for (int k = 0; k < (kF8TLoadsPerWave + 1) / 2; ++k) asm volatile("" : "+v"(dma_pk[k]));
      __syncthreads();
      const bool spread = t + 2 < ntiles && one_piece(t + 2);
      const void* sbn = cache;
      if (spread) sbn = uniform_ptr_d(cache + (size_t)slot_of(kt0 + (t + 2) * kF8BN) * kCache);
      else if (t + 2 < ntiles) issue(t + 2);
      const uint32_t nbase = lds0 + ((t + 2) % kF8TStages) * kF8TileB;
      const uint8_t* Z = sZ + (t % kF8TStages) * kF8TileB;
      const int kt = kt0 + t * kF8BN;
      std::array<f32x16, 2> s = spread ? scores_t(Z, sbn, nbase, std::integral_constant<bool, true>())
                                       : scores_t(Z, sbn, nbase, std::integral_constant<bool, false>());
      // register i of block mb holds key kt + 32 hf + 16 mb + i
      if (kt < k0 || kt + kF8BN > k1) {
        const int lo = k0 - kt - 32 * hf, hi = k1 - kt - 32 * hf;  // valid: lo <= c < hi
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = 16 * mb + i;
            if (c < lo || c >= hi) s[mb][i] = -INFINITY;
          }
      }
      return s;
    };
    {
      const std::array<f32x16, 2> s = front(0);
#pragma unroll
      for (int i = 0; i < 12; ++i) softmax_piece(s, i, true);
      settle(s);
      take_probs();
    }
    for (int t = 1; t < ntiles; ++t) {
      const std::array<f32x16, 2> s = front(t);
      value_product(sZ + ((t - 1) % kF8TStages) * kF8TileB, pprev,
                    [&](int i) __attribute__((always_inline)) { softmax_piece(s, i, false); });
      settle(s);
      take_probs();
    }
    value_product(sZ + ((ntiles - 1) % kF8TStages) * kF8TileB, pprev,
                  [&](int) __attribute__((always_inline)) {});
    l_run = sum_with_lane32(l_run);
    if (hvalid) {
      const size_t base = ((size_t)(w + b) * a.H + head);
      // O^T register i of block md: dim 32 md + 8 (i / 4) + 4 hf + i % 4
      uint16_t* op = a.part_o + ((size_t)(w + b) * (kLora / 8) * a.H + head) * 8 + hf * 4;
#pragma unroll
      for (int md = 0; md < 16; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v;
          v[0] = pack_bf16x2(o[md][g * 4 + 0], o[md][g * 4 + 1]);
          v[1] = pack_bf16x2(o[md][g * 4 + 2], o[md][g * 4 + 3]);
          *(u32x2*)(op + (size_t)(4 * md + g) * a.H * 8) = v;
        }
      if (hf == 0) {
        a.part_ml[base * 2 + 0] = m_ref - kF8Bias;
        a.part_ml[base * 2 + 1] = l_run;
      }
    }
    pos = seg_end;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// 3. combine the partial states: o_lat[b, h, :] (bf16 hi + lo)
// ---------------------------------------------------------------------------
// One wave per (sequence, head), lane l owns dims 8 l .. 8 l + 7: the maximum
// over the partials first, then their weighted sum. Thousands of independent
// waves keep many loads in flight. o_lat is written as a bf16 pair (hi, lo)
// so that the projection, on bf16 MFMA, sees it unrounded to 8 bits.

// Recompute, in one wave, the partial of (range w, sequence b, head h) against
// the exact maximum m (log2 domain) the split kernel recorded: plain fp32,
// one key per lane for the scores. Returns the lane's 8 dims and the sum.
// Only reached for extreme score ranges.
__device__ void recompute_partial(const CombineArgs& c, int w, int b, int h, float m,
                                  float (&acc)[8], float& lsum) {
  const int lane = threadIdx.x & 63;
  const uint32_t lo = max(c.wstart[w], c.cum[b]);
  const uint32_t hi = min(c.wstart[w + 1], c.cum[b + 1]);
  const int k0 = (int)(lo - c.cum[b]), k1 = (int)(hi - c.cum[b]);
  const uint16_t* qa = c.q_abs + ((size_t)b * c.H + h) * kCache;
  const size_t esz = c.fp8 ? 1 : 2;
  auto row_of = [&](int key) -> const uint8_t* {
    const int lp = key / c.ps;
    int pg = lp < c.maxp ? c.page_table[(size_t)b * c.maxp + lp] : 0;
    if (pg < 0 || pg >= c.num_pages) pg = 0;
    return (const uint8_t*)c.cache + ((size_t)pg * c.ps + (key - lp * c.ps)) * kCache * esz;
  };
  auto elem = [&](const uint8_t* z, int e) -> float {
    return c.fp8 ? e4m3_to_f32(z[e]) : bf16_to_f32(((const uint16_t*)z)[e]);
  };
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  lsum = 0.f;
  for (int kc = k0; kc < k1; kc += 64) {
    const int key = kc + lane;
    float p = 0.f;
    if (key < k1) {
      const uint8_t* z = row_of(key);
      float sc = 0.f;
      for (int e = 0; e < kCache; ++e) sc = fmaf(bf16_to_f32(qa[e]), elem(z, e), sc);
      p = __builtin_amdgcn_exp2f(sc * c.scale_log2 - m);
    }
    const int n = min(64, k1 - kc);
    for (int k = 0; k < n; ++k) {
      const float pk = __shfl(p, k, 64);
      const uint8_t* z = row_of(kc + k);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(pk, elem(z, 8 * lane + j), acc[j]);
      lsum += pk;
    }
  }
}

// One wave merges all 512 dims of (sequence b, head h), recomputing marked
// partials: the path taken when any partial of the workgroup's heads is marked.
__device__ void combine_head(const CombineArgs& c, int b, int h, int lane) {
  if (h >= c.H) return;
  const int2 span = c.wspan[b];
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if (span.y >= span.x) {
    // the maximum over the partials: lanes stride over the ranges
    float M = -INFINITY;
    for (int w0 = span.x; w0 <= span.y; w0 += 64) {
      const int w = w0 + lane;
      if (w <= span.y && c.wstart[w] < c.wstart[w + 1])  // empty range: no partial
        M = fmaxf(M, c.part_ml[((size_t)(w + b) * c.H + h) * 2]);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
    // the weighted sum, four ranges' states and outputs loaded together
    float L = 0.f;
    for (int w0 = span.x; w0 <= span.y; w0 += 4) {
      bool ok[4];
      float m[4], l[4];
      f32x4 v0[4], v1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = w0 + j;
        ok[j] = w <= span.y && c.wstart[w] < c.wstart[w + 1];
        const size_t base = (size_t)(w + b) * c.H + h;
        const uint16_t* po = c.part_o + (((size_t)(w + b) * (kLora / 8) + lane) * c.H + h) * 8;
        if (ok[j]) {
          m[j] = c.part_ml[base * 2];
          l[j] = c.part_ml[base * 2 + 1];
          const u32x4 pv = *(const u32x4*)(po);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            v0[j][2 * e] = bf16_lo(pv[e]);
            v0[j][2 * e + 1] = bf16_hi(pv[e]);
            v1[j][2 * e] = bf16_lo(pv[2 + e]);
            v1[j][2 * e + 1] = bf16_hi(pv[2 + e]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!ok[j]) continue;
        float ow[8];
        float lj = l[j];
        if (lj < 0.f) {  // marked partial: recompute (wave-uniform)
          recompute_partial(c, w0 + j, b, h, m[j], ow, lj);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) { ow[e] = v0[j][e]; ow[4 + e] = v1[j][e]; }
        }
        const float wt = __builtin_amdgcn_exp2f(m[j] - M);
        L += wt * lj;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wt, ow[e], acc[e]);
      }
    }
    // a sink adds e^sink to the denominator (L and acc are relative to 2^M)
    if (c.sink) L += __builtin_amdgcn_exp2f(c.sink[b] * 1.44269504088896341f - M);
    const float inv = 1.f / L;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv;
  }
  u32x4 hi, lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
    lo[j] = pack_bf16x2(acc[2 * j] - bf16_lo(hi[j]), acc[2 * j + 1] - bf16_hi(hi[j]));
  }
  uint16_t* orow = c.o_lat + ((size_t)b * c.H + h) * (2 * kLora);
  *(u32x4*)(orow + 8 * lane) = hi;
  *(u32x4*)(orow + kLora + 8 * lane) = lo;
}

// Grid (B, ceil(H / 32), 4): a workgroup merges the partials of sequence b
// for 32 heads and a quarter of the 512 dims. The partial outputs are stored
// in bf16 [slot][dim / 8][head][dim % 8], so lane (head = lane / 2, half =
// lane % 2) of a wave reading one group of eight dims for 32 heads reads
// 512 bytes in one piece. First the per-head maximum over the partials (eight range lanes per
// head, reduced through LDS); if any partial of these heads is marked, the
// workgroup of quarter 0 merges them one head per wave with recomputation.
__global__ void __launch_bounds__(256) decode_combine_kernel(CombineArgs c) {
  __shared__ float s_m[8][32];
  const int b = blockIdx.x;
  const int hb = blockIdx.y * 32;
  const int gq = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int2 span = c.wspan[b];
  {
    const int hh = tid & 31, wi = tid >> 5;
    const int h1 = hb + hh;
    float M = -INFINITY;
    bool marked = false;
    if (h1 < c.H) {
      for (int w = span.x + wi; w <= span.y; w += 8) {
        if (c.wstart[w] < c.wstart[w + 1]) {  // empty range: no partial
          const float* ml = c.part_ml + ((size_t)(w + b) * c.H + h1) * 2;
          M = fmaxf(M, ml[0]);
          marked = marked || ml[1] < 0.f;
        }
      }
    }
    s_m[wi][hh] = M;
    if (__syncthreads_or(marked)) {
      if (gq == 0)
        for (int k = wave; k < 32; k += 4) combine_head(c, b, hb + k, lane);
      return;
    }
  }
  const int hl = lane >> 1, half = lane & 1;
  const int head = hb + hl;
  if (head >= c.H) return;
  float Mh = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) Mh = fmaxf(Mh, s_m[j][hl]);
  const int g0 = gq * 16 + wave * 4;  // this wave's four groups of eight dims
  float acc[4][4];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[gg][e] = 0.f;
  if (span.y >= span.x) {
    float L = 0.f;
    // eight ranges per round, every load of a round issued before any use (a
    // sequence spans a handful of ranges, so most take one round)
    constexpr int kBatch = 8;
    for (int w0 = span.x; w0 <= span.y; w0 += kBatch) {
      float m[kBatch], l[kBatch];
      u32x2 pv[kBatch][4];
      bool ok[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int w = w0 + j;
        // empty range: no partial (weight 0)
        ok[j] = w <= span.y && c.wstart[w] < c.wstart[w + 1];
        const size_t slot = (size_t)(w + b);
        m[j] = 0.f;
        l[j] = 0.f;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) pv[j][gg] = u32x2{0u, 0u};
        if (ok[j]) {
          const float* ml = c.part_ml + (slot * c.H + head) * 2;
          m[j] = ml[0];
          l[j] = ml[1];
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            pv[j][gg] = *(const u32x2*)(c.part_o + ((slot * (kLora / 8) + g0 + gg) * c.H + head) * 8 +
                                        half * 4);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float wt = ok[j] ? __builtin_amdgcn_exp2f(m[j] - Mh) : 0.f;
        L += wt * l[j];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          acc[gg][0] = fmaf(wt, bf16_lo(pv[j][gg][0]), acc[gg][0]);
          acc[gg][1] = fmaf(wt, bf16_hi(pv[j][gg][0]), acc[gg][1]);
          acc[gg][2] = fmaf(wt, bf16_lo(pv[j][gg][1]), acc[gg][2]);
          acc[gg][3] = fmaf(wt, bf16_hi(pv[j][gg][1]), acc[gg][3]);
        }
      }
    }
    // a sink adds e^sink to the denominator (L and acc are relative to 2^Mh)
    if (c.sink) L += __builtin_amdgcn_exp2f(c.sink[b] * 1.44269504088896341f - Mh);
    const float inv = 1.f / L;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[gg][e] *= inv;
  }
  uint16_t* orow = c.o_lat + ((size_t)b * c.H + head) * (2 * kLora);
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    u32x2 hi, lo;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      hi[j] = pack_bf16x2(acc[gg][2 * j], acc[gg][2 * j + 1]);
      lo[j] = pack_bf16x2(acc[gg][2 * j] - bf16_lo(hi[j]), acc[gg][2 * j + 1] - bf16_hi(hi[j]));
    }
    const int d = (g0 + gg) * 8 + half * 4;
    *(u32x2*)(orow + d) = hi;
    *(u32x2*)(orow + kLora + d) = lo;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode_absorb(uint16_t* q_abs, const uint16_t* q, const uint16_t* w_uk, int B,
                                int H, const PrefixArgs& pa, hipStream_t stream) {
  const dim3 grid(H + 1, (B + 63) / 64);
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(256), 0, stream, q_abs, q, w_uk, B, H, pa);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL(decode_split_f8_kernel, dim3(a.G), dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_split_kernel, dim3(a.G), dim3(kDecThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const CombineArgs& c, hipStream_t stream) {
  const dim3 grid(c.B, (c.H + 31) / 32, 4);
  hipLaunchKernelGGL(decode_combine_kernel, grid, dim3(256), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_decode_project(uint16_t* out, const uint16_t* o_lat, const uint16_t* w_uv,
                                 int B, int H, hipStream_t stream) {
  // out[b, h, d] = sum_l o_lat[b, h, l] w_uv[h, d, l]: K = 512, N = 128; o_lat
  // rows hold hi then lo (2 x 512 bf16)
  const int ntn = kV / 32;
  const int tiles = ((B + 31) / 32) * ntn;
  const dim3 grid((tiles + 3) / 4, H);
  hipLaunchKernelGGL((head_gemm_kernel<kLora, true>), grid, dim3(256), 0, stream, out,
                     o_lat, w_uv, B, kV, (long)H * 2 * kLora, (long)2 * kLora,
                     (long)kV * kLora, (long)H * kV, (long)kV, ntn);
  return hipGetLastError();
}

}  // namespace mla
