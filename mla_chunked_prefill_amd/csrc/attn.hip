// Causal MLA prefill attention over one chunk of up-projected keys/values
// ("flare_mla_prefill_dispatch" page: q_depth 192 = 128 nope + 64 rope,
// kv_num_heads 1 for the rope part, v_depth 128, cache_offsets shifting the
// causal diagonal; bf16 or float8_e4m3fn inputs, bf16 output).
//
// Work decomposition. A workgroup (4 waves, 256 threads) owns one block of 128
// queries of one sequence and one head; each wave owns 32 of the queries.
// Keys are streamed in tiles of 64 rows aligned to the chunk buffer's 64-row
// grid; rows that belong to other sequences are masked.
//
// Tile movement. Every tile (K_nope, the shared k_rope rows and the value
// tile V^T) goes from global memory straight into LDS with 16-byte direct
// loads (global_load_lds_dwordx4): each lane's source offset inside a tile is
// fixed for the whole kernel, only the scalar tile base changes, so a tile
// costs ten load instructions per wave and no vector ALU work. Two LDS stages
// alternate: while a wave computes on tile t, the loads of tile t+1 fill the
// other stage, and one barrier per tile separates the two uses of a stage.
// Within a stage every row's 16-byte chunks are XOR-permuted by a function of
// the row so that the operand reads below hit distinct LDS banks.
//
// MFMA orientation. Scores are computed transposed, S^T = K Q^T, on
// mfma 32x32x16: rows are keys, columns are queries, so each lane owns one
// query column and 16 keys per 32-key block. Row statistics of the softmax are
// then in-lane reductions plus one exchange with the lane 32 away. The rows of
// K are fed to the MFMA in a permuted order (bits 2 and 3 of the row index
// swapped) so that every lane's 16 accumulator registers hold 2 x 8
// consecutive keys: converted to bf16 they are directly the B operand of the
// value product O^T += V^T P^T, whose A operand reads 8 consecutive keys of the
// transposed value tile from LDS with one 16-byte load.
//
// The k_rope tile (one head shared by all query heads) is read next to K_nope,
// so the 192-deep score reduction is 12 MFMA steps of 16.
//
// Softmax runs online in the log2 domain (scale * log2(e) folded into one
// multiply). Its state (max, sum, unnormalised output) is carried across the
// chunks of a sequence through the workspace; a query's output is written in
// the chunk that holds its last visible key.
#include <type_traits>

#include "kernels.hpp"

namespace mla {

constexpr int kAttnBM = 128;  // queries per workgroup
constexpr int kAttnBN = 64;   // keys per tile
constexpr int kAttnAhead = 4; // LDS operands read this many MFMAs ahead

typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));  // 32 e4m3 values

// Rescale the output accumulator only when a query's running maximum grows by
// more than this many (log2) units; in between, probabilities are formed
// against the stale maximum and stay below 2^8, exact in fp32 and bf16 range.
constexpr float kRescaleSlack = 8.0f;

// LDS layout of one stage: K_nope rows, k_rope rows, then V^T (128 dims x 64
// keys). Row sizes in bytes; every region is a whole number of 4 KB (one 1 KB
// direct load per wave).
template <bool kFp8>
struct AttnStage {
  static constexpr int kNopeRowB = kFp8 ? kNope : 2 * kNope;  // 128 / 256
  static constexpr int kRopeRowB = kFp8 ? kRope : 2 * kRope;  // 64 / 128
  static constexpr int kVRowB = 2 * kAttnBN;                  // 128
  static constexpr int kNopeB = kAttnBN * kNopeRowB;
  static constexpr int kRopeB = kAttnBN * kRopeRowB;
  static constexpr int kVB = kV * kVRowB;
  static constexpr int kRopeOff = kNopeB;
  static constexpr int kVOff = kNopeB + kRopeB;
  static constexpr int kBytes = kNopeB + kRopeB + kVB;
  static constexpr int kNopeLoads = kNopeB / 4096;  // per wave
  static constexpr int kRopeLoads = kRopeB / 4096;
  static constexpr int kVLoads = kVB / 4096;
  static constexpr int kLoads = kNopeLoads + kRopeLoads + kVLoads;
};

// Chunk permutations (XOR on the low chunk-index bits, so a row's chunks stay
// in the row). With rows fed in the order kappa(lane) the score reads of any
// 8 or 16 consecutive lanes touch distinct 16-byte bank groups of a 128- or
// 256-byte LDS line, and so do the value reads (rows in lane order).
__device__ __forceinline__ int swz3(int r) { return ((r & 3) | ((r >> 1) & 4)) ^ ((r >> 2) & 1); }
__device__ __forceinline__ int swz4(int r) { return swz3(r) | ((r << 1) & 8); }
__device__ __forceinline__ int swzv(int d) { return (d & 7) ^ ((d >> 3) & 1); }
template <int kChunks>
__device__ __forceinline__ int swz_rows(int r) {
  return kChunks >= 16 ? swz4(r) : (kChunks == 8 ? swz3(r) : (swz3(r) & 3));
}
// e4m3 rows (K_nope 128 bytes = 8 chunks, k_rope 64 bytes = 4 chunks), read
// 32 bytes per lane by the fp8 score MFMA: the 16 rows a read serves at once
// land on distinct 16-byte bank groups
template <int kChunks>
__device__ __forceinline__ int swz_rows_f8(int r) {
  return kChunks == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes, read from
// sbase + voff, land at LDS byte address lds + 16 l (lds and sbase are
// wave-uniform). Inline assembly keeps the compiler from treating later LDS
// reads as dependent on it (it would wait for every load in flight); the
// kernel orders these loads itself with s_waitcnt vmcnt and barriers. The asm
// sets m0 on every call; the kernels keep no value of their own in m0.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Per-lane source offset (bytes, inside a tile) of direct load `i` of a region
// whose LDS rows hold kChunks 16-byte chunks and whose global rows are
// `gstride` bytes apart (kValue: the value tile's permutation).
template <int kChunks, bool kValue = false, bool kF8 = false>
__device__ __forceinline__ uint32_t dma_src(int i, int lane, uint32_t gstride) {
  const int p = i * 64 + lane;
  const int r = p / kChunks;
  const int j = (p % kChunks) ^ (kValue ? swzv(r) : (kF8 ? swz_rows_f8<kChunks>(r) : swz_rows<kChunks>(r)));
  return (uint32_t)r * gstride + (uint32_t)j * 16u;
}

template <bool kFp8>
__global__ void __launch_bounds__(256, 2) prefill_attn_kernel(AttnArgs a) {
  using L = AttnStage<kFp8>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * L::kBytes];

  // XCD-aware order: consecutive workgroups of one XCD share a head.
  const int total = a.n_slots * a.H;
  const int per_xcd = gridDim.x >> 3;
  const int rem = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (rem >= total) return;
  const int h = rem / a.n_slots;
  const int slot = rem - h * a.n_slots;
  const int2 e = a.sched[slot];
  if (e.x < 0) return;
  const int nrows = *a.bl_c;
  if (nrows <= 0) return;
  const int b = e.x;
  const int qblk = e.y;
  const uint32_t t0 = a.offs[b];
  const int n_b = (int)(a.offs[b + 1] - t0);
  // rows and positions fit in 31 bits (the host bounds every size below 2^31)
  const int c_b = (int)a.clen[b];
  const int r0 = (int)a.bro_c[b];
  const int len = (int)a.bro_c[b + 1] - r0;
  const int co = (int)a.co_c[b];
  const int q_lo = qblk * kAttnBM;
  const int q_hi = min(q_lo + kAttnBM, n_b);
  if (len <= 0 || q_lo >= n_b) return;
  const int P_hi = c_b + q_hi - 1;
  if (co > P_hi) return;
  const int kv_end = min(len, P_hi - co + 1);  // keys j < kv_end can be visible

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int qi = q_lo + wave * 32 + l32;
  const bool qvalid = qi < n_b;
  const int P = c_b + qi;
  const bool active = qvalid && P >= co;
  const size_t t = (size_t)t0 + qi;
  // visible buffer rows of this query: [r0, r_hi]
  const int r_hi = active ? r0 + min(len - 1, P - co) : r0 - 1;
  // wave-uniform bounds: rows every valid query of the wave sees, and rows any sees
  const int wq_lo = q_lo + wave * 32;
  const int wq_hi = min(wq_lo + 32, n_b);  // exclusive
  const bool wave_active = wq_lo < n_b && c_b + wq_hi - 1 >= co;
  const int w_all_hi = r0 + min(len - 1, c_b + wq_lo - co);     // may be < r0
  const int w_any_hi = r0 + min(len - 1, c_b + wq_hi - 1 - co);

  // Q fragments: B operand of S^T = K Q^T (lane: query l32; bf16: depth
  // 16 ks + 8 hf .. + 7; e4m3: depth 64 ks + 32 hf .. + 31 for the fp8 MFMA)
  bf16x8 qf[12];
  i32x8 qf8[3];
  if (kFp8) {
    const uint8_t* qp = (const uint8_t*)a.q + (t * a.H + h) * kQDepth + hf * 32;
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const u32x4 lo = qvalid ? *(const u32x4*)(qp + ks * 64) : u32x4{0, 0, 0, 0};
      const u32x4 hi = qvalid ? *(const u32x4*)(qp + ks * 64 + 16) : u32x4{0, 0, 0, 0};
      qf8[ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  } else {
    const uint16_t* qp = (const uint16_t*)a.q + (t * a.H + h) * kQDepth + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      u32x4 v = qvalid ? *(const u32x4*)(qp + ks * 16) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[4];
  float m_run = -INFINITY;  // reference maximum (log2 domain, scaled)
  float l_run = 0.f;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[md][i] = 0.f;
  if (active && co > 0) {
    const float* cp = a.carry_o + (t * a.H + h) * kV;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = *(const f32x4*)(cp + md * 32 + g * 8 + hf * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[md][g * 4 + j] = v[j];
      }
    m_run = a.carry_ml[(t * a.H + h) * 2 + 0];
    l_run = a.carry_ml[(t * a.H + h) * 2 + 1];
  }

  // ---- per-lane LDS read offsets (bytes inside a stage) ----
  // permuted K row fed by this lane: bits 2 and 3 of l32 swapped
  const int kappa = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  constexpr int kNopeC = L::kNopeRowB / 16;
  constexpr int kRopeC = L::kRopeRowB / 16;
  // bf16: nb[ks] / rb[ks] read 16 bytes of step ks; e4m3: nb[2 ks + c] /
  // rb[c] read chunk 4 ks + 2 hf + c (nope) or 2 hf + c (rope) of row kappa
  int nb[8], rb[4], vb[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (kFp8)
      nb[kk] = kappa * L::kNopeRowB +
               (((4 * (kk >> 1) + 2 * hf + (kk & 1)) ^ swz_rows_f8<kNopeC>(kappa)) * 16);
    else nb[kk] = kappa * L::kNopeRowB + (((2 * kk + hf) ^ swz_rows<kNopeC>(kappa)) * 16);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kFp8)
      rb[kk] = L::kRopeOff + kappa * L::kRopeRowB +
               (((2 * hf + (kk & 1)) ^ swz_rows_f8<kRopeC>(kappa)) * 16);
    else
      rb[kk] = L::kRopeOff + kappa * L::kRopeRowB + (((2 * kk + hf) ^ swz_rows<kRopeC>(kappa)) * 16);
    vb[kk] = L::kVOff + l32 * L::kVRowB + (((2 * kk + hf) ^ swzv(l32)) * 16);
  }

  // ---- per-lane direct-load source offsets (bytes inside a tile) ----
  uint32_t src_n[L::kNopeLoads], src_r[L::kRopeLoads], src_v[L::kVLoads];
#pragma unroll
  for (int k = 0; k < L::kNopeLoads; ++k)
    src_n[k] = dma_src<kNopeC, false, kFp8>(wave + 4 * k, lane, L::kNopeRowB);
#pragma unroll
  for (int k = 0; k < L::kRopeLoads; ++k)
    src_r[k] = dma_src<kRopeC, false, kFp8>(wave + 4 * k, lane, L::kRopeRowB);
#pragma unroll
  for (int k = 0; k < L::kVLoads; ++k)
    src_v[k] = dma_src<8, true>(wave + 4 * k, lane, (uint32_t)a.max_rows * 2u);

  const uint8_t* kn_head = (const uint8_t*)a.k_nope + (size_t)h * a.max_rows * L::kNopeRowB;
  const uint8_t* kr_base = (const uint8_t*)a.krope;
  const uint8_t* v_head = (const uint8_t*)a.v_t + (size_t)h * kV * a.max_rows * 2;
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)smem);

  auto issue = [&](int tb, int stage) {
    const uint32_t base = lds0 + stage * L::kBytes;
    const void* sn = uniform_ptr(kn_head + (size_t)tb * L::kNopeRowB);
    const void* sr = uniform_ptr(kr_base + (size_t)tb * L::kRopeRowB);
    const void* sv = uniform_ptr(v_head + (size_t)tb * 2);
#pragma unroll
    for (int k = 0; k < L::kNopeLoads; ++k)
      dma16(sn, src_n[k], base + (wave + 4 * k) * 1024);
#pragma unroll
    for (int k = 0; k < L::kRopeLoads; ++k)
      dma16(sr, src_r[k], base + L::kRopeOff + (wave + 4 * k) * 1024);
#pragma unroll
    for (int k = 0; k < L::kVLoads; ++k)
      dma16(sv, src_v[k], base + L::kVOff + (wave + 4 * k) * 1024);
  };

  const float sl2 = a.scale_log2;
  const int tile_begin = r0 & ~(kAttnBN - 1);
  // never past the buffer, even if a caller's max_rows is smaller than the chunk
  const int tile_end = min(r0 + kv_end, a.max_rows);
  const int n_tiles = tile_end > tile_begin ? (tile_end - tile_begin + kAttnBN - 1) / kAttnBN : 0;

  auto body = [&](auto stage_c, int tt) {
    constexpr int S = decltype(stage_c)::value;
    const int tb = tile_begin + tt * kAttnBN;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile tt landed for every wave; the other stage is free
    if (tt + 1 < n_tiles) issue(tb + kAttnBN, S ^ 1);
    if (!wave_active || tb > w_any_hi) return;
    const uint8_t* st = smem + S * L::kBytes;

    // ---- S^T = K Q^T for 64 keys x 32 queries ----
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
    if (kFp8) {
      // three 64-deep steps (nope 0..63, nope 64..127, rope) on
      // v_mfma_f32_32x32x64_f8f6f4, twice the rate of the 16-deep fp8 form
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int o0 = ks < 2 ? nb[2 * ks] + mb * 32 * L::kNopeRowB : rb[0] + mb * 32 * L::kRopeRowB;
          const int o1 = ks < 2 ? nb[2 * ks + 1] + mb * 32 * L::kNopeRowB : rb[1] + mb * 32 * L::kRopeRowB;
          const u32x4 lo = *(const u32x4*)(st + o0);
          const u32x4 hi = *(const u32x4*)(st + o1);
          const i32x8 ka = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          s[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qf8[ks], s[mb], 0, 0, 0, 0, 0, 0);
        }
      }
    } else {
      // fragment i = 2 ks + mb, read kAttnAhead fragments ahead into rotating
      // registers; the fences keep each read that far ahead of its MFMA
      auto kload = [&](int i) __attribute__((always_inline)) {
        const int ks = i >> 1, mb = i & 1;
        const int off = ks < 8 ? nb[ks] + mb * 32 * L::kNopeRowB
                               : rb[ks - 8] + mb * 32 * L::kRopeRowB;
        return *(const bf16x8*)(st + off);
      };
      bf16x8 kf[kAttnAhead];
#pragma unroll
      for (int i = 0; i < kAttnAhead; ++i) kf[i] = kload(i);
#pragma unroll
      for (int i = 0; i < 24; ++i) {
        s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % kAttnAhead], qf[i >> 1], s[i & 1], 0, 0, 0);
        if (i + kAttnAhead < 24) kf[i % kAttnAhead] = kload(i + kAttnAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- online softmax (log2 domain), lazily rescaled ----
    // register i of block mb holds the key at tile row 32*mb + 16*(i/8) + 8*hf + i%8
    if (tb < r0 || tb + kAttnBN - 1 > w_all_hi) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = tb + mb * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
          if (kr < r0 || kr > r_hi) s[mb][i] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
    tmax = max_with_lane32(tmax);
    const float mt = tmax * sl2;
    const bool grow = mt > m_run + kRescaleSlack;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[md][i] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    float psum = 0.f;
    // probabilities of 16-key step ks as the B operand of the value product:
    // part j (0..3) forms keys 2 j, 2 j + 1 of each half-step's 8
    uint32_t pw[4][4];
    auto prob = [&](int ks, int j) __attribute__((always_inline)) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][(ks & 1) * 8 + 2 * j], sl2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][(ks & 1) * 8 + 2 * j + 1], sl2, neg_m));
      psum += p0 + p1;
      pw[ks][j] = pack_bf16x2(p0, p1);
    };
    auto pbf = [&](int ks) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, u32x4{pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]});
    };

    // ---- O^T += V^T P^T ----
    // fragment i = 4 ks + md, read kAttnAhead fragments ahead; step ks + 1's
    // probabilities are formed between step ks's MFMAs (the fences keep both)
    auto vload = [&](int i) __attribute__((always_inline)) {
      return *(const bf16x8*)(st + vb[i >> 2] + (i & 3) * 32 * L::kVRowB);
    };
    bf16x8 vf[kAttnAhead];
#pragma unroll
    for (int i = 0; i < kAttnAhead; ++i) vf[i] = vload(i);
#pragma unroll
    for (int j = 0; j < 4; ++j) prob(0, j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % kAttnAhead], pbf(i >> 2), o[i & 3], 0, 0, 0);
      if (i + kAttnAhead < 16) vf[i % kAttnAhead] = vload(i + kAttnAhead);
      if ((i >> 2) < 3) prob((i >> 2) + 1, i & 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    psum = sum_with_lane32(psum);
    l_run += psum;
  };

  // q and the carry are in registers before any tile load is in flight, so
  // the waits of the tile loop count only tile loads. The builtin (gfx9
  // encoding: vmcnt 0, other counters unlimited) tells the compiler that its
  // own loads are complete; otherwise it would wait for them, and with them
  // for the tile loads it cannot see, inside the loop.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (n_tiles > 0) issue(tile_begin, 0);
  for (int tt = 0; tt < n_tiles; tt += 2) {
    body(std::integral_constant<int, 0>(), tt);
    if (tt + 1 < n_tiles) body(std::integral_constant<int, 1>(), tt + 1);
  }

  if (!active) return;
  // O^T register i of block md holds dim 32*md + 8*(i/4) + 4*hf + i%4
  if (P < co + len) {  // last visible key is in this chunk: normalise and write
    // a sink adds e^sink to the denominator (l_run and o are relative to
    // 2^m_run; no visible key: m_run = -inf, the sink term inf, the output 0)
    const float l_tot = a.sink ? l_run + __builtin_amdgcn_exp2f(a.sink[b] * 1.44269504088896341f - m_run)
                               : l_run;
    const float inv = 1.0f / l_tot;
    uint16_t* op = a.out + (t * a.H + h) * kV;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(o[md][g * 4 + 0] * inv, o[md][g * 4 + 1] * inv);
        w[1] = pack_bf16x2(o[md][g * 4 + 2] * inv, o[md][g * 4 + 3] * inv);
        *(u32x2*)(op + md * 32 + g * 8 + hf * 4) = w;
      }
  } else {  // carry the state to the next chunk
    float* cp = a.carry_o + (t * a.H + h) * kV;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = o[md][g * 4 + j];
        *(f32x4*)(cp + md * 32 + g * 8 + hf * 4) = v;
      }
    if (hf == 0) {
      a.carry_ml[(t * a.H + h) * 2 + 0] = m_run;
      a.carry_ml[(t * a.H + h) * 2 + 1] = l_run;
    }
  }
}

// Query-block schedule: for every sequence its blocks of 128 queries, last
// (most keys) first; slots past the total are marked (-1, -1).
__global__ void __launch_bounds__(256) attn_schedule_kernel(int2* sched, const uint32_t* offs,
                                                             int B, int n_slots) {
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int nblk = 0;
    if (b < B) nblk = (int)((offs[b + 1] - offs[b] + kAttnBM - 1) / kAttnBM);
    s_scan[tid] = nblk;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int v = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int start = s_carry + s_scan[tid] - nblk;
    for (int j = 0; j < nblk; ++j)
      if (start + j < n_slots) sched[start + j] = make_int2(b, nblk - 1 - j);
    __syncthreads();
    if (tid == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  for (int k = s_carry + tid; k < n_slots; k += 256) sched[k] = make_int2(-1, -1);
}

int attn_num_slots(int B, int total_q) { return (total_q + kAttnBM - 1) / kAttnBM + B; }

hipError_t launch_attn_schedule(int2* sched, const uint32_t* offs, int B, int n_slots,
                                hipStream_t stream) {
  hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(256), 0, stream, sched, offs, B,
                     n_slots);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const AttnArgs& a, bool fp8, hipStream_t stream) {
  const long total = (long)a.n_slots * a.H;
  const long grid = (total + 7) / 8 * 8;
  if (fp8) hipLaunchKernelGGL(prefill_attn_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(prefill_attn_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
