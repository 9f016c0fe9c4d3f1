// Causal MLA prefill attention over one chunk of up-projected keys/values
// ("flare_mla_prefill_dispatch" page: q_depth 192 = 128 nope + 64 rope,
// kv_num_heads 1 for the rope part, v_depth 128, cache_offsets shifting the
// causal diagonal; bf16 or float8_e4m3fn inputs, bf16 output).
//
// Work decomposition. A workgroup (4 waves, 256 threads) owns one block of 128
// queries of one sequence and one head; each wave owns 32 of the queries.
// Keys are streamed in tiles of 64 rows aligned to the chunk buffer's 64-row
// grid (so every global load is 16-byte aligned); rows that belong to other
// sequences are masked.
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
// The k_rope tile (one head shared by all query heads) sits beside K_nope in
// the same LDS row, so the 192-deep score reduction is 12 MFMA steps.
//
// Softmax runs online in the log2 domain (scale * log2(e) folded into one
// multiply). Its state (max, sum, unnormalised output) is carried across the
// chunks of a sequence through the workspace; a query's output is written in
// the chunk that holds its last visible key.
#include "kernels.hpp"

namespace mla {

constexpr int kAttnBM = 128;           // queries per workgroup
constexpr int kAttnBN = 64;            // keys per tile
constexpr int kKRowBf16 = kQDepth + 8; // LDS K row, bf16 elements (400 B)
constexpr int kKRowFp8 = kQDepth + 16; // LDS K row, bytes (208 B)
constexpr int kVRow = kAttnBN + 8;     // LDS V^T row, bf16 elements (144 B)


typedef long fp8x8;  // 8 e4m3 values in one 64-bit register pair

// Rescale the output accumulator only when a query's running maximum grows by
// more than this many (log2) units; in between, probabilities are formed
// against the stale maximum and stay below 2^8, exact in fp32 and bf16 range.
constexpr float kRescaleSlack = 8.0f;

// Per-thread staging registers of one key tile (global -> registers -> LDS).
template <bool kFp8>
struct TileRegs;
template <>
struct TileRegs<false> {
  u32x4 kn[4], kr[2], v[4];
};
template <>
struct TileRegs<true> {
  u32x4 kn[2], kr[1], v[4];
};

template <bool kFp8>
__device__ __forceinline__ void load_tile(TileRegs<kFp8>& R, const AttnArgs& a, int h, int tb,
                                          int r0, int len, int tid) {
  const int lo = max(r0, 0);
  const int hi = min(r0 + len, a.max_rows);
  const bool full = tb >= lo && tb + kAttnBN <= hi;  // uniform across the workgroup
  const size_t kbase = (size_t)h * a.max_rows;
  if (kFp8) {
    const uint8_t* kn = (const uint8_t*)a.k_nope;
    const uint8_t* kr = (const uint8_t*)a.krope;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256;
      const int gr = tb + (c >> 3);
      const bool ok = full || (gr >= lo && gr < hi);
      R.kn[it] = ok ? *(const u32x4*)(kn + (kbase + gr) * kNope + (c & 7) * 16) : u32x4{0, 0, 0, 0};
    }
    {
      const int gr = tb + (tid >> 2);
      const bool ok = full || (gr >= lo && gr < hi);
      ((u32x4*)R.kr)[0] = ok ? *(const u32x4*)(kr + (size_t)gr * kRope + (tid & 3) * 16)
                             : u32x4{0, 0, 0, 0};
    }
  } else {
    const uint16_t* kn = (const uint16_t*)a.k_nope;
    const uint16_t* kr = (const uint16_t*)a.krope;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + it * 256;
      const int gr = tb + (c >> 4);
      const bool ok = full || (gr >= lo && gr < hi);
      ((u32x4*)R.kn)[it] =
          ok ? *(const u32x4*)(kn + (kbase + gr) * kNope + (c & 15) * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256;
      const int gr = tb + (c >> 3);
      const bool ok = full || (gr >= lo && gr < hi);
      ((u32x4*)R.kr)[it] =
          ok ? *(const u32x4*)(kr + (size_t)gr * kRope + (c & 7) * 8) : u32x4{0, 0, 0, 0};
    }
  }
  const uint16_t* vbase = a.v_t + (size_t)h * kV * a.max_rows;
#pragma unroll
  for (int it = 0; it < 4; ++it) {  // V^T: 128 dims x 8 chunks of 8 keys
    const int c = tid + it * 256;
    const int k0 = tb + (c & 7) * 8;
    u32x4 v = *(const u32x4*)(vbase + (size_t)(c >> 3) * a.max_rows + k0);
    if (!full && (k0 < lo || k0 + 8 > hi)) {  // zero keys outside this sequence
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ka = k0 + 2 * j;
        uint32_t w = v[j];
        if (ka < lo || ka >= hi) w &= 0xFFFF0000u;
        if (ka + 1 < lo || ka + 1 >= hi) w &= 0x0000FFFFu;
        v[j] = w;
      }
    }
    R.v[it] = v;
  }
}

template <bool kFp8>
__device__ __forceinline__ void store_tile(const TileRegs<kFp8>& R, uint8_t* sK, uint16_t* sV,
                                           int tid) {
  if (kFp8) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256;
      *(u32x4*)(sK + (c >> 3) * kKRowFp8 + (c & 7) * 16) = R.kn[it];
    }
    *(u32x4*)(sK + (tid >> 2) * kKRowFp8 + kNope + (tid & 3) * 16) = ((const u32x4*)R.kr)[0];
  } else {
    uint16_t* k16 = (uint16_t*)sK;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + it * 256;
      *(u32x4*)(k16 + (c >> 4) * kKRowBf16 + (c & 15) * 8) = ((const u32x4*)R.kn)[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256;
      *(u32x4*)(k16 + (c >> 3) * kKRowBf16 + kNope + (c & 7) * 8) = ((const u32x4*)R.kr)[it];
    }
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + it * 256;
    *(u32x4*)(sV + (c >> 3) * kVRow + (c & 7) * 8) = R.v[it];
  }
}

template <bool kFp8>
__global__ void __launch_bounds__(256, 2) prefill_attn_kernel(AttnArgs a) {
  constexpr int kKBytes = kFp8 ? kAttnBN * kKRowFp8 : kAttnBN * kKRowBf16 * 2;
  __shared__ __attribute__((aligned(16))) uint8_t sK[kKBytes];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kV * kVRow];

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
  const int kv_end = min(len, P_hi - co + 1);             // keys j < kv_end can be visible
  const int all_vis = min(len, c_b + q_lo - co + 1);      // keys j < all_vis visible to all

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int qi = q_lo + wave * 32 + l32;
  const bool qvalid = qi < n_b;
  const int P = c_b + qi;
  const bool active = qvalid && P >= co;
  const size_t t = (size_t)t0 + qi;
  // visible buffer rows of this query: [r0, r_hi]
  const int r_hi = active ? r0 + min(len - 1, P - co) : r0 - 1;
  const bool wave_active = __ballot(active) != 0;

  // Q fragments: B operand of S^T = K Q^T (lane: query l32, depth 8*hf + 16*ks ..)
  bf16x8 qf[12];
  fp8x8 qf8[12];
  if (kFp8) {
    const uint8_t* qp = (const uint8_t*)a.q + (t * a.H + h) * kQDepth + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) qf8[ks] = qvalid ? *(const fp8x8*)(qp + ks * 16) : 0;
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

  // permuted K row fed by this lane: swap bits 2 and 3 of l32
  const int kappa = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const float sl2 = a.scale_log2;

  const int tile_begin = r0 & ~(kAttnBN - 1);
  // never past the buffer, even if a caller's max_rows is smaller than the chunk
  const int tile_end = min(r0 + kv_end, a.max_rows);

  TileRegs<kFp8> R;
  if (tile_begin < tile_end) load_tile<kFp8>(R, a, h, tile_begin, r0, len, tid);

  for (int tb = tile_begin; tb < tile_end; tb += kAttnBN) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile<kFp8>(R, sK, sV, tid);
    __syncthreads();
    if (tb + kAttnBN < tile_end) load_tile<kFp8>(R, a, h, tb + kAttnBN, r0, len, tid);
    if (!wave_active) continue;

    // ---- S^T = K Q^T for 64 keys x 32 queries ----
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (kFp8) {
          const fp8x8 ka = *(const fp8x8*)(sK + (mb * 32 + kappa) * kKRowFp8 + ks * 16 + hf * 8);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(ka, qf8[ks], s[mb], 0, 0, 0);
        } else {
          const bf16x8 ka = *(const bf16x8*)((const uint16_t*)sK +
                                             (mb * 32 + kappa) * kKRowBf16 + ks * 16 + hf * 8);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[mb], 0, 0, 0);
        }
      }
    }

    // ---- online softmax (log2 domain), lazily rescaled ----
    // register i of block mb holds the key at tile row 32*mb + 16*(i/8) + 8*hf + i%8
    if ((tb < r0) || (tb + kAttnBN > r0 + all_vis)) {
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
    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][(ks & 1) * 8 + 2 * j], sl2, neg_m));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][(ks & 1) * 8 + 2 * j + 1], sl2, neg_m));
        psum += p0 + p1;
        w[j] = pack_bf16x2(p0, p1);
      }
      pb[ks] = __builtin_bit_cast(bf16x8, w);
    }
    psum = sum_with_lane32(psum);
    l_run += psum;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int md = 0; md < 4; ++md) {
        const bf16x8 va = *(const bf16x8*)(sV + (md * 32 + l32) * kVRow + ks * 16 + hf * 8);
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[md], 0, 0, 0);
      }
    }
  }

  if (!active) return;
  // O^T register i of block md holds dim 32*md + 8*(i/4) + 4*hf + i%4
  if (P < co + len) {  // last visible key is in this chunk: normalise and write
    const float inv = 1.0f / l_run;
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
