// Kernel argument blocks and launchers shared between the libmla HIP sources.
#pragma once

#include "common.hpp"

namespace mla {
struct GatherArgs {
  uint16_t* latn;
  void* krope;
  const void* cache;
  const int32_t* page_table;
  const uint32_t* bro_c;
  const uint32_t* co_c;
  const int32_t* bl_c;
  const uint16_t* gamma;
  const uint16_t* freqs;
  int B, ps, maxp, num_pages, max_rows, max_seq_len;
  float eps;
};
struct KvWriteArgs {
  void* cache;               // [num_pages][ps][576] bf16 or e4m3fn, written
  const int32_t* page_table; // [B][maxp]
  const uint16_t* input;     // [total][576] bf16: the new tokens' raw rows
  const uint32_t* offs;      // [B+1] input_row_offsets
  const uint32_t* clen;      // [B] cache_lengths
  const uint16_t* gamma;
  const uint16_t* freqs;
  int B, total, ps, maxp, num_pages, max_seq_len;
  float eps;
};
struct GemmArgs {
  void* k_out;
  uint16_t* vt_out;
  const uint16_t* a;
  const uint16_t* wk;
  const uint16_t* wuv;
  const int32_t* bl_c;
  int H, max_rows;
};
struct AttnArgs {
  uint16_t* out;
  const void* q;
  const void* k_nope;
  const uint16_t* v_t;
  const void* krope;
  const uint32_t* offs;
  const uint32_t* clen;
  const uint32_t* bro_c;
  const uint32_t* co_c;
  const int32_t* bl_c;
  float* carry_o;
  float* carry_ml;
  const int2* sched;
  const float* sink;         // [B] sink logits (natural log, scaled-score units), or null
  int n_slots, B, H, max_rows;
  float scale_log2;
};
// Page-table entries the split-KV kernel stages in LDS per segment; the host
// sizes key ranges so that a segment never spans more pages.
constexpr int kDecPageWindow = 1024;
struct DecodeArgs {
  const uint16_t* q_abs;     // [B][H][576] bf16
  const void* cache;         // [num_pages][ps][576] bf16 or e4m3fn
  const int32_t* page_table; // [B][maxp]
  const uint32_t* cum;       // [B+1] prefix sums of the context lengths
  const uint32_t* wstart;    // [G+1] first key of every key range
  const int32_t* wfirst;     // [G] first sequence every key range touches
  uint16_t* part_o;          // [G + B][512 / 8][H][8] bf16: dims by groups of 8
  float* part_ml;            // [G + B][H][2]
  int B, H, ps, maxp, num_pages, G;
  float scale_log2;
};
struct CombineArgs {
  uint16_t* o_lat;           // [B][H][2][512] bf16: hi then lo
  const uint16_t* part_o;    // [G + B][512 / 8][H][8] bf16
  float* part_ml;            // [G + B][H][2] (max in the log2 domain, sum; a
                             // negative sum marks a partial to recompute)
  const uint32_t* cum;       // [B+1]
  const uint32_t* wstart;    // [G+1]
  const int2* wspan;         // [B]: first and last key range touching each sequence
  const uint16_t* q_abs;     // [B][H][576], for recomputation
  const void* cache;
  const int32_t* page_table;
  int B, H, G, ps, maxp, num_pages;
  float scale_log2;
  const float* sink;         // [B] sink logits, or null
  bool fp8;                  // cache holds e4m3fn codes (else bf16)
};
hipError_t launch_plan(uint32_t*, uint32_t*, int32_t*, uint32_t*, const uint32_t*,
                       const uint32_t*, int, int, uint32_t, hipStream_t);
// fp8 cache, fp8 krope, processed (rows copied as stored, no RMSNorm/RoPE)
hipError_t launch_gather(const GatherArgs&, bool, bool, bool, hipStream_t);
hipError_t launch_kv_write(const KvWriteArgs&, bool, hipStream_t);
hipError_t launch_up_project(const GemmArgs&, bool, hipStream_t);
int attn_num_slots(int B, int total_q);
hipError_t launch_attn_schedule(int2*, const uint32_t*, int, int, hipStream_t);
hipError_t launch_prefill_attn(const AttnArgs&, bool, hipStream_t);
// split-KV range tables: cum [B+1], wstart [G+1], wspan [B], wfirst [G] from the
// context lengths min(ctx[b] + add, max_ctx)
struct PrefixArgs {
  uint32_t* cum;
  const uint32_t* ctx;
  uint32_t add;
  int B;
  uint32_t max_ctx;
  uint32_t* wstart;
  int2* wspan;
  int32_t* wfirst;
  int G;
};
// q_abs, and the range tables in one extra workgroup
hipError_t launch_decode_absorb(uint16_t*, const uint16_t*, const uint16_t*, int, int,
                                const PrefixArgs&, hipStream_t);
hipError_t launch_decode_split(const DecodeArgs&, bool, hipStream_t);
hipError_t launch_decode_combine(const CombineArgs&, hipStream_t);
hipError_t launch_decode_project(uint16_t*, const uint16_t*, const uint16_t*, int, int,
                                 hipStream_t);
// streaming read of bytes (a multiple of 16) from src; one word per workgroup to out
hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* out, int groups,
                           hipStream_t stream);
}  // namespace mla
