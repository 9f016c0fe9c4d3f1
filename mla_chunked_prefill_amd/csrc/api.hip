// C ABI of libmla.so: host-side validation, workspace layout and kernel
// launches. Declarations and contracts are in include/mla.h.
#include <initializer_list>
#include <math.h>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include <stdarg.h>

#include "../../include/mla.h"
#include "kernels.hpp"


namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(int32_t d) { return d == MLA_BF16 || d == MLA_FP8_E4M3FN; }

// the kernels move tensor data in 16-byte vectors and direct-to-LDS loads
bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((uintptr_t)p & 15) return true;
  return false;
}
size_t dsize(int32_t d) { return d == MLA_FP8_E4M3FN ? 1 : 2; }

constexpr float kLog2e = 1.4426950408889634f;

// prefill-attention workspace: carry O [Tq][H][128] f32, carry ml [Tq][H][2] f32,
// schedule [n_slots] int2
struct AttnWs {
  float* carry_o;
  float* carry_ml;
  int2* sched;
  size_t bytes;
};
AttnWs attn_ws_layout(char* base, int B, int total_q, int H) {
  AttnWs w;
  size_t off = 0;
  w.carry_o = (float*)(base + off);
  off = align_up(off + (size_t)total_q * H * mla::kV * sizeof(float));
  w.carry_ml = (float*)(base + off);
  off = align_up(off + (size_t)total_q * H * 2 * sizeof(float));
  w.sched = (int2*)(base + off);
  off = align_up(off + (size_t)mla::attn_num_slots(B, total_q) * sizeof(int2));
  w.bytes = off;
  return w;
}

// prefill workspace: latent [R][512] bf16, krope [R][64], K_nope [H][R][128],
// V^T [H][128][R] bf16, then the attention workspace
struct PrefillWs {
  uint16_t* latn;
  void* krope;
  void* k_nope;
  uint16_t* v_t;
  AttnWs attn;
  size_t bytes;
};
PrefillWs prefill_ws_layout(char* base, int B, int total_q, int H, int max_rows, int dtype) {
  PrefillWs w;
  size_t off = 0;
  const size_t R = (size_t)max_rows;
  w.latn = (uint16_t*)(base + off);
  off = align_up(off + R * mla::kLora * 2);
  w.krope = base + off;
  off = align_up(off + R * mla::kRope * dsize(dtype));
  w.k_nope = base + off;
  off = align_up(off + (size_t)H * R * mla::kNope * dsize(dtype));
  w.v_t = (uint16_t*)(base + off);
  off = align_up(off + (size_t)H * mla::kV * R * 2);
  w.attn = attn_ws_layout(base ? base + off : nullptr, B, total_q, H);
  off += w.attn.bytes;
  w.bytes = off;
  return w;
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    return 256;  // MI355X
  }
  return n;
}

// Split workgroups over the batch: one per compute unit by default. A range
// of L keys starting mid-page, with its first tile aligned down to 32 keys,
// spans at most (L + 30) / page_size + 2 pages, which must fit the page-table
// window the kernel stages in LDS.
int decode_groups(int B, int max_ctx, int page_size, int num_partitions) {
  int g = num_partitions > 0 ? num_partitions : device_cu_count();
  const long long keys = (long long)B * max_ctx;
  const long long per_group = (long long)(mla::kDecPageWindow - 2) * page_size - 64;
  const long long need = (keys + per_group - 1) / per_group;
  if (g < need) g = (int)need;
  return g;
}

// decode workspace: q_abs [B][H][576] bf16, cum [B+1] u32, wstart [G+1] u32,
// wspan [B] int2, wfirst [G] i32, part_o [G+B][64][H][8] bf16, part_ml [G+B][H][2] f32, o_lat
// [B][H][2][512] bf16 (hi, lo). G split workgroups cover the batch's
// concatenated contexts in equal ranges.
struct DecodeWs {
  uint16_t* q_abs;
  uint32_t* cum;
  uint32_t* wstart;
  int2* wspan;
  int32_t* wfirst;
  uint16_t* part_o;
  float* part_ml;
  uint16_t* o_lat;
  int G;
  size_t bytes;
};
DecodeWs decode_ws_layout(char* base, int B, int H, int max_ctx, int page_size,
                          int num_partitions, int cache_dtype) {
  DecodeWs w;
  w.G = decode_groups(B, max_ctx, page_size, num_partitions);
  const size_t slots = (size_t)w.G + B;
  size_t off = 0;
  w.q_abs = (uint16_t*)(base + off);
  off = align_up(off + (size_t)B * H * mla::kCache * 2);
  w.cum = (uint32_t*)(base + off);
  off = align_up(off + (size_t)(B + 1) * sizeof(uint32_t));
  w.wstart = (uint32_t*)(base + off);
  off = align_up(off + (size_t)(w.G + 1) * sizeof(uint32_t));
  w.wspan = (int2*)(base + off);
  off = align_up(off + (size_t)B * sizeof(int2));
  w.wfirst = (int32_t*)(base + off);
  off = align_up(off + (size_t)w.G * sizeof(int32_t));
  w.part_o = (uint16_t*)(base + off);
  off = align_up(off + slots * H * mla::kLora * sizeof(uint16_t));
  w.part_ml = (float*)(base + off);
  off = align_up(off + slots * H * 2 * sizeof(float));
  w.o_lat = (uint16_t*)(base + off);
  off = align_up(off + (size_t)B * H * 2 * mla::kLora * 2);
  w.bytes = off;
  return w;
}

// One chunk's rows into the contiguous buffers (no argument checks). processed:
// the pool rows are copied as stored; otherwise they are normalised and rotated.
int gather_rows(void* latent_out, void* krope_out, int32_t krope_dtype, const void* kv_cache,
                int32_t cache_dtype, bool processed, const int32_t* page_table,
                const uint32_t* bro_c, const uint32_t* co_c, const int32_t* bl_c,
                const void* gamma, const void* freqs, int32_t B, int32_t page_size,
                int32_t maxp, int32_t num_pages, int32_t max_rows, int32_t freqs_len, float eps,
                hipStream_t stream) {
  mla::GatherArgs a;
  a.latn = (uint16_t*)latent_out;
  a.krope = krope_out;
  a.cache = kv_cache;
  a.page_table = page_table;
  a.bro_c = bro_c;
  a.co_c = co_c;
  a.bl_c = bl_c;
  a.gamma = (const uint16_t*)gamma;
  a.freqs = (const uint16_t*)freqs;
  a.B = B;
  a.ps = page_size;
  a.maxp = maxp;
  a.num_pages = num_pages;
  a.max_rows = max_rows;
  a.max_seq_len = freqs_len;
  a.eps = eps;
  return hip_status(mla::launch_gather(a, cache_dtype == MLA_FP8_E4M3FN,
                                       krope_dtype == MLA_FP8_E4M3FN, processed, stream),
                    "gather kernel");
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dtype or dimension";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* mla_last_error(void) { return g_last_error; }

int mla_hbm_read(const void* src, size_t bytes, uint32_t* out, int32_t groups,
                 hipStream_t stream) {
  if (!src || !out) return fail(MLA_ERR_INVALID_ARG, "mla_hbm_read: null pointer");
  if (misaligned({src}) || bytes % 16 != 0 || bytes == 0 || groups < 1 || groups > (1 << 20))
    return fail(MLA_ERR_INVALID_ARG, "mla_hbm_read: bytes=%zu groups=%d", bytes, groups);
  return hip_status(mla::launch_hbm_read(src, bytes, out, groups, stream), "read kernel");
}

int mla_prefill_plan(uint32_t* buffer_row_offsets, uint32_t* cache_offsets,
                     int32_t* buffer_lengths, uint32_t* chunks_needed,
                     const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                     int32_t batch_size, int32_t max_chunks, uint32_t buffer_token_size,
                     hipStream_t stream) {
  if (!buffer_row_offsets || !cache_offsets || !buffer_lengths || !input_row_offsets ||
      !cache_lengths)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_plan: null pointer");
  if (batch_size < 1 || max_chunks < 1 || buffer_token_size < 1)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_plan: batch_size=%d max_chunks=%d T=%u",
                batch_size, max_chunks, buffer_token_size);
  if ((uint64_t)batch_size * buffer_token_size >= (1ull << 31))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_plan: batch_size * T must be < 2^31");
  return hip_status(mla::launch_plan(buffer_row_offsets, cache_offsets, buffer_lengths,
                                     chunks_needed, input_row_offsets, cache_lengths,
                                     batch_size, max_chunks, buffer_token_size, stream),
                    "plan kernel");
}

int mla_gather_norm_rope(void* latent_out, void* krope_out, int32_t krope_dtype,
                         const void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                         const uint32_t* buffer_row_offsets_c, const uint32_t* cache_offsets_c,
                         const int32_t* buffer_length_c, const void* kv_norm_gamma,
                         const void* freqs_cis, int32_t batch_size, int32_t page_size,
                         int32_t max_pages_per_seq, int32_t num_pages, int32_t max_rows,
                         int32_t max_seq_len, float epsilon, hipStream_t stream) {
  if (!latent_out || !krope_out || !kv_cache || !page_table || !buffer_row_offsets_c ||
      !cache_offsets_c || !buffer_length_c || !kv_norm_gamma || !freqs_cis)
    return fail(MLA_ERR_INVALID_ARG, "mla_gather_norm_rope: null pointer");
  if (misaligned({latent_out, krope_out, kv_cache, kv_norm_gamma, freqs_cis}))
    return fail(MLA_ERR_INVALID_ARG, "mla_gather_norm_rope: tensor not 16-byte aligned");
  if (!dtype_ok(krope_dtype) || !dtype_ok(cache_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "mla_gather_norm_rope: dtype");
  if (batch_size < 1 || page_size < 1 || max_pages_per_seq < 1 || num_pages < 1 ||
      max_rows < 1 || max_seq_len < 1 || !(epsilon >= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "mla_gather_norm_rope: sizes");
  return gather_rows(latent_out, krope_out, krope_dtype, kv_cache, cache_dtype, false,
                     page_table, buffer_row_offsets_c, cache_offsets_c, buffer_length_c,
                     kv_norm_gamma, freqs_cis, batch_size, page_size, max_pages_per_seq,
                     num_pages, max_rows, max_seq_len, epsilon, stream);
}

static int kv_write_rows(void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                         const void* kv_input, const uint32_t* input_row_offsets,
                         const uint32_t* cache_lengths, const void* kv_norm_gamma,
                         const void* freqs_cis, int32_t batch_size, int32_t total_tokens,
                         int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                         int32_t max_seq_len, float epsilon, hipStream_t stream);

int mla_kv_write(void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                 const void* kv_input, const uint32_t* input_row_offsets,
                 const uint32_t* cache_lengths, const void* kv_norm_gamma, const void* freqs_cis,
                 int32_t batch_size, int32_t total_tokens, int32_t page_size,
                 int32_t max_pages_per_seq, int32_t num_pages, int32_t max_seq_len, float epsilon,
                 hipStream_t stream) {
  if (!kv_cache || !page_table || !kv_input || !input_row_offsets || !cache_lengths ||
      !kv_norm_gamma || !freqs_cis)
    return fail(MLA_ERR_INVALID_ARG, "mla_kv_write: null pointer");
  if (misaligned({kv_cache, kv_input, kv_norm_gamma, freqs_cis}))
    return fail(MLA_ERR_INVALID_ARG, "mla_kv_write: tensor not 16-byte aligned");
  if (!dtype_ok(cache_dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_kv_write: dtype");
  if (batch_size < 1 || total_tokens < 0 || page_size < 1 || max_pages_per_seq < 1 ||
      num_pages < 1 || max_seq_len < 1 || !(epsilon >= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "mla_kv_write: sizes");
  return kv_write_rows(kv_cache, cache_dtype, page_table, kv_input, input_row_offsets,
                       cache_lengths, kv_norm_gamma, freqs_cis, batch_size, total_tokens,
                       page_size, max_pages_per_seq, num_pages, max_seq_len, epsilon, stream);
}

// The KV write launch (arguments already checked).
static int kv_write_rows(void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                         const void* kv_input, const uint32_t* input_row_offsets,
                         const uint32_t* cache_lengths, const void* kv_norm_gamma,
                         const void* freqs_cis, int32_t batch_size, int32_t total_tokens,
                         int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                         int32_t max_seq_len, float epsilon, hipStream_t stream) {
  if (total_tokens == 0) return MLA_OK;
  mla::KvWriteArgs a;
  a.cache = kv_cache;
  a.page_table = page_table;
  a.input = (const uint16_t*)kv_input;
  a.offs = input_row_offsets;
  a.clen = cache_lengths;
  a.gamma = (const uint16_t*)kv_norm_gamma;
  a.freqs = (const uint16_t*)freqs_cis;
  a.B = batch_size;
  a.total = total_tokens;
  a.ps = page_size;
  a.maxp = max_pages_per_seq;
  a.num_pages = num_pages;
  a.max_seq_len = max_seq_len;
  a.eps = epsilon;
  return hip_status(mla::launch_kv_write(a, cache_dtype == MLA_FP8_E4M3FN, stream),
                    "kv write kernel");
}

int mla_up_project(void* k_nope_out, void* v_t_out, int32_t k_dtype, const void* latent,
                   const void* w_k, const void* w_uv, const int32_t* buffer_length_c,
                   int32_t num_heads, int32_t max_rows, hipStream_t stream) {
  if (!k_nope_out || !v_t_out || !latent || !w_k || !w_uv || !buffer_length_c)
    return fail(MLA_ERR_INVALID_ARG, "mla_up_project: null pointer");
  if (misaligned({k_nope_out, v_t_out, latent, w_k, w_uv}))
    return fail(MLA_ERR_INVALID_ARG, "mla_up_project: tensor not 16-byte aligned");
  if (!dtype_ok(k_dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_up_project: dtype");
  if (num_heads < 1 || num_heads > 1024 || max_rows < 64 || max_rows % 64 != 0)
    return fail(MLA_ERR_INVALID_ARG, "mla_up_project: num_heads=%d max_rows=%d", num_heads,
                max_rows);
  mla::GemmArgs g;
  g.k_out = k_nope_out;
  g.vt_out = (uint16_t*)v_t_out;
  g.a = (const uint16_t*)latent;
  g.wk = (const uint16_t*)w_k;
  g.wuv = (const uint16_t*)w_uv;
  g.bl_c = buffer_length_c;
  g.H = num_heads;
  g.max_rows = max_rows;
  return hip_status(mla::launch_up_project(g, k_dtype == MLA_FP8_E4M3FN, stream),
                    "up-projection kernel");
}

size_t mla_prefill_attention_workspace_size(int32_t batch_size, int32_t total_q,
                                            int32_t num_heads) {
  if (batch_size < 1 || total_q < 0 || num_heads < 1) return 0;
  return attn_ws_layout(nullptr, batch_size, total_q, num_heads).bytes;
}

static int attention_common(void* output, const void* q, int32_t dtype, const void* k_nope,
                            const void* v_t, const void* krope,
                            const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                            const uint32_t* bro_c, const uint32_t* co_c, const int32_t* bl_c,
                            int32_t B, int32_t total_q, int32_t H, int32_t max_rows,
                            float scale, const float* attn_sink, const AttnWs& ws,
                            hipStream_t stream) {
  mla::AttnArgs a;
  a.out = (uint16_t*)output;
  a.q = q;
  a.k_nope = k_nope;
  a.v_t = (const uint16_t*)v_t;
  a.krope = krope;
  a.offs = input_row_offsets;
  a.clen = cache_lengths;
  a.bro_c = bro_c;
  a.co_c = co_c;
  a.bl_c = bl_c;
  a.carry_o = ws.carry_o;
  a.carry_ml = ws.carry_ml;
  a.sched = ws.sched;
  a.n_slots = mla::attn_num_slots(B, total_q);
  a.B = B;
  a.H = H;
  a.max_rows = max_rows;
  a.scale_log2 = scale * kLog2e;
  a.sink = attn_sink;
  return hip_status(mla::launch_prefill_attn(a, dtype == MLA_FP8_E4M3FN, stream),
                    "attention kernel");
}

int mla_prefill_attention(void* output, const void* q, int32_t dtype, const void* k_nope,
                          const void* v_t, const void* krope, const uint32_t* input_row_offsets,
                          const uint32_t* cache_lengths, const uint32_t* buffer_row_offsets_c,
                          const uint32_t* cache_offsets_c, const int32_t* buffer_length_c,
                          int32_t batch_size, int32_t total_q, int32_t num_heads,
                          int32_t max_rows, int32_t max_prompt_len, float scale,
                          const float* attn_sink, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!output || !q || !k_nope || !v_t || !krope || !input_row_offsets || !cache_lengths ||
      !buffer_row_offsets_c || !cache_offsets_c || !buffer_length_c)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_attention: null pointer");
  if (misaligned({output, q, k_nope, v_t, krope, workspace}))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_attention: tensor not 16-byte aligned");
  if (!dtype_ok(dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_attention: dtype");
  if (batch_size < 1 || total_q < 1 || num_heads < 1 || num_heads > 1024 || max_rows < 64 ||
      max_rows % 64 != 0 || max_prompt_len < 1 || !(scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_attention: sizes");
  const size_t need = mla_prefill_attention_workspace_size(batch_size, total_q, num_heads);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "mla_prefill_attention: workspace %zu < %zu",
                workspace_bytes, need);
  AttnWs ws = attn_ws_layout((char*)workspace, batch_size, total_q, num_heads);
  int st = hip_status(mla::launch_attn_schedule(ws.sched, input_row_offsets, batch_size,
                                                mla::attn_num_slots(batch_size, total_q),
                                                stream),
                      "schedule kernel");
  if (st != MLA_OK) return st;
  return attention_common(output, q, dtype, k_nope, v_t, krope, input_row_offsets,
                          cache_lengths, buffer_row_offsets_c, cache_offsets_c,
                          buffer_length_c, batch_size, total_q, num_heads, max_rows, scale,
                          attn_sink, ws, stream);
}

// The chunk loop of a planned prefill (arguments already checked; rows is
// max_rows rounded up to 64): per chunk gather, up-projection, attention with
// the carried softmax state. Chunks whose buffer length is -1 exit on the device.
static int prefill_chunks(void* output, const void* q, int32_t dtype,
                          const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                          const void* kv_cache, int32_t cache_dtype, bool processed,
                          const int32_t* page_table, const uint32_t* buffer_row_offsets,
                          const uint32_t* cache_offsets, const int32_t* buffer_lengths,
                          int32_t max_chunks, int32_t rows, const void* w_k, const void* w_uv,
                          const void* kv_norm_gamma, const void* freqs_cis, int32_t batch_size,
                          int32_t total_q, int32_t num_heads, int32_t page_size,
                          int32_t max_pages_per_seq, int32_t num_pages, int32_t freqs_len,
                          float scale, float epsilon, const float* attn_sink, void* workspace,
                          hipStream_t stream) {
  PrefillWs ws =
      prefill_ws_layout((char*)workspace, batch_size, total_q, num_heads, rows, dtype);
  int st = hip_status(mla::launch_attn_schedule(ws.attn.sched, input_row_offsets, batch_size,
                                                mla::attn_num_slots(batch_size, total_q),
                                                stream),
                      "schedule kernel");
  if (st != MLA_OK) return st;
  for (int c = 0; c < max_chunks; ++c) {
    const uint32_t* bro_c = buffer_row_offsets + (size_t)c * (batch_size + 1);
    const uint32_t* co_c = cache_offsets + (size_t)c * batch_size;
    const int32_t* bl_c = buffer_lengths + c;
    st = gather_rows(ws.latn, ws.krope, dtype, kv_cache, cache_dtype, processed, page_table,
                     bro_c, co_c, bl_c, kv_norm_gamma, freqs_cis, batch_size, page_size,
                     max_pages_per_seq, num_pages, rows, freqs_len, epsilon, stream);
    if (st != MLA_OK) return st;
    st = mla_up_project(ws.k_nope, ws.v_t, dtype, ws.latn, w_k, w_uv, bl_c, num_heads, rows,
                        stream);
    if (st != MLA_OK) return st;
    st = attention_common(output, q, dtype, ws.k_nope, ws.v_t, ws.krope, input_row_offsets,
                          cache_lengths, bro_c, co_c, bl_c, batch_size, total_q, num_heads,
                          rows, scale, attn_sink, ws.attn, stream);
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

size_t mla_prefill_workspace_size(int32_t batch_size, int32_t total_q, int32_t num_heads,
                                  int32_t max_rows, int32_t dtype) {
  if (batch_size < 1 || total_q < 0 || num_heads < 1 || max_rows < 1 || !dtype_ok(dtype))
    return 0;
  const int32_t rows = (max_rows + 63) / 64 * 64;
  return prefill_ws_layout(nullptr, batch_size, total_q, num_heads, rows, dtype).bytes;
}

int mla_prefill(void* output, const void* q, int32_t dtype, const uint32_t* input_row_offsets,
                const uint32_t* cache_lengths, const void* kv_cache, const int32_t* page_table,
                const uint32_t* buffer_row_offsets, const uint32_t* cache_offsets,
                const int32_t* buffer_lengths, int32_t max_chunks, int32_t max_rows,
                const void* w_k, const void* w_uv, const void* kv_norm_gamma,
                const void* freqs_cis, int32_t batch_size, int32_t total_q, int32_t num_heads,
                int32_t max_prompt_len, int32_t page_size, int32_t max_pages_per_seq,
                int32_t num_pages, int32_t max_seq_len, float scale, float epsilon,
                const float* attn_sink,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!output || !q || !input_row_offsets || !cache_lengths || !kv_cache || !page_table ||
      !buffer_row_offsets || !cache_offsets || !buffer_lengths || !w_k || !w_uv ||
      !kv_norm_gamma || !freqs_cis)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill: null pointer");
  if (misaligned({output, q, kv_cache, w_k, w_uv, kv_norm_gamma, freqs_cis, workspace}))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill: tensor not 16-byte aligned");
  if (!dtype_ok(dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_prefill: dtype");
  if (batch_size < 1 || total_q < 1 || num_heads < 1 || num_heads > 1024 || max_chunks < 1 ||
      max_rows < 1 || max_prompt_len < 1 || page_size < 1 || max_pages_per_seq < 1 ||
      num_pages < 1 || max_seq_len < 1 || !(scale > 0.f) || !(epsilon >= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill: sizes");
  const int32_t rows = (max_rows + 63) / 64 * 64;
  const size_t need =
      mla_prefill_workspace_size(batch_size, total_q, num_heads, max_rows, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "mla_prefill: workspace %zu < %zu", workspace_bytes, need);
  return prefill_chunks(output, q, dtype, input_row_offsets, cache_lengths, kv_cache, dtype,
                        false, page_table, buffer_row_offsets, cache_offsets, buffer_lengths,
                        max_chunks, rows, w_k, w_uv, kv_norm_gamma, freqs_cis, batch_size,
                        total_q, num_heads, page_size, max_pages_per_seq, num_pages,
                        max_seq_len, scale, epsilon, attn_sink, workspace, stream);
}

static int decode_body(void* output, const void* q, const uint32_t* context_lengths,
                       uint32_t add, const void* kv_cache, int32_t cache_dtype,
                       const int32_t* page_table, const void* w_uk, const void* w_uv,
                       int32_t batch_size, int32_t num_heads, int32_t page_size,
                       int32_t max_pages_per_seq, int32_t num_pages, int32_t max_context_len,
                       int32_t num_partitions, float scale, const float* attn_sink,
                       void* workspace, hipStream_t stream);

size_t mla_decode_workspace_size(int32_t batch_size, int32_t num_heads, int32_t max_context_len,
                                 int32_t page_size, int32_t num_partitions, int32_t cache_dtype) {
  if (batch_size < 1 || num_heads < 1 || max_context_len < 1 || page_size < 1 ||
      num_partitions < 0 || !dtype_ok(cache_dtype))
    return 0;
  return decode_ws_layout(nullptr, batch_size, num_heads, max_context_len, page_size,
                          num_partitions, cache_dtype)
      .bytes;
}

int mla_decode(void* output, const void* q, const uint32_t* context_lengths,
               const void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
               const void* w_uk, const void* w_uv, int32_t batch_size, int32_t num_heads,
               int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
               int32_t max_context_len, int32_t num_partitions, float scale,
               const float* attn_sink, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (!output || !q || !context_lengths || !kv_cache || !page_table || !w_uk || !w_uv)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: null pointer");
  if (misaligned({output, q, kv_cache, w_uk, w_uv, workspace}))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: tensor not 16-byte aligned");
  if (!dtype_ok(cache_dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_decode: dtype");
  if (batch_size < 1 || num_heads < 1 || num_heads > 128 || page_size < 1 ||
      max_pages_per_seq < 1 || num_pages < 1 || max_context_len < 1 || num_partitions < 0 ||
      num_partitions > 65536 || !(scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: sizes (num_heads must be 1..128)");
  if ((uint64_t)batch_size * (uint64_t)max_context_len >= (1ull << 31) ||
      (uint64_t)num_pages * (uint64_t)page_size >= (1ull << 31))
    return fail(MLA_ERR_INVALID_ARG,
                "mla_decode: batch_size * max_context_len and num_pages * page_size must be < 2^31");
  const size_t need = mla_decode_workspace_size(batch_size, num_heads, max_context_len,
                                                page_size, num_partitions, cache_dtype);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "mla_decode: workspace %zu < %zu", workspace_bytes, need);
  return decode_body(output, q, context_lengths, 0, kv_cache, cache_dtype, page_table, w_uk,
                     w_uv, batch_size, num_heads, page_size, max_pages_per_seq, num_pages,
                     max_context_len, num_partitions, scale, attn_sink, workspace, stream);
}

// Allocation-free decode: the workspace of mla_decode lives in this array, one
// copy per GPU (each device that loads the library holds it until the process
// ends). Host code never passes the array's name to a kernel: its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and is kept per device.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "mla_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_noalloc: device %d beyond %d", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                        "mla_decode_noalloc: hipGetSymbolAddress of the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}
}  // namespace

int mla_decode_noalloc(void* output, const void* q, const uint32_t* context_lengths,
                       const void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                       const void* w_uk, const void* w_uv, int32_t batch_size, int32_t num_heads,
                       int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                       int32_t max_context_len, int32_t num_partitions, float scale,
                       const float* attn_sink, hipStream_t stream) {
  if (!output || !q || !context_lengths || !kv_cache || !page_table || !w_uk || !w_uv)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_noalloc: null pointer");
  if (misaligned({output, q, kv_cache, w_uk, w_uv}))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_noalloc: tensor not 16-byte aligned");
  if (!dtype_ok(cache_dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_noalloc: dtype");
  if (batch_size < 1 || num_heads < 1 || num_heads > 128 || page_size < 1 ||
      max_pages_per_seq < 1 || num_pages < 1 || max_context_len < 1 || num_partitions < 0 ||
      num_partitions > 65536 || !(scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_noalloc: sizes (num_heads must be 1..128)");
  if ((uint64_t)batch_size * (uint64_t)max_context_len >= (1ull << 31) ||
      (uint64_t)num_pages * (uint64_t)page_size >= (1ull << 31))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_noalloc: batch_size * max_context_len and "
                "num_pages * page_size must be < 2^31");
  const size_t need = mla_decode_workspace_size(batch_size, num_heads, max_context_len,
                                                page_size, num_partitions, cache_dtype);
  if (need == 0 || need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE,
                "mla_decode_noalloc: this decode needs %zu bytes of scratch, beyond the "
                "library's fixed %zu (use mla_decode with a workspace)",
                need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != MLA_OK) return st;
  return decode_body(output, q, context_lengths, 0, kv_cache, cache_dtype, page_table, w_uk,
                     w_uv, batch_size, num_heads, page_size, max_pages_per_seq, num_pages,
                     max_context_len, num_partitions, scale, attn_sink, ws, stream);
}

// The absorbed decode (arguments already checked): context length of sequence
// b is context_lengths[b] + add, at most max_context_len.
static int decode_body(void* output, const void* q, const uint32_t* context_lengths,
                       uint32_t add, const void* kv_cache, int32_t cache_dtype,
                       const int32_t* page_table, const void* w_uk, const void* w_uv,
                       int32_t batch_size, int32_t num_heads, int32_t page_size,
                       int32_t max_pages_per_seq, int32_t num_pages, int32_t max_context_len,
                       int32_t num_partitions, float scale, const float* attn_sink,
                       void* workspace, hipStream_t stream) {
  DecodeWs ws = decode_ws_layout((char*)workspace, batch_size, num_heads, max_context_len,
                                 page_size, num_partitions, cache_dtype);
  const bool fp8 = cache_dtype == MLA_FP8_E4M3FN;
  mla::PrefixArgs pa;
  pa.cum = ws.cum;
  pa.ctx = context_lengths;
  pa.add = add;
  pa.B = batch_size;
  pa.max_ctx = (uint32_t)max_context_len;
  pa.wstart = ws.wstart;
  pa.wspan = ws.wspan;
  pa.wfirst = ws.wfirst;
  pa.G = ws.G;
  int st = hip_status(mla::launch_decode_absorb(ws.q_abs, (const uint16_t*)q,
                                                (const uint16_t*)w_uk, batch_size, num_heads, pa,
                                                stream),
                      "absorb kernel");
  if (st != MLA_OK) return st;
  mla::DecodeArgs a;
  a.q_abs = (const uint16_t*)ws.q_abs;
  a.cache = kv_cache;
  a.page_table = page_table;
  a.cum = ws.cum;
  a.wstart = ws.wstart;
  a.wfirst = ws.wfirst;
  a.part_o = ws.part_o;
  a.part_ml = ws.part_ml;
  a.B = batch_size;
  a.H = num_heads;
  a.ps = page_size;
  a.maxp = max_pages_per_seq;
  a.num_pages = num_pages;
  a.G = ws.G;
  a.scale_log2 = scale * kLog2e;
  st = hip_status(mla::launch_decode_split(a, fp8, stream), "split-KV kernel");
  if (st != MLA_OK) return st;
  mla::CombineArgs c;
  c.o_lat = ws.o_lat;
  c.part_o = ws.part_o;
  c.part_ml = ws.part_ml;
  c.cum = ws.cum;
  c.wstart = ws.wstart;
  c.wspan = ws.wspan;
  c.q_abs = (const uint16_t*)ws.q_abs;
  c.cache = kv_cache;
  c.page_table = page_table;
  c.B = batch_size;
  c.H = num_heads;
  c.G = ws.G;
  c.ps = page_size;
  c.maxp = max_pages_per_seq;
  c.num_pages = num_pages;
  c.scale_log2 = scale * kLog2e;
  c.sink = attn_sink;
  c.fp8 = fp8;
  st = hip_status(mla::launch_decode_combine(c, stream), "combine kernel");
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_decode_project((uint16_t*)output, ws.o_lat,
                                               (const uint16_t*)w_uv, batch_size, num_heads,
                                               stream),
                    "projection kernel");
}

size_t mla_decode_sparse_workspace_size(int32_t batch_size, int32_t num_heads, int32_t max_topk,
                                        int32_t num_partitions, int32_t cache_dtype) {
  return mla_decode_workspace_size(batch_size, num_heads, max_topk, 1, num_partitions,
                                   cache_dtype);
}

// The listed rows are a paged context with one row per page: the index list
// is the page table, the pool's rows its pages.
int mla_decode_sparse(void* output, const void* q, const int32_t* topk_lengths,
                      const void* kv_cache, int32_t cache_dtype, const int32_t* d_indices,
                      int32_t indices_stride, const void* w_uk, const void* w_uv,
                      int32_t batch_size, int32_t num_heads, int32_t num_rows, int32_t max_topk,
                      int32_t num_partitions, float scale, const float* attn_sink,
                      void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (!topk_lengths || !d_indices) return fail(MLA_ERR_INVALID_ARG, "mla_decode_sparse: null pointer");
  if (indices_stride < 1 || num_rows < 1 || max_topk < 1 || max_topk > indices_stride)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_sparse: indices_stride=%d num_rows=%d max_topk=%d",
                indices_stride, num_rows, max_topk);
  return mla_decode(output, q, (const uint32_t*)topk_lengths, kv_cache, cache_dtype, d_indices,
                    w_uk, w_uv, batch_size, num_heads, 1, indices_stride, num_rows,
                    max_topk, num_partitions, scale, attn_sink, workspace,
                    workspace_bytes, stream);
}

size_t mla_prefill_decode_workspace_size(int32_t batch_size, int32_t total_q,
                                         int32_t num_heads, int32_t max_seq_len,
                                         int32_t max_rows, int32_t max_cache_len,
                                         int32_t page_size, int32_t indices_stride,
                                         int32_t num_partitions, int32_t cache_dtype) {
  if (batch_size < 1 || total_q < 0 || num_heads < 1 || max_seq_len < 0 || max_cache_len < 0 ||
      page_size < 1 || indices_stride < 0 || num_partitions < 0 || !dtype_ok(cache_dtype))
    return 0;
  if (max_seq_len == 0) return kAlign;  // nothing runs; 0 stays the error value
  if (max_seq_len > 1)
    return mla_prefill_workspace_size(batch_size, total_q, num_heads, max_rows, MLA_BF16);
  if (indices_stride > 0)
    return mla_decode_sparse_workspace_size(batch_size, num_heads, indices_stride,
                                            num_partitions, cache_dtype);
  if (max_cache_len >= INT32_MAX) return 0;
  return mla_decode_workspace_size(batch_size, num_heads, max_cache_len + 1, page_size,
                                   num_partitions, cache_dtype);
}

int mla_prefill_decode(void* output, const void* q, const void* kv_input,
                       const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                       void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                       const uint32_t* buffer_row_offsets, const uint32_t* cache_offsets,
                       const int32_t* buffer_lengths, int32_t max_chunks, int32_t max_rows,
                       const void* w_k, const void* w_uk, const void* w_uv,
                       const void* kv_norm_gamma, const void* freqs_cis, int32_t batch_size,
                       int32_t total_q, int32_t num_heads, int32_t max_seq_len,
                       int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                       int32_t max_cache_len, int32_t freqs_len, float scale, float epsilon,
                       const int32_t* d_indices, int32_t indices_stride,
                       const int32_t* topk_lengths, const float* attn_sink,
                       int32_t num_partitions, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  const char* who = "mla_prefill_decode";
  // every check comes before the first launch
  if (!input_row_offsets || !cache_lengths || !kv_cache || !page_table)
    return fail(MLA_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!dtype_ok(cache_dtype)) return fail(MLA_ERR_UNSUPPORTED, "%s: cache dtype", who);
  if (batch_size < 1 || total_q < 0 || num_heads < 1 || max_seq_len < 0 || page_size < 1 ||
      max_pages_per_seq < 1 || num_pages < 1 || max_cache_len < 0 || freqs_len < 1 ||
      num_partitions < 0 || num_partitions > 65536 || !(scale > 0.f) || !(epsilon >= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "%s: sizes", who);
  if ((max_seq_len == 0) != (total_q == 0))
    return fail(MLA_ERR_INVALID_ARG, "%s: max_seq_len=%d with total_q=%d", who, max_seq_len,
                total_q);
  if ((uint64_t)num_pages * (uint64_t)page_size >= (1ull << 31))
    return fail(MLA_ERR_INVALID_ARG, "%s: num_pages * page_size must be < 2^31", who);
  if (kv_input) {
    if (!kv_norm_gamma || !freqs_cis) return fail(MLA_ERR_INVALID_ARG, "%s: null pointer", who);
    if (misaligned({kv_cache, kv_input, kv_norm_gamma, freqs_cis}))
      return fail(MLA_ERR_INVALID_ARG, "%s: tensor not 16-byte aligned", who);
  }
  const bool sparse = d_indices != nullptr;
  const int32_t num_rows = num_pages * page_size;
  if (max_seq_len > 1) {
    if (!output || !q || !buffer_row_offsets || !cache_offsets || !buffer_lengths || !w_k ||
        !w_uv)
      return fail(MLA_ERR_INVALID_ARG, "%s: null pointer (prefill)", who);
    if (misaligned({output, q, kv_cache, w_k, w_uv, workspace}))
      return fail(MLA_ERR_INVALID_ARG, "%s: tensor not 16-byte aligned", who);
    if (num_heads > 1024 || max_chunks < 1 || max_rows < 1)
      return fail(MLA_ERR_INVALID_ARG, "%s: sizes (prefill)", who);
  } else if (max_seq_len == 1) {
    if (!output || !q || !w_uk || !w_uv)
      return fail(MLA_ERR_INVALID_ARG, "%s: null pointer (decode)", who);
    if (misaligned({output, q, kv_cache, w_uk, w_uv, workspace}))
      return fail(MLA_ERR_INVALID_ARG, "%s: tensor not 16-byte aligned", who);
    if (num_heads > 128) return fail(MLA_ERR_INVALID_ARG, "%s: num_heads must be 1..128", who);
    if (total_q != batch_size)
      return fail(MLA_ERR_INVALID_ARG,
                  "%s: decode takes one new token per sequence (total_q=%d, batch_size=%d)",
                  who, total_q, batch_size);
    if (sparse) {
      if (!topk_lengths || indices_stride < 1)
        return fail(MLA_ERR_INVALID_ARG, "%s: sparse decode needs topk_lengths and "
                    "indices_stride >= 1", who);
      if ((uint64_t)batch_size * (uint64_t)indices_stride >= (1ull << 31))
        return fail(MLA_ERR_INVALID_ARG, "%s: batch_size * indices_stride must be < 2^31", who);
    } else if ((uint64_t)batch_size * ((uint64_t)max_cache_len + 1) >= (1ull << 31)) {
      return fail(MLA_ERR_INVALID_ARG, "%s: batch_size * (max_cache_len + 1) must be < 2^31",
                  who);
    }
  }
  const size_t need = mla_prefill_decode_workspace_size(
      batch_size, total_q, num_heads, max_seq_len, max_rows, max_cache_len, page_size,
      sparse ? indices_stride : 0, num_partitions, cache_dtype);
  if (max_seq_len > 0 && (!workspace || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "%s: workspace %zu < %zu", who, workspace_bytes, need);

  if (kv_input) {
    const int st = kv_write_rows(kv_cache, cache_dtype, page_table, kv_input, input_row_offsets,
                                 cache_lengths, kv_norm_gamma, freqs_cis, batch_size, total_q,
                                 page_size, max_pages_per_seq, num_pages, freqs_len, epsilon,
                                 stream);
    if (st != MLA_OK) return st;
  }
  if (max_seq_len > 1) {
    const int32_t rows = (max_rows + 63) / 64 * 64;
    return prefill_chunks(output, q, MLA_BF16, input_row_offsets, cache_lengths, kv_cache,
                          cache_dtype, true, page_table, buffer_row_offsets, cache_offsets,
                          buffer_lengths, max_chunks, rows, w_k, w_uv, kv_norm_gamma, freqs_cis,
                          batch_size, total_q, num_heads, page_size, max_pages_per_seq,
                          num_pages, freqs_len, scale, epsilon, attn_sink, workspace, stream);
  }
  if (max_seq_len == 1) {
    if (sparse)  // the listed rows as a paged context of one row per page
      return decode_body(output, q, (const uint32_t*)topk_lengths, 0, kv_cache, cache_dtype,
                         d_indices, w_uk, w_uv, batch_size, num_heads, 1, indices_stride,
                         num_rows, indices_stride, num_partitions, scale, attn_sink, workspace,
                         stream);
    return decode_body(output, q, cache_lengths, 1, kv_cache, cache_dtype, page_table, w_uk,
                       w_uv, batch_size, num_heads, page_size, max_pages_per_seq, num_pages,
                       max_cache_len + 1, num_partitions, scale, attn_sink, workspace, stream);
  }
  return MLA_OK;
}

}  // extern "C"
