/*
 * mla.h -- C ABI of libmla.so: MLA chunked prefill and absorbed decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow three Modular MAX kernel-library API pages:
 *   "mla_prefill_plan"              (chunk planner: description and Args),
 *   "mla_prefill_decode_graph_bf16" (latent gather, RMSNorm, RoPE,
 *                                    up-projection with w_k / w_uv, absorbed
 *                                    decode with w_uk / w_uv: description,
 *                                    Parameters and Args),
 *   "flare_mla_prefill_dispatch"    (prefill attention: q_depth 192 = 128 nope
 *                                    + 64 rope, one rope head shared by all
 *                                    query heads, cache_depth 576, bf16 or
 *                                    float8_e4m3fn inputs with bf16 output).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Dimensions are fixed to DeepSeek V2/V3 MLA: qk_nope 128, qk_rope 64,
 *   v_head 128, kv_lora_rank 512, cache row 576 = 512 latent + 64 rope.
 *   num_heads is a runtime argument (1..1024).
 * - Every pointer argument is a DEVICE pointer owned by the caller (for
 *   example memory allocated through torch). The library never allocates,
 *   frees or keeps device memory; scratch space comes from a caller-provided
 *   workspace whose size the matching *_workspace_size function returns.
 * - Every call is asynchronous on the caller's stream and never synchronises
 *   the host, so a sequence of calls can be captured into a HIP graph.
 *   Device-resident plan values (buffer_lengths) are read on the device.
 * - All tensors are dense, row-major and contiguous in the shapes given.
 *   Tensor pointers (activations, caches, weights, outputs, workspaces; not
 *   the small per-sequence offset, length and page-table arrays) must be
 *   16-byte aligned, as device allocations are; a misaligned one is
 *   MLA_ERR_INVALID_ARG.
 *   "bf16" is bfloat16, "e4m3" is OCP float8_e4m3fn (1-4-3, bias 7, no
 *   infinities), each passed as raw storage.
 * - Attention sinks ("mla_prefill_decode_graph_bf16" page, Args
 *   "attn_sink_ptr", an optional float32 sink per batch entry): the
 *   attention entry points take attn_sink, float32 [batch_size] or null. A
 *   sequence's sink is one more logit, in the units of the scaled scores, in
 *   the softmax denominator with a zero value vector: weights become
 *   e^s_j / (sum_k e^s_k + e^sink_b). Null means no sink.
 * - Every function returns MLA_OK (0) or a negative status. Host-checkable
 *   problems (null pointers, sizes out of range, unsupported dtypes, a
 *   workspace that is too small) are reported before anything is enqueued.
 *   Data-dependent preconditions on device values (page ids inside the pool,
 *   positions inside the RoPE table, max_chunks large enough for the batch)
 *   cannot be checked without a synchronisation: kernels clamp or skip
 *   offending rows so that they never read out of bounds, and the results for
 *   such rows are unspecified.
 *   mla_last_error() returns a message for the last failure on the calling
 *   thread.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1) /* null pointer, size out of range           */
#define MLA_ERR_UNSUPPORTED (-2) /* dtype other than bf16 / e4m3 where allowed */
#define MLA_ERR_WORKSPACE (-3)   /* workspace pointer null or too small        */
#define MLA_ERR_HIP (-4)         /* a kernel launch failed                     */

/* storage dtypes */
#define MLA_BF16 0
#define MLA_FP8_E4M3FN 1

/* fixed MLA dimensions */
#define MLA_QK_NOPE 128
#define MLA_QK_ROPE 64
#define MLA_Q_DEPTH 192
#define MLA_V_DEPTH 128
#define MLA_KV_LORA 512
#define MLA_CACHE_DEPTH 576

/*
 * mla_prefill_plan -- split every sequence's cached-plus-new tokens into
 * chunks of at most buffer_token_size tokens per sequence
 * ("mla_prefill_plan" page, description and Args).
 *
 * Sequence b holds L_b = (input_row_offsets[b+1] - input_row_offsets[b]) +
 * cache_lengths[b] tokens, cached ones first. Chunk c takes
 *   len(c, b) = clamp(L_b - c*T, 0, T) tokens starting at position
 *   cache_offsets[c, b] = min(c*T, L_b),
 * packed sequence after sequence in the chunk's contiguous buffer:
 *   buffer_row_offsets[c, 0] = 0, buffer_row_offsets[c, b+1] =
 *   buffer_row_offsets[c, b] + len(c, b),
 *   buffer_lengths[c] = buffer_row_offsets[c, B], or -1 when that is 0
 *   (an unused chunk). Every element of every chunk row is written.
 *
 * Outputs (device):
 *   buffer_row_offsets  uint32 [max_chunks, batch_size + 1]
 *   cache_offsets       uint32 [max_chunks, batch_size]
 *   buffer_lengths      int32  [max_chunks]
 *   chunks_needed       uint32 [1] or NULL: ceil(max_b L_b / T), so the caller
 *                       can check later that max_chunks was large enough.
 * Inputs (device):
 *   input_row_offsets   uint32 [batch_size + 1], cumulative new-token offsets
 *   cache_lengths       uint32 [batch_size], cached tokens per sequence
 * Host scalars: batch_size >= 1, max_chunks >= 1, buffer_token_size >= 1,
 *   batch_size * buffer_token_size < 2^31.
 */
int mla_prefill_plan(uint32_t* buffer_row_offsets, uint32_t* cache_offsets,
                     int32_t* buffer_lengths, uint32_t* chunks_needed,
                     const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                     int32_t batch_size, int32_t max_chunks, uint32_t buffer_token_size,
                     hipStream_t stream);

/*
 * mla_gather_norm_rope -- gather one chunk's raw cache rows from the paged
 * pool, RMSNorm the 512-wide latent with kv_norm_gamma and rotate the 64-wide
 * rope part with freqs_cis ("mla_prefill_decode_graph_bf16" page: Parameters
 * "kv_input_fn"; Args "kv_norm_gamma", "epsilon", "freqs_cis",
 * "buffer_row_offsets", "cache_offsets").
 *
 * For every row r < *buffer_length_c of sequence b (buffer_row_offsets_c[b]
 * <= r < buffer_row_offsets_c[b+1]) at position p = cache_offsets_c[b] +
 * (r - buffer_row_offsets_c[b]), the pool row is
 *   kv_cache[page_table[b, p / page_size], p % page_size, :]   (576 values)
 *   latent_out[r, l] = x_l * gamma_l / sqrt(mean(x^2) + epsilon), x = row[0:512]
 *   krope_out[r, 2i]   = y_2i F_2i - y_2i+1 F_2i+1,   y = row[512:576],
 *   krope_out[r, 2i+1] = y_2i F_2i+1 + y_2i+1 F_2i,   F = freqs_cis[p, :].
 * Arithmetic is fp32; outputs are rounded to bf16 (krope to e4m3 when
 * krope_dtype is MLA_FP8_E4M3FN, saturating at 448).
 *
 *   latent_out    bf16 [max_rows, 512]           (device, written)
 *   krope_out     bf16 or e4m3 [max_rows, 64]    (device, written)
 *   kv_cache      bf16 or e4m3 [num_pages, page_size, 576] (cache_dtype)
 *   page_table    int32 [batch_size, max_pages_per_seq]
 *   buffer_row_offsets_c uint32 [batch_size + 1]  one chunk's plan row
 *   cache_offsets_c      uint32 [batch_size]
 *   buffer_length_c      int32 [1]  rows in this chunk; -1 makes the call a no-op
 *   kv_norm_gamma bf16 [512];  freqs_cis bf16 [max_seq_len, 64]
 * Rows whose page id or position is out of range are written as zeros.
 */
int mla_gather_norm_rope(void* latent_out, void* krope_out, int32_t krope_dtype,
                         const void* kv_cache, int32_t cache_dtype,
                         const int32_t* page_table,
                         const uint32_t* buffer_row_offsets_c,
                         const uint32_t* cache_offsets_c,
                         const int32_t* buffer_length_c,
                         const void* kv_norm_gamma, const void* freqs_cis,
                         int32_t batch_size, int32_t page_size, int32_t max_pages_per_seq,
                         int32_t num_pages, int32_t max_rows, int32_t max_seq_len,
                         float epsilon, hipStream_t stream);

/*
 * mla_kv_write -- store the new tokens' latent rows in the paged cache,
 * normalised and rotated ("mla_prefill_decode_graph_bf16" page: Parameters
 * "kv_input_fn", the new tokens' raw latent [tot_seq_len, 576]; Args
 * "kv_norm_gamma", "epsilon", "freqs_cis", "input_row_offsets" and the paged
 * KV cache). This is the state decode reads: rows as stored.
 *
 * Token t of sequence b (input_row_offsets[b] <= t < input_row_offsets[b+1])
 * sits at position p = cache_lengths[b] + (t - input_row_offsets[b]); with
 * x = kv_input[t, 0:512], y = kv_input[t, 512:576], F = freqs_cis[p, :]:
 *   kv_cache[page_table[b, p / page_size], p % page_size, l]       = x_l * gamma_l / sqrt(mean(x^2) + epsilon)
 *   kv_cache[page_table[b, p / page_size], p % page_size, 512 + 2i] = y_2i F_2i - y_2i+1 F_2i+1
 *   kv_cache[...,                                          512 + 2i+1] = y_2i F_2i+1 + y_2i+1 F_2i
 * Arithmetic is fp32; the stored values are rounded to bf16, or to e4m3
 * (nearest even, saturating at 448) when cache_dtype is MLA_FP8_E4M3FN.
 *
 *   kv_cache      bf16 or e4m3 [num_pages, page_size, 576] (device, written)
 *   page_table    int32 [batch_size, max_pages_per_seq]
 *   kv_input      bf16 [total_tokens, 576]
 *   input_row_offsets uint32 [batch_size + 1]; cache_lengths uint32 [batch_size]
 *   kv_norm_gamma bf16 [512];  freqs_cis bf16 [max_seq_len, 64]
 * Only the new tokens' slots are written. Tokens whose logical page is past
 * max_pages_per_seq, whose page id is outside [0, num_pages) or whose position
 * is not below max_seq_len are skipped. Two tokens mapping to one slot (a
 * page table that repeats a page) race.
 */
int mla_kv_write(void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                 const void* kv_input, const uint32_t* input_row_offsets,
                 const uint32_t* cache_lengths, const void* kv_norm_gamma, const void* freqs_cis,
                 int32_t batch_size, int32_t total_tokens, int32_t page_size,
                 int32_t max_pages_per_seq, int32_t num_pages, int32_t max_seq_len, float epsilon,
                 hipStream_t stream);

/*
 * mla_up_project -- K_nope and V from the normalised latent
 * ("mla_prefill_decode_graph_bf16" page, Args "w_k" and "w_uv"):
 *   K_nope[r, h, d] = sum_l w_k[h*128 + d, l] latent[r, l]
 *   V[r, h, d]      = sum_l w_uv[h, d, l]     latent[r, l]
 * for r < *buffer_length_c; bf16 MFMA with fp32 accumulation. Rows from
 * *buffer_length_c up to the next multiple of 64 are written as zeros (the
 * attention's last key tile of a chunk reads them, masked).
 *
 * Output layouts are the ones the attention kernel streams:
 *   k_nope_out  [num_heads, max_rows, 128], bf16 or e4m3 (k_dtype)
 *   v_t_out     [num_heads, 128, max_rows], bf16: V transposed per head
 * Inputs: latent bf16 [max_rows, 512]; w_k bf16 [num_heads*128, 512];
 *   w_uv bf16 [num_heads, 128, 512]; buffer_length_c int32 [1] (-1: no-op).
 * max_rows must be a multiple of 64 (the row stride of both outputs).
 */
int mla_up_project(void* k_nope_out, void* v_t_out, int32_t k_dtype,
                   const void* latent, const void* w_k, const void* w_uv,
                   const int32_t* buffer_length_c, int32_t num_heads, int32_t max_rows,
                   hipStream_t stream);

/*
 * mla_prefill_attention_workspace_size / mla_prefill_attention -- one chunk of
 * causal MLA prefill attention ("flare_mla_prefill_dispatch" page: Args q,
 * k, v, k_rope, valid_length, max_prompt_len, scale, cache_offsets;
 * Parameters kv_num_heads = 1 for the rope part, q_depth 192).
 *
 * Query i of sequence b (token t = input_row_offsets[b] + i) sits at absolute
 * position P = cache_lengths[b] + i and sees the keys of this chunk at
 * positions p = cache_offsets_c[b] + j <= P, j < len(b). Its score is
 *   s = scale * (q[t, h, 0:128] . K_nope[r, h, :] + q[t, h, 128:192] . krope[r, :])
 * with r = buffer_row_offsets_c[b] + j; krope has one head shared by all query
 * heads. Softmax state (running max, sum, unnormalised output) is carried
 * across the chunks of a sequence in the workspace; a query's output
 *   output[t, h, :] = sum_p softmax(s)_p V[p, h, :]
 * is written (bf16) in the chunk that holds its last visible key. Chunks must
 * be issued in order and each sequence's keys must appear in increasing,
 * contiguous position ranges, as mla_prefill_plan produces them.
 *
 *   output   bf16 [total_q, num_heads, 128]                  (written)
 *   q        bf16 or e4m3 (dtype) [total_q, num_heads, 192]  nope first
 *   k_nope   [num_heads, max_rows, 128]  bf16, or e4m3 when dtype is e4m3
 *   v_t      bf16 [num_heads, 128, max_rows]
 *   krope    [max_rows, 64]  bf16, or e4m3 when dtype is e4m3
 *   input_row_offsets uint32 [B+1]; cache_lengths uint32 [B]
 *   buffer_row_offsets_c uint32 [B+1]; cache_offsets_c uint32 [B];
 *   buffer_length_c int32 [1] (-1: no-op)
 *   max_prompt_len: host upper bound on the new tokens of any sequence
 *   workspace: mla_prefill_attention_workspace_size(...) bytes, holding the
 *   carried softmax state and the query-block schedule. A sequence's carry is
 *   read only when cache_offsets_c[b] > 0, i.e. when earlier chunks held its
 *   first keys, so no reset is needed between prefills.
 */
size_t mla_prefill_attention_workspace_size(int32_t batch_size, int32_t total_q,
                                            int32_t num_heads);
int mla_prefill_attention(void* output, const void* q, int32_t dtype,
                          const void* k_nope, const void* v_t, const void* krope,
                          const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                          const uint32_t* buffer_row_offsets_c,
                          const uint32_t* cache_offsets_c,
                          const int32_t* buffer_length_c,
                          int32_t batch_size, int32_t total_q, int32_t num_heads,
                          int32_t max_rows, int32_t max_prompt_len, float scale,
                          const float* attn_sink, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * mla_prefill_workspace_size / mla_prefill -- the whole chunked prefill for a
 * planned batch: for every chunk c < max_chunks (in order) gather + RMSNorm +
 * RoPE, up-projection, and attention with the carried softmax state
 * ("mla_prefill_decode_graph_bf16" page, prefill branch, called once per
 * chunk with that chunk's plan row). Chunks with buffer_lengths[c] == -1 are
 * skipped on the device.
 *
 *   output        bf16 [total_q, num_heads, 128]
 *   q             bf16 or e4m3 (dtype) [total_q, num_heads, 192]
 *   kv_cache      [num_pages, page_size, 576] raw latent + raw rope rows,
 *                 same dtype as q
 *   page_table    int32 [batch_size, max_pages_per_seq]
 *   buffer_row_offsets uint32 [max_chunks, B+1]; cache_offsets uint32
 *                 [max_chunks, B]; buffer_lengths int32 [max_chunks]  (the plan)
 *   w_k bf16 [num_heads*128, 512]; w_uv bf16 [num_heads, 128, 512]
 *   kv_norm_gamma bf16 [512]; freqs_cis bf16 [max_seq_len, 64]
 *   max_rows: host upper bound on every buffer_lengths[c] (B * T always is)
 * With dtype MLA_FP8_E4M3FN the scores are computed from e4m3 q, K_nope and
 * krope on fp8 MFMA, and the value product in bf16.
 */
size_t mla_prefill_workspace_size(int32_t batch_size, int32_t total_q, int32_t num_heads,
                                  int32_t max_rows, int32_t dtype);
int mla_prefill(void* output, const void* q, int32_t dtype,
                const uint32_t* input_row_offsets, const uint32_t* cache_lengths,
                const void* kv_cache, const int32_t* page_table,
                const uint32_t* buffer_row_offsets, const uint32_t* cache_offsets,
                const int32_t* buffer_lengths, int32_t max_chunks, int32_t max_rows,
                const void* w_k, const void* w_uv, const void* kv_norm_gamma,
                const void* freqs_cis, int32_t batch_size, int32_t total_q,
                int32_t num_heads, int32_t max_prompt_len, int32_t page_size,
                int32_t max_pages_per_seq, int32_t num_pages, int32_t max_seq_len,
                float scale, float epsilon, const float* attn_sink, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * mla_decode_workspace_size / mla_decode -- absorbed MLA decode, one new token
 * per sequence ("mla_prefill_decode_graph_bf16" page, decode branch and Args
 * "w_uk", "w_uv", "num_partitions_in"; "flare_mla_prefill_dispatch" page:
 * kv_num_heads 1, cache_depth 576):
 *   q_lat[b, h, :] = w_uk[h] (512x128) . q[b, h, 0:128]
 *   s_p = scale * (q_lat . Z_p[0:512] + q[b, h, 128:192] . Z_p[512:576])
 *   o_lat = sum_p softmax(s)_p Z_p[0:512];  output[b, h, :] = w_uv[h] (128x512) . o_lat
 * over the rows Z_p, p < context_lengths[b], of sequence b as stored in the
 * pool (already normalised and rotated).
 *
 * Split-KV: the batch's contexts are laid end to end and cut into
 * num_partitions equal key ranges, one workgroup each (0 = one per compute
 * unit); ranges that span sequences produce one partial state per sequence,
 * merged by log-sum-exp. The library raises the count when a range would span
 * more than 1022 pages. The workspace size depends on all of its arguments.
 *
 *   output     bf16 [batch_size, num_heads, 128]
 *   q          bf16 [batch_size, num_heads, 192]
 *   context_lengths uint32 [batch_size]  (includes the new token; 0 gives zeros)
 *   kv_cache   bf16 or e4m3 (cache_dtype) [num_pages, page_size, 576]
 *   page_table int32 [batch_size, max_pages_per_seq]
 *   w_uk bf16 [num_heads, 512, 128]; w_uv bf16 [num_heads, 128, 512]
 *   max_context_len: host upper bound on every context length (a longer
 *   device value counts as max_context_len; its result is unspecified)
 *   Limits: num_heads <= 128; batch_size * max_context_len < 2^31;
 *   num_pages * page_size < 2^31.
 * With an e4m3 cache both products run on fp8 MFMA: the absorbed query is
 * quantised per (sequence, head) to e4m3 under a power-of-two scale folded
 * into the score scale, and the probabilities are e4m3 values 2^(s - m + 7)
 * against a running maximum m per head (raised, with the partial output
 * rescaled, whenever a tile's scores exceed it by more than 1.5 log2 units).
 */
size_t mla_decode_workspace_size(int32_t batch_size, int32_t num_heads,
                                 int32_t max_context_len, int32_t page_size,
                                 int32_t num_partitions, int32_t cache_dtype);
int mla_decode(void* output, const void* q, const uint32_t* context_lengths,
               const void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
               const void* w_uk, const void* w_uv, int32_t batch_size, int32_t num_heads,
               int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
               int32_t max_context_len, int32_t num_partitions, float scale,
               const float* attn_sink, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation with the same kernels, its
 * workspace taken from a scratch array built into the library instead of a
 * caller buffer. The call allocates nothing; the caller still passes every
 * input and the output.
 *
 * The scratch array holds MLA_NOALLOC_SCRATCH_BYTES (128 MiB); every GPU the
 * library runs on holds its own copy until the process ends. A decode whose
 * workspace (mla_decode_workspace_size with the same arguments) exceeds it
 * is rejected with MLA_ERR_WORKSPACE before anything is enqueued; decode_b64's
 * shape (64 sequences, 128 heads, contexts to 32k, one partition per compute
 * unit) needs about 65 MiB. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give unspecified results. Nothing in
 * the array has to start at zero; a call leaves its contents behind. The
 * first call on a device looks up the array's device address (no
 * allocation); make it outside graph capture.
 * Arguments, limits and errors: as mla_decode, without workspace and
 * workspace_bytes.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
int mla_decode_noalloc(void* output, const void* q, const uint32_t* context_lengths,
                       const void* kv_cache, int32_t cache_dtype, const int32_t* page_table,
                       const void* w_uk, const void* w_uv, int32_t batch_size, int32_t num_heads,
                       int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                       int32_t max_context_len, int32_t num_partitions, float scale,
                       const float* attn_sink, hipStream_t stream);

/*
 * mla_hbm_read -- measurement helper, not part of the attention path: reads
 * `bytes` (a multiple of 16, src 16-byte aligned) once with streaming 16-byte
 * loads from `groups` workgroups of 256 threads and stores one XOR word per
 * workgroup into out (uint32 [groups], device). Timing it gives the practical
 * HBM read rate that the decode and gather rates are compared with.
 */
int mla_hbm_read(const void* src, size_t bytes, uint32_t* out, int32_t groups,
                 hipStream_t stream);

/* Text for a status code, and the message of the calling thread's last failure. */
const char* mla_status_string(int status);
const char* mla_last_error(void);

/*
 * mla_decode_sparse_workspace_size / mla_decode_sparse -- absorbed decode of
 * one new token per sequence over an explicit list of cache rows
 * ("mla_prefill_decode_graph_bf16" page: Parameters "sparse_mla",
 * "sparse_indices_stride"; Args "d_indices", "indices_stride",
 * "topk_lengths").
 *
 * Sequence b attends over the pool rows d_indices[b * indices_stride + j],
 * j < topk_lengths[b], exactly as mla_decode attends over a context (rows used
 * as stored; a row is page * page_size + slot of the pool viewed as
 * [num_rows, 576]). Rows may repeat (a repeated row counts twice). A sequence
 * that lists no row outputs zeros.
 *
 *   output       bf16 [batch_size, num_heads, 128]   (device, written)
 *   q            bf16 [batch_size, num_heads, 192]
 *   topk_lengths int32 [batch_size], each in [0, max_topk]
 *   kv_cache     bf16 or e4m3 [num_rows, 576] (cache_dtype)
 *   d_indices    int32 [batch_size, indices_stride], each in [0, num_rows)
 *   w_uk, w_uv, num_heads, num_partitions, scale: as mla_decode.
 * max_topk <= indices_stride. The workspace holds at least
 * mla_decode_sparse_workspace_size(batch_size, num_heads, max_topk,
 * num_partitions, cache_dtype) bytes. Lengths above max_topk count as
 * max_topk; indices outside [0, num_rows) read row 0; the results of such
 * sequences are unspecified.
 */
size_t mla_decode_sparse_workspace_size(int32_t batch_size, int32_t num_heads, int32_t max_topk,
                                        int32_t num_partitions, int32_t cache_dtype);
int mla_decode_sparse(void* output, const void* q, const int32_t* topk_lengths,
                      const void* kv_cache, int32_t cache_dtype, const int32_t* d_indices,
                      int32_t indices_stride, const void* w_uk, const void* w_uv,
                      int32_t batch_size, int32_t num_heads, int32_t num_rows, int32_t max_topk,
                      int32_t num_partitions, float scale, const float* attn_sink,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_prefill_decode_workspace_size / mla_prefill_decode -- the graph op as
 * one call ("mla_prefill_decode_graph_bf16" page: description, prefill or
 * decode chosen by the batch's maximum sequence length; Parameters
 * "kv_input_fn", "sparse_mla"; Args "max_seq_len", "d_indices",
 * "indices_stride", "topk_lengths", "attn_sink_ptr", "num_partitions_in").
 *
 * Steps, in stream order:
 *  1. kv_input not null: the new tokens' raw rows are stored normalised and
 *     rotated in their paged slots (mla_kv_write with total_q tokens and
 *     freqs_len table rows).
 *  2. max_seq_len > 1 -- prefill: the planned chunk loop of mla_prefill, but
 *     every pool row (cached and new) is read as stored, already normalised
 *     and rotated, the form step 1 writes; gamma and freqs_cis are not read
 *     by this step. q is bf16.
 *     max_seq_len == 1 -- decode: every sequence brings exactly one token
 *     (total_q must equal batch_size); q row b attends over the sequence's
 *     cache_lengths[b] + 1 rows (the cached ones and the new one) as
 *     mla_decode does, or, when d_indices is not null, over its listed rows
 *     as mla_decode_sparse does (max_topk = indices_stride, the pool viewed
 *     as num_pages * page_size rows).
 *     max_seq_len == 0 -- no query (total_q must be 0); only step 1 runs.
 *
 *   max_seq_len: host value, the largest number of new tokens of any
 *     sequence in the batch; it picks the branch.
 *   max_cache_len: host upper bound on every cache_lengths[b] (decode).
 *   buffer_row_offsets, cache_offsets, buffer_lengths, max_chunks, max_rows:
 *     the plan, as mla_prefill (prefill only; may be null for decode).
 *   w_k (prefill), w_uk (decode), w_uv (both); kv_norm_gamma and freqs_cis
 *     [freqs_len, 64] are read only by step 1.
 *   d_indices, indices_stride, topk_lengths: sparse decode, or null / 0.
 *   attn_sink: float32 [batch_size] or null, in either branch.
 *   num_partitions: split-KV workgroups of the decode branch, 0 = one per
 *     compute unit. It and every grid are host values, so the call can be
 *     captured into a HIP graph and replayed with new device data.
 * Other arguments as mla_kv_write, mla_prefill and mla_decode. The workspace
 * holds at least mla_prefill_decode_workspace_size(...) bytes for the branch
 * max_seq_len selects (indices_stride 0 for dense decode).
 */
size_t mla_prefill_decode_workspace_size(int32_t batch_size, int32_t total_q,
                                         int32_t num_heads, int32_t max_seq_len,
                                         int32_t max_rows, int32_t max_cache_len,
                                         int32_t page_size, int32_t indices_stride,
                                         int32_t num_partitions, int32_t cache_dtype);
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
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
