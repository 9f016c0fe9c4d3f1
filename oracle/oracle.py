"""NumPy fp64 oracle for MLA chunked prefill and absorbed decode.

TEST INFRASTRUCTURE. Only tests/, the smoke check and the benchmark's CPU
baseline call this module. It shares no code with the HIP path.

Every input is decoded exactly from its storage bits (bf16 or float8_e4m3fn) to
float64, and nothing is rounded afterwards. Computations follow the plain
definitions: per-sequence loops, a materialised masked score matrix, a full
(not online) softmax. Library matrix products serve as steps; there is no
blocking or fusion beyond what the definitions state.

Sources, all Modular MAX kernel-library API pages:
- "mla_prefill_plan": description (chunks of buffer_token_size, per-chunk
  buffer offsets, cache offsets and buffer lengths) and Args.
- "mla_prefill_decode_graph_bf16": description (prefill or decode by the
  batch's maximum sequence length), Parameters (kv_input_fn: 576 = 512 latent
  + 64 rope per cache row) and Args (q, freqs_cis, kv_norm_gamma, scale,
  epsilon, w_k, w_uk, w_uv, buffer_row_offsets, cache_offsets).
- "flare_mla_prefill_dispatch": Parameters (kv_num_heads = 1, q_depth 192 =
  128 nope + 64 rope, cache_depth 576, dtype bfloat16 or float8_e4m3fn,
  output_type bfloat16) and Args (k_rope shared by all heads, valid_length,
  scale, cache_offsets).

Readings where the pages leave a step open (each is listed in the design notes):
- Chunks cap the tokens of each sequence: chunk c holds positions
  [c*T, min((c+1)*T, L_b)) of sequence b (mla_prefill_plan page, Args
  "buffer_token_size", read as a per-sequence cap on a chunk's tokens).
- cache_offsets of a sequence with no rows in a chunk is min(c*T, L_b); unused
  chunks are written in full with buffer_lengths = -1.
- RoPE rotates adjacent pairs (2i, 2i+1) by the complex number whose real and
  imaginary parts are freqs_cis[p, 2i] and freqs_cis[p, 2i+1].
- Prefill reads raw cache rows; RMSNorm and RoPE apply to every gathered row.
  Decode reads rows as stored. q is used as given (its rope half already
  rotated).
- Query i of sequence b sits at absolute position cache_len[b] + i and sees
  keys at positions p <= cache_len[b] + i.
- Chunking only bounds memory: the result is attention over all visible keys.
- The single graph-op call (prefill_decode) writes the new tokens processed,
  then reads the pool as stored in both branches; max_seq_len counts a
  sequence's new tokens: above 1 prefill, 1 decode.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Storage decoding
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64: the bits are the upper half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP float8_e4m3fn codes -> float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); there are no infinities and S.1111.111 is NaN.
    The dtype is named on the flare_mla_prefill_dispatch page (Parameters,
    "dtype": bfloat16 or float8_e4m3fn).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def decode_storage(arr: np.ndarray) -> np.ndarray:
    """Decode uint16 (bf16) or uint8 (e4m3fn) storage to float64."""
    if arr.dtype == np.uint16:
        return bf16_to_f64(arr)
    if arr.dtype == np.uint8:
        return e4m3fn_to_f64(arr)
    raise TypeError(f"unknown storage dtype {arr.dtype}")


# ---------------------------------------------------------------------------
# Plan (mla_prefill_plan page: description and Args)
# ---------------------------------------------------------------------------


def plan(input_row_offsets, cache_lengths, buffer_token_size: int, max_chunks: int):
    """Chunk plan of a ragged batch.

    Sequence b holds L_b = (offsets[b+1] - offsets[b]) + cache_len[b] tokens,
    cached ones first. Chunk c takes len(c, b) = clamp(L_b - c*T, 0, T) of them,
    starting at position cache_offsets[c, b] = min(c*T, L_b). The chunk's rows
    are packed sequence after sequence: buffer_row_offsets[c, b] is the running
    sum of len over earlier sequences, buffer_row_offsets[c, B] the total, and
    buffer_lengths[c] that total, or -1 for a chunk with no rows.

    Returns (buffer_row_offsets uint32 [C, B+1], cache_offsets uint32 [C, B],
    buffer_lengths int32 [C]).
    """
    offs = [int(x) for x in np.asarray(input_row_offsets).ravel()]
    clen = [int(x) for x in np.asarray(cache_lengths).ravel()]
    B = len(clen)
    T = int(buffer_token_size)
    C = int(max_chunks)
    if T < 1 or C < 1 or len(offs) != B + 1:
        raise ValueError("bad plan arguments")
    L = [offs[b + 1] - offs[b] + clen[b] for b in range(B)]
    bro = np.zeros((C, B + 1), dtype=np.uint32)
    co = np.zeros((C, B), dtype=np.uint32)
    bl = np.zeros(C, dtype=np.int32)
    for c in range(C):
        total = 0
        for b in range(B):
            start = min(c * T, L[b])
            n = min(T, L[b] - start)
            co[c, b] = start
            bro[c, b] = total
            total += n
        bro[c, B] = total
        bl[c] = total if total > 0 else -1
    return bro, co, bl


# ---------------------------------------------------------------------------
# Latent rows: gather, RMSNorm, RoPE (mla_prefill_decode_graph_bf16 page:
# Parameters "kv_input_fn", Args "kv_norm_gamma", "epsilon", "freqs_cis")
# ---------------------------------------------------------------------------


def gather_rows(pool: np.ndarray, page_table: np.ndarray, b: int,
                positions: np.ndarray, page_size: int) -> np.ndarray:
    """Rows of sequence b at the given logical positions, from the paged pool.

    Position p lives in logical page p // page_size at slot p % page_size; the
    page table maps the logical page to a physical page of the pool.
    """
    positions = np.asarray(positions, dtype=np.int64)
    flat = pool.reshape(-1, pool.shape[-1])
    phys = page_table[b, positions // page_size].astype(np.int64) * page_size \
        + positions % page_size
    return flat[phys]


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x * gamma / sqrt(mean(x^2) + eps) along the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * gamma / np.sqrt(ms + eps)


def rope(y: np.ndarray, freqs_rows: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (y[2i], y[2i+1]) by (F[2i] + i F[2i+1])."""
    yr, yi = y[..., 0::2], y[..., 1::2]
    fc, fs = freqs_rows[..., 0::2], freqs_rows[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = yr * fc - yi * fs
    out[..., 1::2] = yr * fs + yi * fc
    return out


def norm_rope_rows(raw: np.ndarray, positions: np.ndarray, gamma: np.ndarray,
                   freqs: np.ndarray, eps: float, lora: int):
    """Split raw cache rows into the normalised latent and the rotated rope part."""
    x = raw[:, :lora]
    y = raw[:, lora:]
    return rms_norm(x, gamma, eps), rope(y, freqs[np.asarray(positions, np.int64)])


# ---------------------------------------------------------------------------
# KV write path (mla_prefill_decode_graph_bf16 page: Parameters "kv_input_fn",
# the new tokens' raw latent [tot_seq_len, 576]; Args "kv_norm_gamma",
# "epsilon", "freqs_cis", "input_row_offsets" and the paged KV cache)
# ---------------------------------------------------------------------------


def kv_write(pool: np.ndarray, page_table: np.ndarray, kv_input: np.ndarray,
             input_row_offsets, cache_lengths, gamma: np.ndarray, freqs: np.ndarray,
             eps: float, page_size: int, lora: int = 512) -> np.ndarray:
    """The pool (values, any float dtype) after storing every new token's row,
    normalised and rotated: token i of sequence b (row input_row_offsets[b] + i
    of kv_input) sits at position cache_lengths[b] + i; its stored row is the
    RMSNorm'd latent (times gamma) followed by the rope part rotated for that
    position, in the slot the page table gives the position. Tokens whose
    logical page is outside the page table, whose page id is outside the pool,
    or whose position is outside freqs are not written. The reading: this is
    the processed-cache convention decode reads (rows as stored)."""
    out = np.array(pool, dtype=np.float64, copy=True)
    flat = out.reshape(-1, out.shape[-1])
    num_pages = pool.shape[0]
    off = np.asarray(input_row_offsets, dtype=np.int64)
    clen = np.asarray(cache_lengths, dtype=np.int64)
    for b in range(len(clen)):
        rows = np.asarray(kv_input[off[b]:off[b + 1]], dtype=np.float64)
        pos = clen[b] + np.arange(rows.shape[0], dtype=np.int64)
        lp = pos // page_size
        ok = (lp < page_table.shape[1]) & (pos < freqs.shape[0])
        pg = np.where(ok, page_table[b, np.minimum(lp, page_table.shape[1] - 1)], -1)
        ok &= (pg >= 0) & (pg < num_pages)
        if not ok.any():
            continue
        latn, kr = norm_rope_rows(rows[ok], pos[ok], gamma, freqs, eps, lora)
        flat[pg[ok].astype(np.int64) * page_size + pos[ok] % page_size] = \
            np.concatenate([latn, kr], axis=1)
    return out


# ---------------------------------------------------------------------------
# Up-projection (mla_prefill_decode_graph_bf16 page: Args "w_k", "w_uv")
# ---------------------------------------------------------------------------


def up_project(latn: np.ndarray, w_k: np.ndarray, w_uv: np.ndarray, num_heads: int):
    """K_nope[r, h, d] = sum_l w_k[h*nope + d, l] latn[r, l];
    V[r, h, d] = sum_l w_uv[h, d, l] latn[r, l]."""
    R = latn.shape[0]
    nope = w_k.shape[0] // num_heads
    k = (latn @ w_k.T).reshape(R, num_heads, nope)
    v = np.einsum("rl,hdl->rhd", latn, w_uv)
    return k, v


# ---------------------------------------------------------------------------
# Decoded workload views
# ---------------------------------------------------------------------------


class Decoded:
    """float64 views of a prefill workload's inputs."""

    def __init__(self, wl):
        self.wl = wl
        d = wl.dims
        self.nope, self.rope, self.v, self.lora = d.nope, d.rope, d.v, d.lora
        self.H = wl.num_heads
        self.q = decode_storage(wl.q)
        self.pool = decode_storage(wl.pool)
        self.gamma = bf16_to_f64(wl.gamma)
        self.freqs = bf16_to_f64(wl.freqs)
        self.w_k = bf16_to_f64(wl.w_k)
        self.w_uv = bf16_to_f64(wl.w_uv)
        self.w_uk = bf16_to_f64(wl.w_uk)
        self.offs = [int(x) for x in wl.input_row_offsets]
        self.clen = [int(x) for x in wl.cache_lengths]
        self.B = len(self.clen)

    def seq_keys(self, b: int, upto: int | None = None):
        """Processed keys of sequence b for positions [0, upto):
        (latn [n, lora], krope [n, rope])."""
        L = self.offs[b + 1] - self.offs[b] + self.clen[b]
        n = L if upto is None else min(L, upto)
        pos = np.arange(n)
        raw = gather_rows(self.pool, self.wl.page_table, b, pos, self.wl.page_size)
        return norm_rope_rows(raw, pos, self.gamma, self.freqs, self.wl.eps, self.lora)


# ---------------------------------------------------------------------------
# Prefill attention (flare_mla_prefill_dispatch page; causal mask shifted by
# the cached length)
# ---------------------------------------------------------------------------


def _masked_softmax_rows(s: np.ndarray, visible: np.ndarray, sink=None) -> np.ndarray:
    """Softmax of the visible scores of every row. A sink (mla_prefill_decode
    _graph_bf16 page: Args "attn_sink_ptr", per-batch attention sink weights)
    is one more logit in the denominator whose value vector is zero: weights
    e^s_j / (sum_k e^s_k + e^sink). A row with no visible key and a sink gets
    all-zero weights."""
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    if sink is not None and np.isfinite(sink):
        m = np.maximum(m, sink)
    e = np.where(visible, np.exp(s - m), 0.0)
    den = np.sum(e, axis=-1, keepdims=True)
    if sink is not None and np.isfinite(sink):
        den = den + np.exp(sink - m)
    return e / den


def attend_sequence(qb: np.ndarray, k_nope: np.ndarray, krope: np.ndarray,
                    v: np.ndarray, qpos: np.ndarray, kpos: np.ndarray,
                    scale: float, nope: int, sink=None) -> np.ndarray:
    """Attention of one sequence's queries over its keys, all heads.

    qb [n, H, nope+rope]; k_nope [L, H, nope]; krope [L, rope] (one head shared
    by all query heads); v [L, H, v]. Query at absolute position qpos[i] sees the
    key at kpos[j] iff kpos[j] <= qpos[i]. sink: the sequence's sink logit, or
    None. Returns [n, H, v].
    """
    n, H = qb.shape[0], qb.shape[1]
    out = np.empty((n, H, v.shape[-1]))
    visible = kpos[None, :] <= qpos[:, None]
    rope_scores = np.einsum("nhe,le->hnl", qb[:, :, nope:], krope)
    for h in range(H):
        s = qb[:, h, :nope] @ k_nope[:, h, :].T + rope_scores[h]
        a = _masked_softmax_rows(scale * s, visible, sink)
        out[:, h, :] = a @ v[:, h, :]
    return out


def prefill(wl, dec: Decoded | None = None, sinks=None) -> np.ndarray:
    """Full MLA prefill output [T_q, H, v] in float64 (no chunking); sinks:
    one sink logit per sequence, or None."""
    dec = dec or Decoded(wl)
    out = np.zeros((wl.total_q, dec.H, dec.v))
    for b in range(dec.B):
        n = dec.offs[b + 1] - dec.offs[b]
        if n == 0:
            continue
        latn, krope = dec.seq_keys(b)
        k_nope, v = up_project(latn, dec.w_k, dec.w_uv, dec.H)
        L = latn.shape[0]
        qpos = dec.clen[b] + np.arange(n)
        out[dec.offs[b]:dec.offs[b + 1]] = attend_sequence(
            dec.q[dec.offs[b]:dec.offs[b + 1]], k_nope, krope, v, qpos,
            np.arange(L), wl.scale, dec.nope, None if sinks is None else float(sinks[b]))
    return out


def prefill_sampled(wl, samples, dec: Decoded | None = None) -> np.ndarray:
    """Output rows out[t, h, :] for the listed (t, h) pairs only.

    For large workloads: keys are processed only up to the largest position the
    sampled queries of each sequence can see, and only the sampled heads are
    up-projected.
    """
    dec = dec or Decoded(wl)
    samples = [(int(t), int(h)) for t, h in samples]
    res = np.zeros((len(samples), dec.v))
    seq_of = np.searchsorted(np.asarray(dec.offs[1:]), [t for t, _ in samples],
                             side="right")
    groups: dict = {}
    for idx, ((t, h), b) in enumerate(zip(samples, seq_of)):
        groups.setdefault(int(b), []).append((idx, t, h))
    for b, items in groups.items():
        P_max = max(dec.clen[b] + (t - dec.offs[b]) for _, t, _ in items)
        latn, krope = dec.seq_keys(b, P_max + 1)
        kpos = np.arange(latn.shape[0])
        by_head: dict = {}
        for it in items:
            by_head.setdefault(it[2], []).append(it)
        for h, its in by_head.items():
            k_h = latn @ dec.w_k[h * dec.nope:(h + 1) * dec.nope].T
            v_h = latn @ dec.w_uv[h].T
            for idx, t, _ in its:
                qv = dec.q[t, h]
                P = dec.clen[b] + (t - dec.offs[b])
                s = wl.scale * (k_h @ qv[:dec.nope] + krope @ qv[dec.nope:])
                a = _masked_softmax_rows(s[None, :], (kpos <= P)[None, :])[0]
                res[idx] = a @ v_h
    return res


def prefill_chunked(wl, dec: Decoded | None = None, buffer_token_size: int | None = None):
    """Prefill evaluated chunk by chunk through the plan, merging partial
    softmax states (m, l, O) across chunks; reaches prefill() up to rounding.
    Returns (out [T_q, H, v], plan tuple)."""
    dec = dec or Decoded(wl)
    T = wl.buffer_token_size if buffer_token_size is None else buffer_token_size
    Lmax = max([dec.offs[b + 1] - dec.offs[b] + dec.clen[b] for b in range(dec.B)] + [1])
    C = (Lmax + T - 1) // T + 1
    bro, co, bl = plan(wl.input_row_offsets, wl.cache_lengths, T, C)
    H = dec.H
    m = np.full((wl.total_q, H), -np.inf)
    ell = np.zeros((wl.total_q, H))
    acc = np.zeros((wl.total_q, H, dec.v))
    for c in range(C):
        if bl[c] < 0:
            continue
        for b in range(dec.B):
            nrows = int(bro[c, b + 1]) - int(bro[c, b])
            n = dec.offs[b + 1] - dec.offs[b]
            if nrows == 0 or n == 0:
                continue
            kpos = int(co[c, b]) + np.arange(nrows)
            raw = gather_rows(dec.pool, wl.page_table, b, kpos, wl.page_size)
            latn, krope = norm_rope_rows(raw, kpos, dec.gamma, dec.freqs, wl.eps, dec.lora)
            k_nope, v = up_project(latn, dec.w_k, dec.w_uv, H)
            qpos = dec.clen[b] + np.arange(n)
            vis = kpos[None, :] <= qpos[:, None]
            t0 = dec.offs[b]
            for h in range(H):
                qb = dec.q[t0:t0 + n, h]
                s = wl.scale * (qb[:, :dec.nope] @ k_nope[:, h].T + qb[:, dec.nope:] @ krope.T)
                s = np.where(vis, s, -np.inf)
                mc = np.max(s, axis=1)
                has = np.isfinite(mc)
                m_new = np.where(has, np.maximum(m[t0:t0 + n, h], mc), m[t0:t0 + n, h])
                alpha = np.where(np.isfinite(m[t0:t0 + n, h]),
                                 np.exp(m[t0:t0 + n, h] - np.where(has, m_new, 0.0)), 0.0)
                alpha = np.where(has, alpha, 1.0)
                p = np.where(vis, np.exp(s - np.where(has, m_new, 0.0)[:, None]), 0.0)
                ell[t0:t0 + n, h] = alpha * ell[t0:t0 + n, h] + p.sum(axis=1)
                acc[t0:t0 + n, h] = alpha[:, None] * acc[t0:t0 + n, h] + p @ v[:, h]
                m[t0:t0 + n, h] = m_new
    return acc / ell[:, :, None], (bro, co, bl)


# ---------------------------------------------------------------------------
# Absorbed decode (mla_prefill_decode_graph_bf16 page: decode branch, Args
# "w_uk", "w_uv"; flare_mla_prefill_dispatch page: kv_num_heads 1,
# cache_depth 576)
# ---------------------------------------------------------------------------


class DecodedDecode:
    def __init__(self, wl):
        self.wl = wl
        d = wl.dims
        self.nope, self.rope, self.v, self.lora = d.nope, d.rope, d.v, d.lora
        self.H = wl.num_heads
        self.q = decode_storage(wl.q)
        self.pool = decode_storage(wl.pool)
        self.w_uk = bf16_to_f64(wl.w_uk)
        self.w_uv = bf16_to_f64(wl.w_uv)
        self.ctx = [int(x) for x in wl.context_lens]


def decode_one(qrow: np.ndarray, Z: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
               scale: float, nope: int, lora: int, sink=None) -> np.ndarray:
    """Absorbed decode of one token, all heads.

    qrow [H, nope+rope]; Z [ctx, lora+rope] cache rows as stored (one KV head);
    q_lat[h] = w_uk[h] @ q_nope[h]; s = scale * (q_lat . Z[:, :lora] +
    q_rope . Z[:, lora:]); o_lat = softmax(s) @ Z[:, :lora]; out[h] = w_uv[h] @ o_lat.
    sink: a sink logit in the softmax denominator, or None. Returns [H, v].
    """
    qlat = np.einsum("hld,hd->hl", w_uk, qrow[:, :nope])
    s = scale * (qlat @ Z[:, :lora].T + qrow[:, nope:] @ Z[:, lora:].T)
    a = _masked_softmax_rows(s, np.ones(s.shape, dtype=bool), sink)
    olat = a @ Z[:, :lora]
    return np.einsum("hdl,hl->hd", w_uv, olat)


def decode(wl, dec: DecodedDecode | None = None, batch_indices=None, sinks=None) -> np.ndarray:
    """Absorbed decode output [B, H, v] (or only the listed sequences); sinks:
    one sink logit per sequence, or None."""
    dec = dec or DecodedDecode(wl)
    idx = range(len(dec.ctx)) if batch_indices is None else list(batch_indices)
    out = np.zeros((len(idx), dec.H, dec.v))
    for i, b in enumerate(idx):
        Z = gather_rows(dec.pool, wl.page_table, b, np.arange(dec.ctx[b]), wl.page_size)
        out[i] = decode_one(dec.q[b], Z, dec.w_uk, dec.w_uv, wl.scale, dec.nope, dec.lora,
                            None if sinks is None else float(sinks[b]))
    return out


def decode_sparse(q: np.ndarray, pool: np.ndarray, d_indices: np.ndarray, topk_lengths,
                  w_uk: np.ndarray, w_uv: np.ndarray, scale: float, nope: int = 128,
                  lora: int = 512, sinks=None) -> np.ndarray:
    """Sparse absorbed decode (mla_prefill_decode_graph_bf16 page: Parameters
    "sparse_mla", "sparse_indices_stride"; Args "d_indices" (physical KV row
    indices per sequence), "indices_stride", "topk_lengths"): token b attends
    over the pool rows d_indices[b, 0:topk_lengths[b]] as stored, a physical
    row being page * page_size + slot of the pool flattened to rows. A
    sequence that lists no row outputs zeros. Values, not storage bits.
    Returns [B, H, v]."""
    flat = np.asarray(pool, dtype=np.float64).reshape(-1, pool.shape[-1])
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], w_uv.shape[0], w_uv.shape[1]))
    for b in range(q.shape[0]):
        k = int(topk_lengths[b])
        if k <= 0:
            continue
        Z = flat[np.asarray(d_indices[b, :k], dtype=np.int64)]
        out[b] = decode_one(q[b], Z, w_uk, w_uv, scale, nope, lora,
                            None if sinks is None else float(sinks[b]))
    return out


def prefill_decode(q, input_row_offsets, cache_lengths, pool, page_table, page_size: int,
                   w_k, w_uk, w_uv, gamma, freqs, scale: float, eps: float, max_seq_len: int,
                   kv_input=None, d_indices=None, topk_lengths=None, sinks=None,
                   nope: int = 128, lora: int = 512):
    """The graph op as one call (mla_prefill_decode_graph_bf16 page:
    description, the batch's maximum sequence length selects prefill or
    decode; Parameters "kv_input_fn", "sparse_mla"; Args "max_seq_len",
    "d_indices", "topk_lengths", "attn_sink_ptr"). Values, not storage bits.

    1. With kv_input (the new tokens' raw rows), every new token is first
       stored processed in the pool (kv_write).
    2. max_seq_len > 1, prefill: the queries of sequence b (rows
       input_row_offsets[b] .. input_row_offsets[b+1] of q, at positions
       cache_lengths[b] + i) attend causally over the sequence's rows at
       positions [0, cache_lengths[b] + n_b) read as stored, the latent part
       up-projected through w_k and w_uv, the rope part shared by all heads.
       max_seq_len == 1, decode: every sequence brings one token; q row b
       attends, absorbed through w_uk, over its rows at positions
       [0, cache_lengths[b] + 1), or with d_indices over the listed pool rows
       (decode_sparse); the result is projected through w_uv.
       max_seq_len == 0: no query.
    The reading: max_seq_len counts a sequence's new tokens (the query
    length), and both branches read the pool in the processed form the write
    stores. Returns (output [T_q, H, v], the pool after the write)."""
    off = np.asarray(input_row_offsets, dtype=np.int64)
    clen = np.asarray(cache_lengths, dtype=np.int64)
    B = len(clen)
    q = np.asarray(q, dtype=np.float64)
    H = w_uv.shape[0]
    pool = np.asarray(pool, dtype=np.float64)
    if kv_input is not None:
        pool = kv_write(pool, page_table, kv_input, off, clen, gamma, freqs, eps, page_size, lora)
    out = np.zeros((q.shape[0], H, w_uv.shape[1]))
    sink = (lambda b: None) if sinks is None else (lambda b: float(sinks[b]))
    if max_seq_len > 1:
        for b in range(B):
            n = int(off[b + 1] - off[b])
            if n == 0:
                continue
            L = int(clen[b]) + n
            rows = gather_rows(pool, page_table, b, np.arange(L), page_size)
            k_nope, v = up_project(rows[:, :lora], w_k, w_uv, H)
            qpos = clen[b] + np.arange(n)
            out[off[b]:off[b + 1]] = attend_sequence(q[off[b]:off[b + 1]], k_nope,
                                                     rows[:, lora:], v, qpos, np.arange(L),
                                                     scale, nope, sink(b))
    elif max_seq_len == 1:
        if np.any(off[1:] - off[:-1] != 1):
            raise ValueError("decode takes exactly one new token per sequence")
        if d_indices is not None:
            out[:] = decode_sparse(q, pool, d_indices, topk_lengths, w_uk, w_uv, scale, nope,
                                   lora, sinks)
        else:
            for b in range(B):
                Z = gather_rows(pool, page_table, b, np.arange(int(clen[b]) + 1), page_size)
                out[b] = decode_one(q[b], Z, w_uk, w_uv, scale, nope, lora, sink(b))
    return out, pool


def decode_split(wl, num_splits: int, dec: DecodedDecode | None = None) -> np.ndarray:
    """Decode with the context cut into num_splits parts whose partial softmax
    states are merged by log-sum-exp; reaches decode() up to rounding."""
    dec = dec or DecodedDecode(wl)
    out = np.zeros((len(dec.ctx), dec.H, dec.v))
    for b in range(len(dec.ctx)):
        Z = gather_rows(dec.pool, wl.page_table, b, np.arange(dec.ctx[b]), wl.page_size)
        qrow = dec.q[b]
        qlat = np.einsum("hld,hd->hl", dec.w_uk, qrow[:, :dec.nope])
        bounds = np.linspace(0, dec.ctx[b], num_splits + 1).astype(int)
        ms, ls, os_ = [], [], []
        for s0, s1 in zip(bounds[:-1], bounds[1:]):
            if s1 <= s0:
                continue
            Zs = Z[s0:s1]
            s = wl.scale * (qlat @ Zs[:, :dec.lora].T + qrow[:, dec.nope:] @ Zs[:, dec.lora:].T)
            m = np.max(s, axis=1)
            e = np.exp(s - m[:, None])
            ms.append(m)
            ls.append(e.sum(axis=1))
            os_.append(e @ Zs[:, :dec.lora])
        M = np.max(np.stack(ms), axis=0)
        w = [np.exp(mi - M) for mi in ms]
        lsum = sum(wi * li for wi, li in zip(w, ls))
        olat = sum(wi[:, None] * oi for wi, oi in zip(w, os_)) / lsum[:, None]
        out[b] = np.einsum("hdl,hl->hd", dec.w_uv, olat)
    return out

