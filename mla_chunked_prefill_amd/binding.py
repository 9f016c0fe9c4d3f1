"""Python binding of libmla.so: argument marshalling only.

Every function here has the name of a C entry point of include/mla.h, checks
the tensors it is given (device, dtype, shape, contiguity), and passes their
device pointers and the current HIP stream to the library. All computation
runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_OK = 0
MLA_BF16 = 0
MLA_FP8_E4M3FN = 1

NOPE, ROPE, QD, VD, LORA, CACHE = 128, 64, 192, 128, 512, 576

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_U = ctypes.c_uint32
_F = ctypes.c_float
_S = ctypes.c_size_t

_SIGNATURES = {
    "mla_prefill_plan": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _U, _P]),
    "mla_gather_norm_rope": (_I, [_P, _P, _I, _P, _I, _P, _P, _P, _P, _P, _P,
                                  _I, _I, _I, _I, _I, _I, _F, _P]),
    "mla_kv_write": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "mla_up_project": (_I, [_P, _P, _I, _P, _P, _P, _P, _I, _I, _P]),
    "mla_prefill_attention_workspace_size": (_S, [_I, _I, _I]),
    "mla_prefill_attention": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _I, _I, _I, _I, _I, _F, _P, _P, _S, _P]),
    "mla_prefill_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "mla_prefill": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P,
                         _I, _I, _I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _S, _P]),
    "mla_decode_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "mla_decode": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                        _P, _P, _S, _P]),
    "mla_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                _F, _P, _P]),
    "mla_decode_sparse_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "mla_decode_sparse": (_I, [_P, _P, _P, _P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F,
                               _P, _P, _S, _P]),
    "mla_prefill_decode_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "mla_prefill_decode": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I,
                                _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                _F, _F, _P, _I, _P, _P, _I, _P, _S, _P]),
    "mla_hbm_read": (_I, [_P, _S, _P, _I, _P]),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGNATURES)


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmla.so once; raise if it has not been built. The MLA_LIB
    environment variable names another build of the library to load."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MLA_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m mla_chunked_prefill_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != MLA_OK:
        detail = load().mla_last_error().decode()
        raise MlaError(fn, status, detail)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return MLA_FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


def _sink_ptr(attn_sink, B):
    """Pointer of an optional float32 [B] tensor of sink logits (None: no sink)."""
    if attn_sink is None:
        return None
    _expect(attn_sink, torch.float32, (B,), "attn_sink")
    return _ptr(attn_sink)


def _expect(t, dtype, shape=None, name="tensor"):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def mla_prefill_plan(buffer_row_offsets, cache_offsets, buffer_lengths, input_row_offsets,
                     cache_lengths, buffer_token_size: int, chunks_needed=None, stream=None):
    C, B1 = buffer_row_offsets.shape
    B = B1 - 1
    _expect(buffer_row_offsets, torch.uint32, (C, B + 1), "buffer_row_offsets")
    _expect(cache_offsets, torch.uint32, (C, B), "cache_offsets")
    _expect(buffer_lengths, torch.int32, (C,), "buffer_lengths")
    _expect(input_row_offsets, torch.uint32, (B + 1,), "input_row_offsets")
    _expect(cache_lengths, torch.uint32, (B,), "cache_lengths")
    if chunks_needed is not None:
        _expect(chunks_needed, torch.uint32, (1,), "chunks_needed")
    st = load().mla_prefill_plan(_ptr(buffer_row_offsets), _ptr(cache_offsets),
                                 _ptr(buffer_lengths), _ptr(chunks_needed),
                                 _ptr(input_row_offsets), _ptr(cache_lengths), B, C,
                                 int(buffer_token_size), _stream(stream))
    _check("mla_prefill_plan", st)


def mla_gather_norm_rope(latent_out, krope_out, kv_cache, page_table, buffer_row_offsets_c,
                         cache_offsets_c, buffer_length_c, kv_norm_gamma, freqs_cis,
                         epsilon: float, stream=None):
    R = latent_out.shape[0]
    B = page_table.shape[0]
    _expect(latent_out, torch.bfloat16, (R, LORA), "latent_out")
    if tuple(krope_out.shape) != (R, ROPE):
        raise ValueError("krope_out shape")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != CACHE:
        raise ValueError("kv_cache shape")
    _expect(page_table, torch.int32, None, "page_table")
    _expect(buffer_row_offsets_c, torch.uint32, (B + 1,), "buffer_row_offsets_c")
    _expect(cache_offsets_c, torch.uint32, (B,), "cache_offsets_c")
    _expect(buffer_length_c, torch.int32, (1,), "buffer_length_c")
    _expect(kv_norm_gamma, torch.bfloat16, (LORA,), "kv_norm_gamma")
    _expect(freqs_cis, torch.bfloat16, None, "freqs_cis")
    st = load().mla_gather_norm_rope(
        _ptr(latent_out), _ptr(krope_out), _dtype_code(krope_out), _ptr(kv_cache),
        _dtype_code(kv_cache), _ptr(page_table), _ptr(buffer_row_offsets_c),
        _ptr(cache_offsets_c), _ptr(buffer_length_c), _ptr(kv_norm_gamma), _ptr(freqs_cis),
        B, kv_cache.shape[1], page_table.shape[1], kv_cache.shape[0], R, freqs_cis.shape[0],
        float(epsilon), _stream(stream))
    _check("mla_gather_norm_rope", st)


def mla_kv_write(kv_cache, page_table, kv_input, input_row_offsets, cache_lengths,
                 kv_norm_gamma, freqs_cis, epsilon: float, stream=None):
    B = cache_lengths.shape[0]
    if kv_cache.dim() != 3 or kv_cache.shape[2] != CACHE:
        raise ValueError("kv_cache shape")
    _expect(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table shape")
    _expect(kv_input, torch.bfloat16, (kv_input.shape[0], CACHE), "kv_input")
    _expect(input_row_offsets, torch.uint32, (B + 1,), "input_row_offsets")
    _expect(cache_lengths, torch.uint32, (B,), "cache_lengths")
    _expect(kv_norm_gamma, torch.bfloat16, (LORA,), "kv_norm_gamma")
    _expect(freqs_cis, torch.bfloat16, (freqs_cis.shape[0], ROPE), "freqs_cis")
    st = load().mla_kv_write(
        _ptr(kv_cache), _dtype_code(kv_cache), _ptr(page_table), _ptr(kv_input),
        _ptr(input_row_offsets), _ptr(cache_lengths), _ptr(kv_norm_gamma), _ptr(freqs_cis),
        B, kv_input.shape[0], kv_cache.shape[1], page_table.shape[1], kv_cache.shape[0],
        freqs_cis.shape[0], float(epsilon), _stream(stream))
    _check("mla_kv_write", st)


def mla_up_project(k_nope_out, v_t_out, latent, w_k, w_uv, buffer_length_c, stream=None):
    H = w_uv.shape[0]
    R = latent.shape[0]
    _expect(latent, torch.bfloat16, (R, LORA), "latent")
    if tuple(k_nope_out.shape) != (H, R, NOPE):
        raise ValueError("k_nope_out shape")
    _expect(v_t_out, torch.bfloat16, (H, VD, R), "v_t_out")
    _expect(w_k, torch.bfloat16, (H * NOPE, LORA), "w_k")
    _expect(w_uv, torch.bfloat16, (H, VD, LORA), "w_uv")
    _expect(buffer_length_c, torch.int32, (1,), "buffer_length_c")
    st = load().mla_up_project(_ptr(k_nope_out), _ptr(v_t_out), _dtype_code(k_nope_out),
                               _ptr(latent), _ptr(w_k), _ptr(w_uv), _ptr(buffer_length_c), H,
                               R, _stream(stream))
    _check("mla_up_project", st)


def mla_prefill_attention_workspace_size(batch_size: int, total_q: int, num_heads: int) -> int:
    return int(load().mla_prefill_attention_workspace_size(batch_size, total_q, num_heads))


def mla_prefill_attention(output, q, k_nope, v_t, krope, input_row_offsets, cache_lengths,
                          buffer_row_offsets_c, cache_offsets_c, buffer_length_c,
                          max_prompt_len: int, scale: float, workspace, stream=None,
                          attn_sink=None):
    Tq, H = q.shape[0], q.shape[1]
    B = cache_lengths.shape[0]
    R = krope.shape[0]
    _expect(output, torch.bfloat16, (Tq, H, VD), "output")
    if tuple(q.shape) != (Tq, H, QD):
        raise ValueError("q shape")
    if tuple(k_nope.shape) != (H, R, NOPE):
        raise ValueError("k_nope shape")
    _expect(v_t, torch.bfloat16, (H, VD, R), "v_t")
    _expect(input_row_offsets, torch.uint32, (B + 1,), "input_row_offsets")
    st = load().mla_prefill_attention(
        _ptr(output), _ptr(q), _dtype_code(q), _ptr(k_nope), _ptr(v_t), _ptr(krope),
        _ptr(input_row_offsets), _ptr(cache_lengths), _ptr(buffer_row_offsets_c),
        _ptr(cache_offsets_c), _ptr(buffer_length_c), B, Tq, H, R, int(max_prompt_len),
        float(scale), _sink_ptr(attn_sink, B), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_prefill_attention", st)


def mla_prefill_workspace_size(batch_size: int, total_q: int, num_heads: int, max_rows: int,
                               dtype: int) -> int:
    return int(load().mla_prefill_workspace_size(batch_size, total_q, num_heads, max_rows,
                                                 dtype))


def mla_prefill(output, q, input_row_offsets, cache_lengths, kv_cache, page_table,
                buffer_row_offsets, cache_offsets, buffer_lengths, max_rows: int, w_k, w_uv,
                kv_norm_gamma, freqs_cis, max_prompt_len: int, scale: float, epsilon: float,
                workspace, stream=None, attn_sink=None):
    Tq, H = q.shape[0], q.shape[1]
    B = cache_lengths.shape[0]
    C = buffer_lengths.shape[0]
    _expect(output, torch.bfloat16, (Tq, H, VD), "output")
    if q.dtype != kv_cache.dtype:
        raise TypeError("q and kv_cache must share a dtype")
    _expect(buffer_row_offsets, torch.uint32, (C, B + 1), "buffer_row_offsets")
    _expect(cache_offsets, torch.uint32, (C, B), "cache_offsets")
    _expect(w_k, torch.bfloat16, (H * NOPE, LORA), "w_k")
    _expect(w_uv, torch.bfloat16, (H, VD, LORA), "w_uv")
    st = load().mla_prefill(
        _ptr(output), _ptr(q), _dtype_code(q), _ptr(input_row_offsets), _ptr(cache_lengths),
        _ptr(kv_cache), _ptr(page_table), _ptr(buffer_row_offsets), _ptr(cache_offsets),
        _ptr(buffer_lengths), C, int(max_rows), _ptr(w_k), _ptr(w_uv), _ptr(kv_norm_gamma),
        _ptr(freqs_cis), B, Tq, H, int(max_prompt_len), kv_cache.shape[1],
        page_table.shape[1], kv_cache.shape[0], freqs_cis.shape[0], float(scale),
        float(epsilon), _sink_ptr(attn_sink, B), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_prefill", st)


def mla_decode_workspace_size(batch_size: int, num_heads: int, max_context_len: int,
                              page_size: int, num_partitions: int, cache_dtype: int) -> int:
    return int(load().mla_decode_workspace_size(batch_size, num_heads, max_context_len,
                                                page_size, num_partitions, cache_dtype))


def mla_decode(output, q, context_lengths, kv_cache, page_table, w_uk, w_uv,
               max_context_len: int, scale: float, workspace, num_partitions: int = 0,
               stream=None, attn_sink=None):
    B, H = q.shape[0], q.shape[1]
    _expect(output, torch.bfloat16, (B, H, VD), "output")
    _expect(q, torch.bfloat16, (B, H, QD), "q")
    _expect(context_lengths, torch.uint32, (B,), "context_lengths")
    _expect(w_uk, torch.bfloat16, (H, LORA, NOPE), "w_uk")
    _expect(w_uv, torch.bfloat16, (H, VD, LORA), "w_uv")
    st = load().mla_decode(
        _ptr(output), _ptr(q), _ptr(context_lengths), _ptr(kv_cache), _dtype_code(kv_cache),
        _ptr(page_table), _ptr(w_uk), _ptr(w_uv), B, H, kv_cache.shape[1], page_table.shape[1],
        kv_cache.shape[0], int(max_context_len), int(num_partitions), float(scale),
        _sink_ptr(attn_sink, B), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("mla_decode", st)


def mla_decode_noalloc(output, q, context_lengths, kv_cache, page_table, w_uk, w_uv,
                       max_context_len: int, scale: float, num_partitions: int = 0,
                       stream=None, attn_sink=None):
    """mla_decode with its workspace in the library's fixed scratch array."""
    B, H = q.shape[0], q.shape[1]
    _expect(output, torch.bfloat16, (B, H, VD), "output")
    _expect(q, torch.bfloat16, (B, H, QD), "q")
    _expect(context_lengths, torch.uint32, (B,), "context_lengths")
    _expect(w_uk, torch.bfloat16, (H, LORA, NOPE), "w_uk")
    _expect(w_uv, torch.bfloat16, (H, VD, LORA), "w_uv")
    st = load().mla_decode_noalloc(
        _ptr(output), _ptr(q), _ptr(context_lengths), _ptr(kv_cache), _dtype_code(kv_cache),
        _ptr(page_table), _ptr(w_uk), _ptr(w_uv), B, H, kv_cache.shape[1], page_table.shape[1],
        kv_cache.shape[0], int(max_context_len), int(num_partitions), float(scale),
        _sink_ptr(attn_sink, B), _stream(stream))
    _check("mla_decode_noalloc", st)


def mla_decode_sparse_workspace_size(batch_size: int, num_heads: int, max_topk: int,
                                     num_partitions: int, cache_dtype: int) -> int:
    return int(load().mla_decode_sparse_workspace_size(batch_size, num_heads, max_topk,
                                                       num_partitions, cache_dtype))


def mla_decode_sparse(output, q, topk_lengths, kv_cache, d_indices, w_uk, w_uv, max_topk: int,
                      scale: float, workspace, num_partitions: int = 0, stream=None,
                      attn_sink=None):
    B, H = q.shape[0], q.shape[1]
    _expect(output, torch.bfloat16, (B, H, VD), "output")
    _expect(q, torch.bfloat16, (B, H, QD), "q")
    _expect(topk_lengths, torch.int32, (B,), "topk_lengths")
    _expect(d_indices, torch.int32, None, "d_indices")
    if d_indices.dim() != 2 or d_indices.shape[0] != B:
        raise ValueError("d_indices shape")
    if kv_cache.dim() != 2 or kv_cache.shape[1] != CACHE:
        raise ValueError("kv_cache shape: [num_rows, 576]")
    _expect(w_uk, torch.bfloat16, (H, LORA, NOPE), "w_uk")
    _expect(w_uv, torch.bfloat16, (H, VD, LORA), "w_uv")
    st = load().mla_decode_sparse(
        _ptr(output), _ptr(q), _ptr(topk_lengths), _ptr(kv_cache), _dtype_code(kv_cache),
        _ptr(d_indices), d_indices.shape[1], _ptr(w_uk), _ptr(w_uv), B, H, kv_cache.shape[0],
        int(max_topk), int(num_partitions), float(scale), _sink_ptr(attn_sink, B),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_decode_sparse", st)


def mla_prefill_decode_workspace_size(batch_size: int, total_q: int, num_heads: int,
                                      max_seq_len: int, max_rows: int, max_cache_len: int,
                                      page_size: int, indices_stride: int, num_partitions: int,
                                      cache_dtype: int) -> int:
    return int(load().mla_prefill_decode_workspace_size(
        batch_size, total_q, num_heads, max_seq_len, max_rows, max_cache_len, page_size,
        indices_stride, num_partitions, cache_dtype))


def mla_prefill_decode(output, q, input_row_offsets, cache_lengths, kv_cache, page_table,
                       w_uk, w_uv, kv_norm_gamma, freqs_cis, max_seq_len: int,
                       max_cache_len: int, scale: float, epsilon: float, workspace,
                       kv_input=None, w_k=None, plan_tensors=None, max_rows: int = 0,
                       d_indices=None, topk_lengths=None, attn_sink=None,
                       num_partitions: int = 0, stream=None):
    """The graph op as one call: optional KV write of kv_input, then prefill
    (max_seq_len > 1, plan_tensors = (buffer_row_offsets, cache_offsets,
    buffer_lengths) and w_k needed) or decode (max_seq_len == 1; sparse when
    d_indices is given) over the pool as stored."""
    Tq = q.shape[0]
    B = cache_lengths.shape[0]
    H = w_uv.shape[0]
    _expect(output, torch.bfloat16, (Tq, H, VD), "output")
    _expect(q, torch.bfloat16, (Tq, H, QD), "q")
    _expect(input_row_offsets, torch.uint32, (B + 1,), "input_row_offsets")
    _expect(cache_lengths, torch.uint32, (B,), "cache_lengths")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != CACHE:
        raise ValueError("kv_cache shape")
    _expect(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table shape")
    _expect(w_uv, torch.bfloat16, (H, VD, LORA), "w_uv")
    if w_uk is not None:
        _expect(w_uk, torch.bfloat16, (H, LORA, NOPE), "w_uk")
    if w_k is not None:
        _expect(w_k, torch.bfloat16, (H * NOPE, LORA), "w_k")
    _expect(kv_norm_gamma, torch.bfloat16, (LORA,), "kv_norm_gamma")
    _expect(freqs_cis, torch.bfloat16, (freqs_cis.shape[0], ROPE), "freqs_cis")
    if kv_input is not None:
        _expect(kv_input, torch.bfloat16, (Tq, CACHE), "kv_input")
    bro = co = bl = None
    C = 0
    if plan_tensors is not None:
        bro, co, bl = plan_tensors[:3]
        C = bl.shape[0]
        _expect(bro, torch.uint32, (C, B + 1), "buffer_row_offsets")
        _expect(co, torch.uint32, (C, B), "cache_offsets")
        _expect(bl, torch.int32, (C,), "buffer_lengths")
    stride = 0
    if d_indices is not None:
        _expect(d_indices, torch.int32, None, "d_indices")
        if d_indices.dim() != 2 or d_indices.shape[0] != B:
            raise ValueError("d_indices shape")
        _expect(topk_lengths, torch.int32, (B,), "topk_lengths")
        stride = d_indices.shape[1]
    st = load().mla_prefill_decode(
        _ptr(output), _ptr(q), _ptr(kv_input), _ptr(input_row_offsets), _ptr(cache_lengths),
        _ptr(kv_cache), _dtype_code(kv_cache), _ptr(page_table), _ptr(bro), _ptr(co), _ptr(bl),
        C, int(max_rows), _ptr(w_k), _ptr(w_uk), _ptr(w_uv), _ptr(kv_norm_gamma),
        _ptr(freqs_cis), B, Tq, H, int(max_seq_len), kv_cache.shape[1], page_table.shape[1],
        kv_cache.shape[0], int(max_cache_len), freqs_cis.shape[0], float(scale),
        float(epsilon), _ptr(d_indices), stride, _ptr(topk_lengths), _sink_ptr(attn_sink, B),
        int(num_partitions), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("mla_prefill_decode", st)


def mla_hbm_read(src, out, groups: int, stream=None):
    """Streaming read of the whole of src (a measurement helper)."""
    _expect(out, torch.uint32, (groups,), "out")
    st = load().mla_hbm_read(_ptr(src), src.numel() * src.element_size(), _ptr(out),
                             int(groups), _stream(stream))
    _check("mla_hbm_read", st)


# ---------------------------------------------------------------------------
# convenience: plan + workspace + call
# ---------------------------------------------------------------------------

def _plan_into(C, B, dev, input_row_offsets, cache_lengths, buffer_token_size, stream):
    bro = torch.empty((C, B + 1), dtype=torch.uint32, device=dev)
    co = torch.empty((C, B), dtype=torch.uint32, device=dev)
    bl = torch.empty((C,), dtype=torch.int32, device=dev)
    need = torch.empty((1,), dtype=torch.uint32, device=dev)
    mla_prefill_plan(bro, co, bl, input_row_offsets, cache_lengths, buffer_token_size,
                     chunks_needed=need, stream=stream)
    return bro, co, bl, need


def _read_chunks_needed(need, stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    s.synchronize()
    return int(need.cpu()[0])


def plan(input_row_offsets, cache_lengths, buffer_token_size: int,
         max_chunks: int | None = None, stream=None):
    """Run mla_prefill_plan into new device tensors; returns (bro, co, bl, chunks_needed).

    A convenience path with one host read: the planner's chunks_needed is read
    back once. max_chunks None plans exactly as many chunks as the batch needs
    (at least one); a max_chunks below that raises ValueError, since the
    queries of the chunks left out would never be attended. Callers that must
    not synchronise (graph capture) call mla_prefill_plan directly."""
    B = cache_lengths.shape[0]
    dev = cache_lengths.device
    C = 1 if max_chunks is None else int(max_chunks)
    if C < 1:
        raise ValueError(f"max_chunks must be >= 1, got {C}")
    res = _plan_into(C, B, dev, input_row_offsets, cache_lengths, buffer_token_size, stream)
    needed = _read_chunks_needed(res[3], stream)
    if max_chunks is None:
        if needed > C:
            res = _plan_into(needed, B, dev, input_row_offsets, cache_lengths,
                             buffer_token_size, stream)
    elif needed > C:
        raise ValueError(f"max_chunks={C} is below the {needed} chunks of "
                         f"buffer_token_size={int(buffer_token_size)} this batch needs")
    return res


def prefill(q, input_row_offsets, cache_lengths, kv_cache, page_table, w_k, w_uv,
            kv_norm_gamma, freqs_cis, buffer_token_size: int, max_chunks: int | None,
            max_prompt_len: int, scale: float, epsilon: float, max_rows: int | None = None,
            workspace=None, output=None, plan_tensors=None, stream=None, attn_sink=None):
    """Plan and run the whole chunked prefill; returns the bf16 output [Tq, H, 128].

    max_rows defaults to batch_size * buffer_token_size (always enough). Without
    plan_tensors the batch is planned here (plan(): one host read of the chunk
    count; max_chunks None plans as many chunks as needed, a smaller
    max_chunks raises)."""
    B = cache_lengths.shape[0]
    Tq, H = q.shape[0], q.shape[1]
    if max_rows is None:
        max_rows = B * int(buffer_token_size)
    max_rows = (int(max_rows) + 63) // 64 * 64
    if plan_tensors is None:
        plan_tensors = plan(input_row_offsets, cache_lengths, buffer_token_size, max_chunks,
                            stream)
    bro, co, bl = plan_tensors[:3]
    if output is None:
        output = torch.empty((Tq, H, VD), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        nbytes = mla_prefill_workspace_size(B, Tq, H, max_rows, _dtype_code(q))
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    mla_prefill(output, q, input_row_offsets, cache_lengths, kv_cache, page_table, bro, co, bl,
                max_rows, w_k, w_uv, kv_norm_gamma, freqs_cis, max_prompt_len, scale, epsilon,
                workspace, stream=stream, attn_sink=attn_sink)
    return output


def decode(q, context_lengths, kv_cache, page_table, w_uk, w_uv, max_context_len: int,
           scale: float, num_partitions: int = 0, workspace=None, output=None, stream=None,
           attn_sink=None):
    """Absorbed decode; returns the bf16 output [B, H, 128]."""
    B, H = q.shape[0], q.shape[1]
    if output is None:
        output = torch.empty((B, H, VD), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        nbytes = mla_decode_workspace_size(B, H, max_context_len, kv_cache.shape[1],
                                           num_partitions, _dtype_code(kv_cache))
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    mla_decode(output, q, context_lengths, kv_cache, page_table, w_uk, w_uv, max_context_len,
               scale, workspace, num_partitions=num_partitions, stream=stream,
               attn_sink=attn_sink)
    return output


def decode_sparse(q, topk_lengths, kv_cache, d_indices, w_uk, w_uv, max_topk: int,
                  scale: float, num_partitions: int = 0, workspace=None, output=None,
                  stream=None, attn_sink=None):
    """Sparse absorbed decode over the listed pool rows; returns [B, H, 128] bf16.
    kv_cache may be given paged ([num_pages, page_size, 576]); it is viewed as rows."""
    B, H = q.shape[0], q.shape[1]
    rows = kv_cache.reshape(-1, CACHE)
    if output is None:
        output = torch.empty((B, H, VD), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        nbytes = mla_decode_sparse_workspace_size(B, H, max_topk, num_partitions,
                                                  _dtype_code(kv_cache))
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    mla_decode_sparse(output, q, topk_lengths, rows, d_indices, w_uk, w_uv, max_topk, scale,
                      workspace, num_partitions=num_partitions, stream=stream,
                      attn_sink=attn_sink)
    return output


def prefill_decode(q, input_row_offsets, cache_lengths, kv_cache, page_table, w_uk, w_uv,
                   kv_norm_gamma, freqs_cis, max_seq_len: int, max_cache_len: int,
                   scale: float, epsilon: float, kv_input=None, w_k=None,
                   buffer_token_size: int = 8192, max_chunks: int | None = None,
                   max_rows: int | None = None, d_indices=None, topk_lengths=None,
                   attn_sink=None, num_partitions: int = 0, workspace=None, output=None,
                   plan_tensors=None, stream=None):
    """The graph op as one call (plans the chunks for a prefill unless
    plan_tensors are given: plan(), with one host read of the chunk count;
    max_chunks None plans as many as needed, a smaller max_chunks raises);
    returns the bf16 output [total_q, H, 128]."""
    B = cache_lengths.shape[0]
    Tq, H = q.shape[0], w_uv.shape[0]
    if max_seq_len > 1:
        if max_rows is None:
            max_rows = B * int(buffer_token_size)
        max_rows = (int(max_rows) + 63) // 64 * 64
        if plan_tensors is None:
            plan_tensors = plan(input_row_offsets, cache_lengths, buffer_token_size,
                                max_chunks, stream)
    else:
        max_rows = 0
    stride = 0 if d_indices is None else d_indices.shape[1]
    if output is None:
        output = torch.empty((Tq, H, VD), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        nbytes = mla_prefill_decode_workspace_size(B, Tq, H, max_seq_len, max_rows,
                                                   max_cache_len, kv_cache.shape[1], stride,
                                                   num_partitions, _dtype_code(kv_cache))
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    mla_prefill_decode(output, q, input_row_offsets, cache_lengths, kv_cache, page_table, w_uk,
                       w_uv, kv_norm_gamma, freqs_cis, max_seq_len, max_cache_len, scale,
                       epsilon, workspace, kv_input=kv_input, w_k=w_k,
                       plan_tensors=plan_tensors, max_rows=max_rows, d_indices=d_indices,
                       topk_lengths=topk_lengths, attn_sink=attn_sink,
                       num_partitions=num_partitions, stream=stream)
    return output
