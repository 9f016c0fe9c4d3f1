"""Copy a workload's storage bits to device tensors (no arithmetic)."""
from __future__ import annotations

import numpy as np
import torch


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def _store(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return _bf16(a, device)
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(device)
    raise TypeError(a.dtype)


def _u32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32)).to(device)


def _i32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def prefill_tensors(wl, device="cuda") -> dict:
    return dict(
        q=_store(wl.q, device), kv_cache=_store(wl.pool, device),
        page_table=_i32(wl.page_table, device),
        input_row_offsets=_u32(wl.input_row_offsets, device),
        cache_lengths=_u32(wl.cache_lengths, device),
        kv_norm_gamma=_bf16(wl.gamma, device), freqs_cis=_bf16(wl.freqs, device),
        w_k=_bf16(wl.w_k, device), w_uv=_bf16(wl.w_uv, device), w_uk=_bf16(wl.w_uk, device))


def decode_tensors(wl, device="cuda") -> dict:
    return dict(
        q=_store(wl.q, device), kv_cache=_store(wl.pool, device),
        page_table=_i32(wl.page_table, device), context_lengths=_u32(wl.context_lens, device),
        w_uk=_bf16(wl.w_uk, device), w_uv=_bf16(wl.w_uv, device))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> numpy uint16 storage bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def fp8_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()
