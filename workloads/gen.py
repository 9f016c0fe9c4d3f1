"""Seeded synthetic workloads for MLA chunked prefill and absorbed decode.

This module holds none of the method's arithmetic. It draws random numbers,
rounds them to the storage dtypes (bf16 by round-to-nearest-even, e4m3fn through
torch's cast), lays sequences out in a shuffled page pool with a page table,
and precomputes the RoPE angle table, which the method takes as an input
("freqs_cis", precomputed rotary frequencies, mla_prefill_decode_graph_bf16
page, Args). Everything is returned as raw storage bits in numpy arrays:
uint16 for bf16, uint8 for float8_e4m3fn, so each consumer decodes them itself.

Value recipe (identical for every workload):
- q, the pool's latent and rope values: N(0, 1) drawn in float32 (tensors of
  more than 4 * 2^20 values in blocks of 2^20, block k from a generator seeded
  by one draw of the workload's generator and k).
- kv_norm_gamma: 1 + N(0, 0.1) (0.1 is the standard deviation).
- w_k, w_uv, w_uk: N(0, 1/sqrt(512)) (standard deviation 1/sqrt(512)).
- fp8 workloads: q and the whole pool are each divided by their own absolute
  maximum (unit amax per tensor) and cast to float8_e4m3fn; weights, gamma and
  the RoPE table stay bf16.
- RoPE table: row p holds 32 interleaved (cos, sin) pairs of p * 10000^(-2i/64).
Draw order: lengths, page permutation, q, pool rows, gamma, w_k, w_uv, w_uk.
Each sequence's pages are a random subset of a shuffled pool that holds
exactly sum_b ceil(L_b / page_size) pages; unused slots of a last page are 0.
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Dims:
    """MLA head dimensions (DeepSeek V2/V3: 128 nope, 64 rope, 128 v, 512 latent)."""
    nope: int = 128
    rope: int = 64
    v: int = 128
    lora: int = 512

    @property
    def q_depth(self) -> int:
        return self.nope + self.rope

    @property
    def cache_depth(self) -> int:
        return self.lora + self.rope


MLA_DIMS = Dims()


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs stay below 0xFF80_8000 after the rounding add: no overflow
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def f32_to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """Cast float32 values to OCP float8_e4m3fn codes (torch's RNE cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


_BLOCK = 1 << 20


def _normals(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) float32 of the given shape. Large tensors are drawn in blocks of
    2^20 values; block k comes from its own generator seeded by (a draw of the
    parent generator, k), so the values do not depend on the thread count."""
    n = int(np.prod(shape))
    if n <= 4 * _BLOCK:
        return rng.standard_normal(shape, dtype=np.float32)
    import concurrent.futures
    base = int(rng.integers(0, 2 ** 63 - 1))
    out = np.empty(n, dtype=np.float32)

    def fill(k):
        g = np.random.default_rng(np.random.SeedSequence(base, spawn_key=(k,)))
        g.standard_normal(out=out[k * _BLOCK:(k + 1) * _BLOCK], dtype=np.float32)

    nblk = (n + _BLOCK - 1) // _BLOCK
    workers = min(16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _normal_bits(rng: np.random.Generator, shape, std: float = 1.0,
                 mean: float = 0.0) -> np.ndarray:
    x = _normals(rng, shape)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return f32_to_bf16_bits(x)


def rope_table_bits(max_seq_len: int, rope: int) -> np.ndarray:
    """[max_seq_len, rope] bf16 table of interleaved (cos, sin) of p * theta_i."""
    i = np.arange(rope // 2, dtype=np.float64)
    theta = 10000.0 ** (-2.0 * i / rope)
    ang = np.arange(max_seq_len, dtype=np.float64)[:, None] * theta[None, :]
    tab = np.empty((max_seq_len, rope), dtype=np.float64)
    tab[:, 0::2] = np.cos(ang)
    tab[:, 1::2] = np.sin(ang)
    return f32_to_bf16_bits(tab.astype(np.float32))


def _page_layout(rng: np.random.Generator, lengths: np.ndarray, page_size: int):
    pages_per_seq = [(int(n) + page_size - 1) // page_size for n in lengths]
    num_pages = max(1, sum(pages_per_seq))
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(1, max(pages_per_seq) if pages_per_seq else 1)
    table = np.zeros((len(lengths), max_pages), dtype=np.int32)
    base = 0
    for b, npg in enumerate(pages_per_seq):
        table[b, :npg] = perm[base:base + npg]
        base += npg
    return table, num_pages


def _fill_pool(rng: np.random.Generator, lengths: np.ndarray, table: np.ndarray,
               num_pages: int, page_size: int, depth: int, fp8: bool) -> np.ndarray:
    """Pool [num_pages, page_size, depth]; row (b, p) sits at the page table's slot."""
    total = int(np.sum(lengths))
    vals = _normals(rng, (total, depth))
    if fp8:
        amax = float(np.max(np.abs(vals))) if total else 1.0
        vals /= np.float32(amax)
        rows = f32_to_e4m3fn_codes(vals)
        pool = np.zeros((num_pages * page_size, depth), dtype=np.uint8)
    else:
        rows = f32_to_bf16_bits(vals)
        pool = np.zeros((num_pages * page_size, depth), dtype=np.uint16)
    del vals
    base = 0
    for b, n in enumerate(lengths):
        n = int(n)
        p = np.arange(n)
        slot = table[b, p // page_size].astype(np.int64) * page_size + p % page_size
        pool[slot] = rows[base:base + n]
        base += n
    return pool.reshape(num_pages, page_size, depth)


@dataclasses.dataclass
class PrefillWorkload:
    """A ragged prefill batch over a paged pool of raw (un-normalised, un-roped) rows."""
    name: str
    seed: int
    dims: Dims
    num_heads: int
    page_size: int
    buffer_token_size: int
    max_chunks: int
    fp8: bool
    new_lens: np.ndarray          # int64 [B]
    cached_lens: np.ndarray       # int64 [B]
    input_row_offsets: np.ndarray  # uint32 [B+1]
    cache_lengths: np.ndarray     # uint32 [B]
    page_table: np.ndarray        # int32 [B, max_pages]
    pool: np.ndarray              # uint16 or uint8 [num_pages, page_size, lora+rope]
    q: np.ndarray                 # uint16 or uint8 [T_q, H, nope+rope]
    gamma: np.ndarray             # uint16 [lora]
    freqs: np.ndarray             # uint16 [max_seq_len, rope]
    w_k: np.ndarray               # uint16 [H*nope, lora]
    w_uv: np.ndarray              # uint16 [H, v, lora]
    w_uk: np.ndarray              # uint16 [H, lora, nope]
    scale: float
    eps: float

    @property
    def batch(self) -> int:
        return len(self.new_lens)

    @property
    def total_q(self) -> int:
        return int(self.input_row_offsets[-1])

    @property
    def seq_lens(self) -> np.ndarray:
        return self.new_lens + self.cached_lens

    @property
    def num_pages(self) -> int:
        return self.pool.shape[0]

    @property
    def max_seq_len(self) -> int:
        return self.freqs.shape[0]


@dataclasses.dataclass
class DecodeWorkload:
    """One new token per sequence over a paged pool of rows used as stored."""
    name: str
    seed: int
    dims: Dims
    num_heads: int
    page_size: int
    fp8: bool
    context_lens: np.ndarray      # uint32 [B], includes the new token
    page_table: np.ndarray        # int32 [B, max_pages]
    pool: np.ndarray              # uint16 or uint8 [num_pages, page_size, lora+rope]
    q: np.ndarray                 # uint16 [B, H, nope+rope]
    w_uk: np.ndarray              # uint16 [H, lora, nope]
    w_uv: np.ndarray              # uint16 [H, v, lora]
    scale: float

    @property
    def batch(self) -> int:
        return len(self.context_lens)

    @property
    def num_pages(self) -> int:
        return self.pool.shape[0]


def make_prefill(name: str, seed: int, new_lens: Sequence[int],
                 cached_lens: Sequence[int], num_heads: int, page_size: int,
                 buffer_token_size: int, max_chunks: Optional[int] = None,
                 fp8: bool = False, dims: Dims = MLA_DIMS,
                 rng: Optional[np.random.Generator] = None,
                 eps: float = 1e-6) -> PrefillWorkload:
    """Build a prefill workload. Lengths are given (already drawn)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    new = np.asarray(new_lens, dtype=np.int64)
    cached = np.asarray(cached_lens, dtype=np.int64)
    lens = new + cached
    B = len(new)
    offs = np.zeros(B + 1, dtype=np.uint32)
    offs[1:] = np.cumsum(new)
    T = int(buffer_token_size)
    need = max(1, max((int(L) + T - 1) // T for L in lens) if B else 1)
    C = need if max_chunks is None else int(max_chunks)
    table, num_pages = _page_layout(rng, lens, page_size)
    H = num_heads
    tq = int(offs[-1])
    if fp8:
        qf = _normals(rng, (tq, H, dims.q_depth))
        amax = float(np.max(np.abs(qf))) if tq else 1.0
        qf /= np.float32(amax)
        q = f32_to_e4m3fn_codes(qf)
        del qf
    else:
        q = _normal_bits(rng, (tq, H, dims.q_depth))
    pool = _fill_pool(rng, lens, table, num_pages, page_size, dims.cache_depth, fp8)
    gamma = _normal_bits(rng, (dims.lora,), std=0.1, mean=1.0)
    wstd = 1.0 / math.sqrt(512.0)
    w_k = _normal_bits(rng, (H * dims.nope, dims.lora), std=wstd)
    w_uv = _normal_bits(rng, (H, dims.v, dims.lora), std=wstd)
    w_uk = _normal_bits(rng, (H, dims.lora, dims.nope), std=wstd)
    max_seq_len = max(1, int(lens.max()) if B else 1)
    freqs = rope_table_bits(max_seq_len, dims.rope)
    return PrefillWorkload(
        name=name, seed=seed, dims=dims, num_heads=H, page_size=page_size,
        buffer_token_size=T, max_chunks=C, fp8=fp8, new_lens=new,
        cached_lens=cached, input_row_offsets=offs,
        cache_lengths=cached.astype(np.uint32), page_table=table, pool=pool, q=q,
        gamma=gamma, freqs=freqs, w_k=w_k, w_uv=w_uv, w_uk=w_uk,
        scale=1.0 / math.sqrt(dims.q_depth), eps=eps)


def make_decode(name: str, seed: int, context_lens: Sequence[int], num_heads: int,
                page_size: int, fp8: bool = False, dims: Dims = MLA_DIMS,
                rng: Optional[np.random.Generator] = None) -> DecodeWorkload:
    """Build an absorbed-decode workload. Context lengths include the new token."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64)
    table, num_pages = _page_layout(rng, ctx, page_size)
    H = num_heads
    q = _normal_bits(rng, (len(ctx), H, dims.q_depth))
    pool = _fill_pool(rng, ctx, table, num_pages, page_size, dims.cache_depth, fp8)
    wstd = 1.0 / math.sqrt(512.0)
    w_uv = _normal_bits(rng, (H, dims.v, dims.lora), std=wstd)
    w_uk = _normal_bits(rng, (H, dims.lora, dims.nope), std=wstd)
    return DecodeWorkload(
        name=name, seed=seed, dims=dims, num_heads=H, page_size=page_size, fp8=fp8,
        context_lens=ctx.astype(np.uint32), page_table=table, pool=pool, q=q,
        w_uk=w_uk, w_uv=w_uv, scale=1.0 / math.sqrt(dims.q_depth))


# Named workloads. Sizes follow DeepSeek V2/V3 MLA (128 heads, 128 nope + 64 rope
# query depth, 128 value depth, 512-wide latent).
PREFILL_RECIPES = {
    # 2 sequences, 5 and 11 new tokens over 0 and 7 cached, 4 heads, 8-token
    # chunks so that several chunks are planned.
    "tiny_b2": dict(seed=0, new=[5, 11], cached=[0, 7], H=4, ps=16, T=8, C=4),
    # one 4096-token prompt, no cache, 128 heads.
    "dsv3_prefill_4k": dict(seed=1, new=[4096], cached=[0], H=128, ps=128, T=8192, C=2),
    # 16 prompts of U{128..4096} new tokens over U{0..8192} cached tokens.
    "ragged_b16_cached": dict(seed=2, B=16, new=(128, 4096), cached=(0, 8192), H=128,
                              ps=128, T=8192, C=3),
    # as above with 8 prompts, q and the pool in float8_e4m3fn.
    "fp8_ragged_b8_cached": dict(seed=3, B=8, new=(128, 4096), cached=(0, 8192), H=128,
                                 ps=128, T=8192, C=3, fp8=True),
}

DECODE_RECIPES = {
    # 64 sequences, one new token each, contexts U{4096..32768}, 128 heads.
    "decode_b64": dict(seed=4, B=64, ctx=(4096, 32768), H=128, ps=64),
    "decode_b64_fp8": dict(seed=4, B=64, ctx=(4096, 32768), H=128, ps=64, fp8=True),
}


def _draw_lengths(r: dict, rng: np.random.Generator):
    if isinstance(r["new"], tuple):
        lo, hi = r["new"]
        new = rng.integers(lo, hi + 1, size=r["B"])
        clo, chi = r["cached"]
        cached = rng.integers(clo, chi + 1, size=r["B"])
    else:
        new, cached = r["new"], r["cached"]
    return np.asarray(new, dtype=np.int64), np.asarray(cached, dtype=np.int64)


def prefill_recipe_lengths(name: str):
    """(new_lens, cached_lens, buffer_token_size, max_chunks) of a named workload,
    without drawing its tensors."""
    r = PREFILL_RECIPES[name]
    new, cached = _draw_lengths(r, np.random.default_rng(r["seed"]))
    return new, cached, r["T"], r["C"]


def prefill_recipe(name: str, **over) -> PrefillWorkload:
    r = dict(PREFILL_RECIPES[name])
    r.update(over)
    rng = np.random.default_rng(r["seed"])
    new, cached = _draw_lengths(r, rng)
    return make_prefill(name, r["seed"], new, cached, r["H"], r["ps"], r["T"],
                        r.get("C"), fp8=r.get("fp8", False), rng=rng)


def decode_recipe(name: str, **over) -> DecodeWorkload:
    r = dict(DECODE_RECIPES[name])
    r.update(over)
    rng = np.random.default_rng(r["seed"])
    lo, hi = r["ctx"]
    ctx = rng.integers(lo, hi + 1, size=r["B"])
    return make_decode(name, r["seed"], ctx, r["H"], r["ps"], fp8=r.get("fp8", False),
                       rng=rng)
