"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each check is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign, an off-by-one mask, a transposed operand, a wrong pairing) fails
at least one of them. None of them re-types an oracle formula or re-calls the
oracle's own library routine on the same expression.
"""
import dataclasses
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, oracle
from workloads import Dims, make_decode, make_prefill, prefill_recipe
from workloads.gen import rope_table_bits

TINY = Dims(nope=6, rope=4, v=5, lora=12)


# ---------------------------------------------------------------------------
# storage decoding
# ---------------------------------------------------------------------------

def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(nan, [math.isnan(brute.e4m3fn(c)) for c in codes])
    assert np.array_equal(ref[~nan], np.array([brute.e4m3fn(c) for c in codes])[~nan])
    # OCP e4m3fn facts: largest finite 448, smallest subnormal 2^-9, no infinity
    assert np.nanmax(got) == 448.0
    assert got[1] == 2.0 ** -9
    assert not np.isinf(got).any()


def test_bf16_sample_codes_match_torch():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, 20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    some = bits[:200]
    assert all(brute.bf16(b) == g or (math.isnan(g)) for b, g in zip(some, got[:200]))


# ---------------------------------------------------------------------------
# plan (mla_prefill_plan page)
# ---------------------------------------------------------------------------

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_plan_worked_example_two_sequences():
    """Hand-worked from the page's Args definitions (tests/golden/
    plan_two_sequences.json holds the derivation): lengths 5 (0 cached) and
    18 (7 cached + 11 new), 8-token chunks, 4 chunk slots."""
    g = json.load(open(os.path.join(GOLDEN, "plan_two_sequences.json")))
    bro, co, bl = oracle.plan(g["input_row_offsets"], g["cache_lengths"],
                              g["buffer_token_size"], g["max_chunks"])
    assert bro.tolist() == g["buffer_row_offsets"]
    assert co.tolist() == g["cache_offsets"]
    assert bl.tolist() == g["buffer_lengths"]
    assert bro.dtype == np.uint32 and co.dtype == np.uint32 and bl.dtype == np.int32


def _check_invariants(offs, clen, T, C, bro, co, bl):
    B = len(clen)
    L = [offs[b + 1] - offs[b] + clen[b] for b in range(B)]
    used = [c for c in range(C) if bl[c] != -1]
    # -1 only after the last used chunk
    if used:
        assert used == list(range(len(used)))
    for c in range(C):
        row = [int(x) for x in bro[c]]
        assert row[0] == 0
        assert all(row[i] <= row[i + 1] for i in range(B))  # monotone over b
        if bl[c] != -1:
            assert bl[c] == row[B] > 0
        else:
            assert row[B] == 0
    for b in range(B):
        covered = []
        for c in range(C):
            n = int(bro[c, b + 1]) - int(bro[c, b])
            assert n <= T
            covered.extend(range(int(co[c, b]), int(co[c, b]) + n))
            if c:
                assert co[c, b] >= co[c - 1, b]  # monotone over chunks
        assert covered == list(range(L[b]))  # every token exactly once, in order


def test_plan_closed_form_equals_token_walk_exhaustive():
    for B in (1, 2):
        for lens in itertools.product(range(0, 7), repeat=2 * B):
            new, cached = lens[:B], lens[B:]
            offs = [0]
            for n in new:
                offs.append(offs[-1] + n)
            for T in range(1, 6):
                C = max(1, (max(a + b for a, b in zip(new, cached)) + T - 1) // T) + 1
                bro, co, bl = oracle.plan(offs, cached, T, C)
                wbro, wco, wbl = brute.plan_walk(offs, cached, T, C)
                assert bro.tolist() == wbro and co.tolist() == wco and bl.tolist() == wbl
                _check_invariants(offs, cached, T, C, bro, co, bl)


def test_plan_random_batches_invariants_and_walk():
    rng = np.random.default_rng(5)
    for _ in range(300):
        B = int(rng.integers(1, 9))
        new = rng.integers(0, 40, B)
        cached = rng.integers(0, 60, B)
        offs = np.concatenate([[0], np.cumsum(new)]).astype(np.uint32)
        T = int(rng.integers(1, 33))
        need = max(1, int(((new + cached).max() + T - 1) // T))
        C = need + int(rng.integers(0, 3))
        bro, co, bl = oracle.plan(offs, cached, T, C)
        wbro, wco, wbl = brute.plan_walk(offs, cached, T, C)
        assert bro.tolist() == wbro and co.tolist() == wco and bl.tolist() == wbl
        _check_invariants([int(x) for x in offs], [int(x) for x in cached], T, C, bro, co, bl)


# ---------------------------------------------------------------------------
# RMSNorm and RoPE
# ---------------------------------------------------------------------------

def test_rms_norm_unit_rms_scale_invariance_and_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 512))
    y = oracle.rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-13)
    assert np.allclose(oracle.rms_norm(3.5 * x, np.ones(512), 0.0), y, rtol=1e-13)
    g = 1 + 0.1 * rng.standard_normal(512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(g),
                                       eps=1e-6).numpy()
    assert np.allclose(oracle.rms_norm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-14)


def _exact_table(positions, rope):
    i = np.arange(rope // 2)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * 10000.0 ** (-2.0 * i / rope)
    t = np.empty((len(positions), rope))
    t[:, 0::2] = np.cos(ang)
    t[:, 1::2] = np.sin(ang)
    return t


def test_rope_identity_norm_composition_and_complex_multiply():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((5, 64))
    # position 0: the stored table row is (1, 0, 1, 0, ...) exactly
    f0 = oracle.bf16_to_f64(rope_table_bits(1, 64))
    assert np.array_equal(f0[0], np.tile([1.0, 0.0], 32))
    assert np.array_equal(oracle.rope(y, np.repeat(f0, 5, axis=0)), y)
    # pair norms preserved
    F = _exact_table([3, 17, 100, 2000, 4095], 64)
    r = oracle.rope(y, F)
    assert np.allclose(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(y[:, 0::2], y[:, 1::2]),
                       rtol=1e-13)
    # R(p1) R(p2) = R(p1 + p2)
    p1, p2 = np.array([5, 9, 300, 1000, 7]), np.array([2, 40, 11, 77, 4000])
    two = oracle.rope(oracle.rope(y, _exact_table(p1, 64)), _exact_table(p2, 64))
    assert np.allclose(two, oracle.rope(y, _exact_table(p1 + p2, 64)), rtol=1e-9, atol=1e-11)
    # complex multiply of adjacent pairs by cis
    yc = torch.view_as_complex(torch.from_numpy(y).reshape(5, 32, 2).contiguous())
    fc = torch.view_as_complex(torch.from_numpy(F).reshape(5, 32, 2).contiguous())
    ref = torch.view_as_real(yc * fc).reshape(5, 64).numpy()
    assert np.allclose(r, ref, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# the two tiers against each other, on tiny inputs
# ---------------------------------------------------------------------------

def _tiny_prefill(seed, new, cached, H=3, ps=4, T=3, fp8=False, dims=TINY):
    return make_prefill("tiny", seed, new, cached, H, ps, T, fp8=fp8, dims=dims)


@pytest.mark.parametrize("fp8", [False, True])
def test_brute_equals_oracle_prefill_tiny_dims(fp8):
    wl = _tiny_prefill(7, [3, 0, 6, 1], [2, 4, 0, 9], fp8=fp8)
    ref = np.array(brute.prefill(wl))
    got = oracle.prefill(wl)
    assert ref.shape == got.shape
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_brute_equals_oracle_decode_tiny_dims():
    for fp8 in (False, True):
        wl = make_decode("tinyd", 3, [1, 5, 9], 3, 4, fp8=fp8, dims=TINY)
        assert np.allclose(oracle.decode(wl), np.array(brute.decode(wl)), rtol=1e-12, atol=1e-13)


def test_brute_equals_oracle_prefill_two_sequence_batch_full_dims():
    wl = prefill_recipe("tiny_b2")
    ref = np.array(brute.prefill(wl))
    got = oracle.prefill(wl)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# attention closed forms and library references
# ---------------------------------------------------------------------------

def _with_q(wl, qvals):
    from workloads import f32_to_bf16_bits
    wl.q = f32_to_bf16_bits(np.asarray(qvals, dtype=np.float32))
    return wl


def test_single_visible_key_returns_its_value():
    wl = _tiny_prefill(3, [4], [0])
    dec = oracle.Decoded(wl)
    out = oracle.prefill(wl, dec)
    latn, _ = dec.seq_keys(0)
    _, v = oracle.up_project(latn, dec.w_k, dec.w_uv, dec.H)
    assert np.allclose(out[0], v[0], rtol=1e-13, atol=1e-14)  # query 0 sees key 0 only


def test_zero_query_gives_prefix_mean_of_values():
    wl = _tiny_prefill(4, [5, 3], [2, 0])
    wl = _with_q(wl, np.zeros(wl.q.shape))
    dec = oracle.Decoded(wl)
    out = oracle.prefill(wl, dec)
    for b in range(2):
        latn, _ = dec.seq_keys(b)
        _, v = oracle.up_project(latn, dec.w_k, dec.w_uv, dec.H)
        for i in range(dec.offs[b + 1] - dec.offs[b]):
            P = dec.clen[b] + i
            assert np.allclose(out[dec.offs[b] + i], v[:P + 1].mean(axis=0), rtol=1e-12)


def test_softmax_weights_sum_to_one_constant_values():
    """With every value row equal to the same vector, each output equals it."""
    rng = np.random.default_rng(5)
    n, L, H = 6, 9, 3
    q = rng.standard_normal((n, H, 10))
    k_nope = rng.standard_normal((L, H, 6))
    krope = rng.standard_normal((L, 4))
    const = rng.standard_normal(5)
    v = np.broadcast_to(const, (L, H, 5)).copy()
    out = oracle.attend_sequence(q, k_nope, krope, v, 3 + np.arange(n), np.arange(L), 0.4, 6)
    assert np.allclose(out, np.broadcast_to(const, out.shape), rtol=1e-13, atol=1e-14)
    # and every output is a convex combination of the visible values
    v = rng.standard_normal((L, H, 5))
    out = oracle.attend_sequence(q, k_nope, krope, v, 3 + np.arange(n), np.arange(L), 0.4, 6)
    for i in range(n):
        vis = v[:3 + i + 1]
        assert (out[i] <= vis.max(axis=0) + 1e-12).all() and (out[i] >= vis.min(axis=0) - 1e-12).all()


def test_matches_torch_sdpa_with_bottom_right_mask():
    wl = _tiny_prefill(6, [5, 7], [4, 0], H=2)
    dec = oracle.Decoded(wl)
    out = oracle.prefill(wl, dec)
    for b in range(2):
        n = dec.offs[b + 1] - dec.offs[b]
        latn, krope = dec.seq_keys(b)
        k_nope, v = oracle.up_project(latn, dec.w_k, dec.w_uv, dec.H)
        L = latn.shape[0]
        K = np.concatenate([k_nope, np.broadcast_to(krope[:, None, :], (L, dec.H, dec.rope))], -1)
        q = torch.from_numpy(dec.q[dec.offs[b]:dec.offs[b + 1]]).permute(1, 0, 2)
        k = torch.from_numpy(K).permute(1, 0, 2)
        vv = torch.from_numpy(np.ascontiguousarray(v)).permute(1, 0, 2)
        # bottom-right aligned causal mask: the last query sees every key
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, vv, attn_mask=mask, scale=wl.scale).permute(1, 0, 2).numpy()
        assert np.allclose(out[dec.offs[b]:dec.offs[b + 1]], ref, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("T", [1, 3, 8, 1000])
def test_chunk_size_invariance(T):
    wl = _tiny_prefill(8, [5, 9, 2], [6, 0, 11])
    ref = oracle.prefill(wl)
    got, (bro, co, bl) = oracle.prefill_chunked(wl, buffer_token_size=T)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_page_permutation_invariance():
    wl = _tiny_prefill(9, [4, 6], [7, 3], ps=2)
    ref = oracle.prefill(wl)
    rng = np.random.default_rng(0)
    perm = rng.permutation(wl.num_pages)  # new position of each old page
    pool = np.empty_like(wl.pool)
    pool[perm] = wl.pool
    wl.pool = pool
    wl.page_table = perm[wl.page_table].astype(np.int32)
    assert np.allclose(oracle.prefill(wl), ref, rtol=1e-13, atol=1e-14)


def test_sampled_rows_equal_full_output():
    wl = _tiny_prefill(10, [7, 4], [3, 9])
    full = oracle.prefill(wl)
    samples = [(0, 0), (3, 2), (6, 1), (8, 0), (10, 2)]
    got = oracle.prefill_sampled(wl, samples)
    for i, (t, h) in enumerate(samples):
        assert np.allclose(got[i], full[t, h], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# decode: absorbed form against the up-projected form, splits, SDPA-MQA
# ---------------------------------------------------------------------------

def _decode_from_prefill(wl):
    """Decode workload whose rows are the processed prefill keys, w_uk taken from w_k."""
    from workloads import DecodeWorkload
    dec = oracle.Decoded(wl)
    d = wl.dims
    rows = np.zeros((wl.num_pages * wl.page_size, d.cache_depth))
    for b in range(dec.B):
        latn, krope = dec.seq_keys(b)
        p = np.arange(latn.shape[0])
        slot = wl.page_table[b, p // wl.page_size].astype(np.int64) * wl.page_size \
            + p % wl.page_size
        rows[slot, :d.lora] = latn
        rows[slot, d.lora:] = krope
    w_uk = wl.w_k.reshape(wl.num_heads, d.nope, d.lora).transpose(0, 2, 1).copy()
    last = [int(x) - 1 for x in wl.input_row_offsets[1:]]
    dwl = DecodeWorkload(name="equiv", seed=0, dims=d, num_heads=wl.num_heads,
                         page_size=wl.page_size, fp8=False,
                         context_lens=wl.seq_lens.astype(np.uint32),
                         page_table=wl.page_table, pool=None, q=wl.q[last], w_uk=w_uk,
                         w_uv=wl.w_uv, scale=wl.scale)
    return dwl, rows.reshape(wl.num_pages, wl.page_size, d.cache_depth), last


def test_absorbed_decode_equals_up_projected_prefill():
    wl = _tiny_prefill(12, [3, 5, 2], [4, 0, 6], H=4)
    ref = oracle.prefill(wl)
    dwl, rows, last = _decode_from_prefill(wl)
    ddec = oracle.DecodedDecode.__new__(oracle.DecodedDecode)
    d = wl.dims
    ddec.wl, ddec.nope, ddec.rope, ddec.v, ddec.lora = dwl, d.nope, d.rope, d.v, d.lora
    ddec.H = wl.num_heads
    ddec.q = oracle.bf16_to_f64(dwl.q)
    ddec.pool = rows
    ddec.w_uk = oracle.bf16_to_f64(dwl.w_uk)
    ddec.w_uv = oracle.bf16_to_f64(dwl.w_uv)
    ddec.ctx = [int(x) for x in dwl.context_lens]
    got = oracle.decode(dwl, ddec)
    assert np.allclose(got, ref[last], rtol=1e-10, atol=1e-12)


def test_absorbed_decode_equals_up_projected_prefill_full_dims():
    wl = prefill_recipe("tiny_b2")
    ref = oracle.prefill(wl)
    dwl, rows, last = _decode_from_prefill(wl)
    ddec = oracle.DecodedDecode.__new__(oracle.DecodedDecode)
    d = wl.dims
    ddec.wl, ddec.nope, ddec.rope, ddec.v, ddec.lora = dwl, d.nope, d.rope, d.v, d.lora
    ddec.H = wl.num_heads
    ddec.q = oracle.bf16_to_f64(dwl.q)
    ddec.pool = rows
    ddec.w_uk = oracle.bf16_to_f64(dwl.w_uk)
    ddec.w_uv = oracle.bf16_to_f64(dwl.w_uv)
    ddec.ctx = [int(x) for x in dwl.context_lens]
    got = oracle.decode(dwl, ddec)
    assert np.allclose(got, ref[last], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 5, 16])
def test_decode_split_invariance(splits):
    wl = make_decode("tinyd", 13, [1, 7, 30, 16], 3, 4, dims=TINY)
    assert np.allclose(oracle.decode_split(wl, splits), oracle.decode(wl), rtol=1e-12, atol=1e-13)


def test_decode_matches_torch_sdpa_single_kv_head():
    wl = make_decode("tinyd", 14, [9, 3], 4, 4, dims=TINY)
    dec = oracle.DecodedDecode(wl)
    out = oracle.decode(wl, dec)
    d = wl.dims
    for b in range(2):
        Z = oracle.gather_rows(dec.pool, wl.page_table, b, np.arange(dec.ctx[b]), wl.page_size)
        # up-projected multi-head form: per head, K = [Z_lat @ w_uk[h] | Z_rope],
        # V = Z_lat @ w_uv[h]^T
        for h in range(dec.H):
            K = np.concatenate([Z[:, :d.lora] @ dec.w_uk[h], Z[:, d.lora:]], axis=1)
            V = Z[:, :d.lora] @ dec.w_uv[h].T
            q = torch.from_numpy(dec.q[b, h][None, None, :])
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, torch.from_numpy(K)[None], torch.from_numpy(V)[None], scale=wl.scale)
            assert np.allclose(out[b, h], ref[0, 0].numpy(), rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# KV write path: every new token lands in exactly the slot of its position
# ---------------------------------------------------------------------------

def test_kv_write_places_each_token_and_touches_nothing_else():
    rng = np.random.default_rng(11)
    ps, num_pages, maxp = 4, 16, 5
    cached = [3, 0, 9]
    new = [6, 2, 0]
    off = np.concatenate([[0], np.cumsum(new)])
    pt = rng.permutation(num_pages)[:3 * maxp].reshape(3, maxp).astype(np.int32)
    pt[0, 2] = -1                      # the page of sequence 0's last token is missing
    pool = rng.standard_normal((num_pages, ps, 576))
    x = rng.standard_normal((int(off[-1]), 576))
    freqs = np.zeros((64, 64))
    freqs[:, 0::2] = 1.0               # identity rotation
    out = oracle.kv_write(pool, pt, x, off, cached, np.ones(512), freqs, 0.0, ps)
    expect = pool.copy()
    written = set()
    for b in range(3):                 # one token at a time, by hand
        for i in range(new[b]):
            p = cached[b] + i
            page = int(pt[b, p // ps])
            if page < 0:
                continue
            row = x[off[b] + i]
            lat = row[:512] / math.sqrt(sum(v * v for v in row[:512]) / 512)
            expect[page, p % ps] = np.concatenate([lat, row[512:]])
            written.add((page, p % ps))
    assert len(written) == 7           # 5 of 6 (one page missing) + 2 + 0 tokens
    assert np.allclose(out, expect, rtol=1e-12, atol=0)
    for pg in range(num_pages):
        for sl in range(ps):
            if (pg, sl) not in written:
                assert np.array_equal(out[pg, sl], pool[pg, sl])


def test_kv_write_rotates_by_the_position_angle():
    # one token at position 5: rope part (1, 0) pairs rotate to (cos, sin) of
    # that position's angles; a unit-rms latent with gamma 2 doubles
    ps = 8
    pt = np.array([[0]], dtype=np.int32)
    pool = np.zeros((1, ps, 576))
    x = np.zeros((1, 576))
    x[0, :512] = 1.0
    x[0, 512::2] = 1.0
    ang = np.outer(np.arange(8), np.arange(32) * 0.1)
    freqs = np.zeros((8, 64))
    freqs[:, 0::2], freqs[:, 1::2] = np.cos(ang), np.sin(ang)
    out = oracle.kv_write(pool, pt, x, [0, 1], [5], np.full(512, 2.0), freqs, 0.0, ps)
    assert np.allclose(out[0, 5, :512], 2.0, rtol=1e-15)
    assert np.allclose(out[0, 5, 512::2], np.cos(ang[5]), atol=1e-15)
    assert np.allclose(out[0, 5, 513::2], np.sin(ang[5]), atol=1e-15)
    assert np.array_equal(out[0, :5], pool[0, :5]) and np.array_equal(out[0, 6:], pool[0, 6:])


# ---------------------------------------------------------------------------
# Sparse decode: attention over an explicit list of pool rows
# ---------------------------------------------------------------------------

def _sparse_inputs(seed=21, ctx=(5, 40, 1), H=4):
    wl = make_decode("sp", seed, list(ctx), H, 8, dims=Dims(nope=16, rope=8, v=16, lora=32))
    dec = oracle.DecodedDecode(wl)
    ps = wl.page_size
    idx = np.zeros((len(ctx), max(ctx) + 3), dtype=np.int32)
    for b, n in enumerate(ctx):   # the physical row of every position, in order
        for p in range(n):
            idx[b, p] = wl.page_table[b, p // ps] * ps + p % ps
    return wl, dec, idx


def test_sparse_decode_over_the_context_in_order_is_decode():
    wl, dec, idx = _sparse_inputs()
    got = oracle.decode_sparse(dec.q, dec.pool, idx, wl.context_lens, dec.w_uk, dec.w_uv,
                               wl.scale, dec.nope, dec.lora)
    assert np.allclose(got, oracle.decode(wl), rtol=1e-12, atol=1e-14)


def test_sparse_decode_is_a_set_function_and_a_single_row_returns_its_projection():
    wl, dec, idx = _sparse_inputs(seed=22, ctx=(30, 1, 12))
    rng = np.random.default_rng(3)
    shuffled = idx.copy()
    for b, n in enumerate(wl.context_lens):
        shuffled[b, :n] = rng.permutation(idx[b, :n])
    a = oracle.decode_sparse(dec.q, dec.pool, idx, wl.context_lens, dec.w_uk, dec.w_uv,
                             wl.scale, dec.nope, dec.lora)
    c = oracle.decode_sparse(dec.q, dec.pool, shuffled, wl.context_lens, dec.w_uk, dec.w_uv,
                             wl.scale, dec.nope, dec.lora)
    assert np.allclose(a, c, rtol=1e-12, atol=1e-14)
    # sequence 1 lists one row: softmax weight 1, output w_uv[h] @ that row's latent
    z = dec.pool.reshape(-1, dec.pool.shape[-1])[idx[1, 0], :dec.lora]
    assert np.allclose(a[1], np.einsum("hdl,l->hd", dec.w_uv, z), rtol=1e-12, atol=1e-14)


def test_sparse_decode_of_an_empty_list_is_zero():
    wl, dec, idx = _sparse_inputs()
    lens = np.array([5, 0, 1])
    got = oracle.decode_sparse(dec.q, dec.pool, idx, lens, dec.w_uk, dec.w_uv, wl.scale,
                               dec.nope, dec.lora)
    assert np.array_equal(got[1], np.zeros_like(got[1])) and np.abs(got[0]).sum() > 0


# ---------------------------------------------------------------------------
# attention sinks: one more logit in the softmax denominator
# ---------------------------------------------------------------------------

def test_sink_with_zero_query_divides_the_prefix_sum_by_count_plus_exp_sink():
    # q = 0 makes every score 0: each visible key weighs 1 / (n + e^sink)
    wl = _tiny_prefill(4, [5, 3], [2, 0])
    wl = _with_q(wl, np.zeros(wl.q.shape))
    dec = oracle.Decoded(wl)
    sinks = np.array([0.7, -1.3])
    out = oracle.prefill(wl, dec, sinks=sinks)
    for b in range(2):
        latn, _ = dec.seq_keys(b)
        _, v = oracle.up_project(latn, dec.w_k, dec.w_uv, dec.H)
        for i in range(dec.offs[b + 1] - dec.offs[b]):
            P = dec.clen[b] + i
            expect = v[:P + 1].sum(axis=0) / (P + 1 + math.exp(sinks[b]))
            assert np.allclose(out[dec.offs[b] + i], expect, rtol=1e-12)


def test_sink_of_minus_infinity_is_no_sink_and_a_huge_sink_silences():
    wl = _tiny_prefill(4, [5, 3], [2, 0])
    dec = oracle.Decoded(wl)
    base = oracle.prefill(wl, dec)
    assert np.array_equal(oracle.prefill(wl, dec, sinks=np.array([-np.inf, -np.inf])), base)
    quiet = oracle.prefill(wl, dec, sinks=np.array([200.0, 200.0]))
    assert np.abs(quiet).max() < 1e-60
    dwl = make_decode("sk", 31, [7, 1, 20], 4, 4, dims=Dims(nope=16, rope=8, v=16, lora=32))
    ddec = oracle.DecodedDecode(dwl)
    assert np.array_equal(oracle.decode(dwl, ddec, sinks=np.full(3, -np.inf)), oracle.decode(dwl, ddec))


def test_decode_sink_with_zero_query_closed_form():
    dwl = make_decode("sk0", 32, [7, 1, 20], 4, 4, dims=Dims(nope=16, rope=8, v=16, lora=32))
    dwl = dataclasses.replace(dwl, q=np.zeros_like(dwl.q))
    ddec = oracle.DecodedDecode(dwl)
    sinks = np.array([1.5, -0.25, 3.0])
    out = oracle.decode(dwl, ddec, sinks=sinks)
    for b, n in enumerate(ddec.ctx):
        Z = oracle.gather_rows(ddec.pool, dwl.page_table, b, np.arange(n), dwl.page_size)
        olat = Z[:, :ddec.lora].sum(axis=0) / (n + math.exp(sinks[b]))
        assert np.allclose(out[b], np.einsum("hdl,l->hd", ddec.w_uv, olat), rtol=1e-12)


# ---------------------------------------------------------------------------
# the graph op as one call: write, then prefill or decode by max_seq_len
# ---------------------------------------------------------------------------

def _unified_inputs(wl):
    """Values of a prefill workload, the pool holding every position's row
    processed (written by kv_write from the raw rows, position by position)."""
    dec = oracle.Decoded(wl)
    lens = [dec.clen[b] + dec.offs[b + 1] - dec.offs[b] for b in range(dec.B)]
    raw = np.concatenate([oracle.gather_rows(dec.pool, wl.page_table, b, np.arange(n),
                                             wl.page_size) for b, n in enumerate(lens)])
    offs = np.concatenate([[0], np.cumsum(lens)])
    done = oracle.kv_write(np.zeros_like(dec.pool), wl.page_table, raw, offs, np.zeros(dec.B),
                           dec.gamma, dec.freqs, wl.eps, wl.page_size, dec.lora)
    return dec, raw, offs, done


def _unified(wl, dec, pool, max_seq_len, **kw):
    return oracle.prefill_decode(dec.q, dec.offs, dec.clen, pool, wl.page_table, wl.page_size,
                                 dec.w_k, dec.w_uk, dec.w_uv, dec.gamma, dec.freqs, wl.scale,
                                 wl.eps, max_seq_len, nope=dec.nope, lora=dec.lora, **kw)


def test_unified_prefill_over_the_written_cache_is_prefill_over_raw_rows():
    wl = _tiny_prefill(41, [3, 5, 2], [4, 0, 6], H=3)
    dec, raw, offs, done = _unified_inputs(wl)
    ref = oracle.prefill(wl, dec)
    got, pool = _unified(wl, dec, done, 5)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)
    assert np.array_equal(pool, done)
    # the call itself writing the new tokens: only the cached positions are in
    # the pool beforehand, the new tokens' raw rows come in as kv_input
    cached_only = done.copy()
    flat = cached_only.reshape(-1, cached_only.shape[-1])
    new_rows = []
    for b in range(dec.B):
        p = dec.clen[b] + np.arange(dec.offs[b + 1] - dec.offs[b])
        flat[wl.page_table[b, p // wl.page_size].astype(np.int64) * wl.page_size
             + p % wl.page_size] = 7.0            # stale values the write must replace
        new_rows.append(raw[offs[b] + p])
    got2, pool2 = _unified(wl, dec, cached_only, 5, kv_input=np.concatenate(new_rows))
    assert np.allclose(got2, ref, rtol=1e-11, atol=1e-13)
    assert np.allclose(pool2, done, rtol=1e-15, atol=0)


def test_unified_decode_branch_equals_the_prefill_branch_for_one_token():
    # absorption: with w_uk[h] = w_k[h]^T the absorbed decode of one new token
    # equals the up-projected prefill of the same token
    wl = _tiny_prefill(42, [1, 1, 1], [4, 0, 9], H=3)
    dec, raw, offs, done = _unified_inputs(wl)
    dec.w_uk = dec.w_k.reshape(dec.H, dec.nope, dec.lora).transpose(0, 2, 1).copy()
    a, _ = _unified(wl, dec, done, 1)
    b, _ = _unified(wl, dec, done, 2)
    assert np.allclose(a, b, rtol=1e-10, atol=1e-12)
    assert np.allclose(a, oracle.prefill(wl, dec), rtol=1e-10, atol=1e-12)
    # sparse over every context row in order is the dense decode branch
    idx = np.full((dec.B, 12), -1, dtype=np.int32)
    for bb in range(dec.B):
        p = np.arange(dec.clen[bb] + 1)
        idx[bb, :len(p)] = wl.page_table[bb, p // wl.page_size] * wl.page_size + p % wl.page_size
    c, _ = _unified(wl, dec, done, 1, d_indices=idx,
                    topk_lengths=[dec.clen[bb] + 1 for bb in range(dec.B)])
    assert np.allclose(c, a, rtol=1e-12, atol=1e-14)
    # sinks pass through to the branch
    s = np.array([0.5, -1.0, 2.0])
    d1, _ = _unified(wl, dec, done, 1, sinks=s)
    d2, _ = _unified(wl, dec, done, 2, sinks=s)
    assert np.allclose(d1, d2, rtol=1e-10, atol=1e-12) and not np.allclose(d1, a)


def test_unified_decode_rejects_ragged_batches_and_zero_length_is_empty():
    wl = _tiny_prefill(43, [2, 1], [3, 1], H=2)
    dec, raw, offs, done = _unified_inputs(wl)
    with pytest.raises(ValueError):
        _unified(wl, dec, done, 1)
    got, pool = _unified(wl, dec, done, 0)
    assert np.array_equal(got, np.zeros_like(got)) and np.array_equal(pool, done)
