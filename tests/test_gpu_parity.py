"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Tolerances: the plan is integer work and must be bit-exact. bf16 outputs must be
within max-abs 2e-2 and mean-abs 2e-3 of the fp64 oracle; outputs computed from
float8_e4m3fn inputs within max-abs 6e-2. Intermediate products (gather, K/V
up-projection) are checked per element against a bound derived from their
rounding: one bf16 rounding of the result (relative 2^-8) plus fp32
accumulation error.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

from oracle import oracle
from workloads import (Dims, decode_recipe, make_decode, make_prefill, prefill_recipe,
                       prefill_recipe_lengths, f32_to_bf16_bits, f32_to_e4m3fn_codes)
from workloads.device import bf16_bits, decode_tensors, fp8_bits, prefill_tensors
from workloads.gen import rope_table_bits

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, FP8_MAX = 2e-2, 2e-3, 6e-2


@pytest.fixture(scope="module")
def B():
    from mla_chunked_prefill_amd import binding
    binding.load()
    return binding


def _f64(t):
    return oracle.bf16_to_f64(bf16_bits(t))


def _say(msg):
    print(msg, flush=True)


def _u32(a):
    return torch.from_numpy(np.asarray(a, dtype=np.uint32)).cuda()


# ---------------------------------------------------------------------------
# plan: bit-exact
# ---------------------------------------------------------------------------

def _plan_gpu(B, offs, clen, T, C):
    bro, co, bl, need = B.plan(_u32(offs), _u32(clen), T, C)
    torch.cuda.synchronize()
    return (bro.cpu().numpy(), co.cpu().numpy(), bl.cpu().numpy(), int(need.cpu()[0]))


@pytest.mark.parametrize("name", ["tiny_b2", "dsv3_prefill_4k", "ragged_b16_cached",
                                  "fp8_ragged_b8_cached"])
def test_plan_bit_exact_named(B, name):
    new, cached, T, C = prefill_recipe_lengths(name)
    offs = np.concatenate([[0], np.cumsum(new)])
    _say(f"plan {name}")
    g = _plan_gpu(B, offs, cached, T, C)
    r = oracle.plan(offs, cached, T, C)
    for a, b in zip(g[:3], r):
        assert a.dtype == b.dtype and np.array_equal(a, b)
    assert g[3] == -(-int((new + cached).max()) // T)


def test_plan_golden_worked_example(B):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "plan_two_sequences.json")))
    bro, co, bl, need = _plan_gpu(B, g["input_row_offsets"], g["cache_lengths"],
                                  g["buffer_token_size"], g["max_chunks"])
    assert bro.tolist() == g["buffer_row_offsets"] and co.tolist() == g["cache_offsets"]
    assert bl.tolist() == g["buffer_lengths"] and need == g["chunks_needed"]


def test_plan_bit_exact_random_and_edges(B):
    rng = np.random.default_rng(123)
    cases = []
    for _ in range(60):
        Bn = int(rng.integers(1, 40))
        cases.append((rng.integers(0, 50, Bn), rng.integers(0, 80, Bn), int(rng.integers(1, 20))))
    cases.append((np.zeros(5, np.int64), np.zeros(5, np.int64), 4))       # nothing at all
    cases.append((np.array([0, 7, 0]), np.array([3, 0, 0]), 1))             # T = 1
    cases.append((rng.integers(0, 9, 700), rng.integers(0, 9, 700), 3))     # > 256 sequences
    cases.append((rng.integers(0, 3000, 1000), rng.integers(0, 3000, 1000), 517))
    for new, cached, T in cases:
        offs = np.concatenate([[0], np.cumsum(new)])
        C = max(1, -(-int((new + cached).max()) // T)) + int(rng.integers(0, 3))
        g = _plan_gpu(B, offs, cached, T, C)
        r = oracle.plan(offs, cached, T, C)
        for a, b in zip(g[:3], r):
            assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# gather + RMSNorm + RoPE
# ---------------------------------------------------------------------------

def _gather_case(B, wl, fp8_rope=False):
    d = oracle.Decoded(wl)
    t = prefill_tensors(wl)
    bro, co, bl, _ = B.plan(t["input_row_offsets"], t["cache_lengths"], wl.buffer_token_size,
                            wl.max_chunks)
    rbro, rco, rbl = oracle.plan(wl.input_row_offsets, wl.cache_lengths, wl.buffer_token_size,
                                 wl.max_chunks)
    R = max(64, (int(wl.batch * wl.buffer_token_size) + 63) // 64 * 64)
    for c in range(wl.max_chunks):
        n = int(rbl[c])
        if n < 0:
            continue
        lat = torch.full((R, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        kr_dtype = torch.float8_e4m3fn if fp8_rope else torch.bfloat16
        kr = torch.zeros((R, 64), dtype=kr_dtype, device="cuda")
        B.mla_gather_norm_rope(lat, kr, t["kv_cache"], t["page_table"], bro[c].contiguous(),
                               co[c].contiguous(), bl[c:c + 1], t["kv_norm_gamma"],
                               t["freqs_cis"], wl.eps)
        torch.cuda.synchronize()
        glat = _f64(lat)[:n]
        gkr = oracle.e4m3fn_to_f64(fp8_bits(kr))[:n] if fp8_rope else _f64(kr)[:n]
        for b in range(wl.batch):
            r0, r1 = int(rbro[c, b]), int(rbro[c, b + 1])
            if r1 == r0:
                continue
            pos = int(rco[c, b]) + np.arange(r1 - r0)
            raw = oracle.gather_rows(d.pool, wl.page_table, b, pos, wl.page_size)
            xl, yr = oracle.norm_rope_rows(raw, pos, d.gamma, d.freqs, wl.eps, 512)
            err = np.abs(glat[r0:r1] - xl)
            assert (err <= 2.0 ** -8 * np.abs(xl) + 1e-5).all(), err.max()
            err = np.abs(gkr[r0:r1] - yr)
            tol = (2.0 ** -3 if fp8_rope else 2.0 ** -8) * np.abs(yr) + (2 ** -9 if fp8_rope else 1e-5)
            assert (err <= tol).all(), err.max()


def test_gather_norm_rope_tiny(B):
    _gather_case(B, prefill_recipe("tiny_b2"))


def test_gather_norm_rope_mid(B):
    wl = make_prefill("mid", 21, [300, 0, 77, 129], [0, 40, 250, 1000], 2, 16, 256)
    _gather_case(B, wl)


def test_gather_norm_rope_fp8_cache(B):
    wl = make_prefill("mid8", 22, [100, 33], [70, 0], 2, 16, 64, fp8=True)
    _gather_case(B, wl, fp8_rope=True)


# ---------------------------------------------------------------------------
# up-projection GEMM
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,R,n", [(2, 128, 128), (3, 256, 201), (1, 64, 1)])
def test_up_project(B, H, R, n):
    rng = np.random.default_rng(H * 1000 + n)
    lat_bits = f32_to_bf16_bits(rng.standard_normal((R, 512), dtype=np.float32))
    wk_bits = f32_to_bf16_bits(rng.standard_normal((H * 128, 512), dtype=np.float32) / 22.6)
    wuv_bits = f32_to_bf16_bits(rng.standard_normal((H, 128, 512), dtype=np.float32) / 22.6)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    kn = torch.full((H, R, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vt = torch.full((H, 128, R), float("nan"), dtype=torch.bfloat16, device="cuda")
    bl = torch.tensor([n], dtype=torch.int32, device="cuda")
    B.mla_up_project(kn, vt, dev(lat_bits), dev(wk_bits), dev(wuv_bits), bl)
    torch.cuda.synchronize()
    lat = oracle.bf16_to_f64(lat_bits)[:n]
    rk, rv = oracle.up_project(lat, oracle.bf16_to_f64(wk_bits), oracle.bf16_to_f64(wuv_bits), H)
    gk = _f64(kn)[:, :n].transpose(1, 0, 2)
    gv = _f64(vt)[:, :, :n].transpose(2, 0, 1)
    # bound: half an ulp of bf16 on the result plus fp32 accumulation of 512 terms
    scale_k = np.sqrt((lat ** 2) @ (oracle.bf16_to_f64(wk_bits) ** 2).T).reshape(n, H, 128)
    assert (np.abs(gk - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-5 * scale_k + 1e-6).all()
    assert (np.abs(gv - rv) <= 2.0 ** -8 * np.abs(rv) + 1e-5 * np.abs(rv).max() + 1e-5).all()
    # rows past the chunk up to the next 64-row tile are zeros: a key tile that
    # runs past the chunk reads finite values
    n64 = min(-(-n // 64) * 64, R)
    assert (_f64(kn)[:, n:n64] == 0).all() and (_f64(vt)[:, :, n:n64] == 0).all()


# ---------------------------------------------------------------------------
# attention on given K/V (one chunk)
# ---------------------------------------------------------------------------

def _attention_given_kv(B, seed, fp8=False, plant=()):
    """mla_prefill_attention on random K/V of one chunk (bf16, or e4m3 q,
    K_nope and k_rope) against the oracle. plant: (sequence, key, query, head)
    entries; that key's k_rope row becomes 20 * sign of that query's rope part
    for that head, which lifts its logit about 100 log2 units above the rest."""
    rng = np.random.default_rng(seed)
    H = 3
    new = np.array([5, 130, 64, 1, 200])
    cached = np.array([0, 70, 0, 300, 129])
    L = new + cached
    offs = np.concatenate([[0], np.cumsum(new)])
    T = int(L.max())
    bro, co, bl = oracle.plan(offs, cached, T, 1)
    R = (int(bl[0]) + 63) // 64 * 64 + 64
    tq = int(offs[-1])
    normal = lambda shape: rng.standard_normal(shape, dtype=np.float32)
    if fp8:
        enc, dec = f32_to_e4m3fn_codes, oracle.e4m3fn_to_f64
        dev_k = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).cuda()
    else:
        enc, dec = f32_to_bf16_bits, oracle.bf16_to_f64
        dev_k = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q_b = enc(normal((tq, H, 192)))
    kn_b = enc(normal((H, R, 128)))
    kr_b = enc(normal((R, 64)))
    vt_b = f32_to_bf16_bits(normal((H, 128, R)))
    for b, key, qi, h in plant:
        row = int(bro[0, b]) + key
        kr_b[row] = enc(20.0 * np.sign(dec(q_b[offs[b] + qi, h, 128:])).astype(np.float32))
    out = torch.full((tq, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.mla_prefill_attention_workspace_size(len(new), tq, H), dtype=torch.uint8,
                     device="cuda")
    scale = 1 / math.sqrt(192)
    B.mla_prefill_attention(out, dev_k(q_b), dev_k(kn_b), dev(vt_b), dev_k(kr_b), _u32(offs),
                            _u32(cached), _u32(bro[0]), _u32(co[0]),
                            torch.tensor(bl, dtype=torch.int32, device="cuda"),
                            int(new.max()), scale, ws)
    torch.cuda.synchronize()
    got = _f64(out)
    q, kn, kr = dec(q_b), dec(kn_b), dec(kr_b)
    vt = oracle.bf16_to_f64(vt_b)
    for b in range(len(new)):
        r0, r1 = int(bro[0, b]), int(bro[0, b + 1])
        ref = oracle.attend_sequence(q[offs[b]:offs[b + 1]], kn[:, r0:r1].transpose(1, 0, 2),
                                     kr[r0:r1], vt[:, :, r0:r1].transpose(2, 0, 1),
                                     cached[b] + np.arange(new[b]), np.arange(L[b]), scale, 128)
        err = np.abs(got[offs[b]:offs[b + 1]] - ref)
        if fp8:
            assert err.max() <= FP8_MAX, (b, err.max())
        else:
            assert err.max() <= BF16_MAX and (err.size == 0 or err.mean() <= BF16_MEAN), (b, err.max())
    return bro


def test_prefill_attention_given_kv(B):
    _attention_given_kv(B, 31)


@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_attention_planted_extreme_keys(B, fp8):
    """Keys whose logits jump ~100 log2 units above the running maximum of the
    queries that see them, in the first and in the second 32-key half of a
    64-key tile and never in a sequence's first tile, so the softmax reference
    must move and the accumulated output rescale by 2^-100 or so without
    overflow. Sequence 4 starts at buffer row 570: its key 120 is row 690 (row
    50 of the tile at 640), its key 200 row 770 (row 2 of the tile at 768);
    sequence 1 starts at row 5: its key 133 is row 138 (row 10 of the tile at
    128)."""
    bro = _attention_given_kv(B, 32, fp8,
                              plant=[(4, 120, 199, 0), (4, 200, 150, 2), (1, 133, 129, 1)])
    # the rows sit where the docstring says (the plan is bit-exact on its own test)
    assert int(bro[0, 4]) == 570 and int(bro[0, 1]) == 5


# ---------------------------------------------------------------------------
# end-to-end prefill
# ---------------------------------------------------------------------------

def _nan_out(*shape):
    """An output tensor filled with NaN, so that a row no workgroup writes
    fails the finiteness check."""
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")


def _run_prefill(B, wl, max_rows=None, max_chunks=-1):
    t = prefill_tensors(wl)
    out = B.prefill(t["q"], t["input_row_offsets"], t["cache_lengths"], t["kv_cache"],
                    t["page_table"], t["w_k"], t["w_uv"], t["kv_norm_gamma"], t["freqs_cis"],
                    wl.buffer_token_size, wl.max_chunks if max_chunks == -1 else max_chunks,
                    int(wl.new_lens.max()), wl.scale, wl.eps, max_rows=max_rows,
                    output=_nan_out(wl.total_q, wl.num_heads, 128))
    torch.cuda.synchronize()
    return _f64(out)


def _assert_close(got, ref, max_abs, mean_abs=None):
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    assert err.max() <= max_abs, f"max-abs {err.max():.3e}"
    if mean_abs is not None:
        assert err.mean() <= mean_abs, f"mean-abs {err.mean():.3e}"
    return err


def test_prefill_tiny_full(B):
    wl = prefill_recipe("tiny_b2")
    _say("prefill tiny_b2")
    _assert_close(_run_prefill(B, wl), oracle.prefill(wl), BF16_MAX, BF16_MEAN)


def test_prefill_multichunk_ragged_full(B):
    # several 64-key tiles, ragged 128-query blocks, sequences split over chunks,
    # an empty prompt and pages of 16
    wl = make_prefill("mid", 41, [300, 77, 0, 129, 1], [0, 250, 33, 1000, 5], 4, 16, 256)
    _say("prefill mid multichunk")
    _assert_close(_run_prefill(B, wl), oracle.prefill(wl), BF16_MAX, BF16_MEAN)


def test_prefill_single_head_chunk_of_one(B):
    wl = make_prefill("t1", 42, [9, 3], [4, 0], 1, 16, 1)
    _assert_close(_run_prefill(B, wl), oracle.prefill(wl), BF16_MAX, BF16_MEAN)


def _oracle_threads() -> int:
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _head_slice(wl, sel):
    """The workload restricted to the heads in sel (their q, w_k, w_uv, w_uk)."""
    d, H = wl.dims, wl.num_heads
    w = dataclasses.replace(wl)
    w.q = np.ascontiguousarray(wl.q[:, sel])
    w.w_k = np.ascontiguousarray(wl.w_k.reshape(H, d.nope, d.lora)[sel].reshape(-1, d.lora))
    w.w_uv = np.ascontiguousarray(wl.w_uv[sel])
    w.w_uk = np.ascontiguousarray(wl.w_uk[sel])
    w.num_heads = len(sel)
    return w


def _oracle_prefill_by_heads(wl, heads_per_slice=16):
    """oracle.prefill over every head, run in head slices (one sequence's
    materialised scores for all 128 heads would not fit in memory) on a
    thread pool; BLAS is held to one thread inside the pool."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    H = wl.num_heads
    slices = [list(range(h, min(h + heads_per_slice, H))) for h in range(0, H, heads_per_slice)]
    out = np.empty((wl.total_q, H, wl.dims.v))
    with threadpool_limits(1), cf.ThreadPoolExecutor(_oracle_threads()) as ex:
        for sel, r in zip(slices, ex.map(lambda sl: oracle.prefill(_head_slice(wl, sl)), slices)):
            out[:, sel[0]:sel[-1] + 1] = r
    return out


def _dense_samples(wl, rng):
    """(t, h) rows for every head of every sequence: the sequence's first and
    last query, one random query of each 128-query block, and the queries on
    both sides of every chunk boundary (the first query whose keys span one
    more chunk, and the one before it)."""
    T = wl.buffer_token_size
    offs = wl.input_row_offsets.astype(np.int64)
    out = []
    for b in range(wl.batch):
        n, c = int(offs[b + 1] - offs[b]), int(wl.cached_lens[b])
        if n == 0:
            continue
        qs = {0, n - 1}
        for blk in range(0, n, 128):
            qs.add(int(rng.integers(blk, min(blk + 128, n))))
        k = (c // T + 1) * T  # first chunk boundary past the cached prefix
        while k < c + n:
            qs.update(i for i in (k - c - 1, k - c) if 0 <= i < n)
            k += T
        out += [(int(offs[b]) + i, h) for i in sorted(qs) for h in range(wl.num_heads)]
    return out


def _oracle_prefill_sampled(wl, samples):
    """oracle.prefill_sampled, one sequence per task of a thread pool."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    dec = oracle.Decoded(wl)
    seq_of = np.searchsorted(wl.input_row_offsets[1:].astype(np.int64),
                             [t for t, _ in samples], side="right")
    groups: dict = {}
    for i, b in enumerate(seq_of):
        groups.setdefault(int(b), []).append(i)
    res = np.empty((len(samples), wl.dims.v))

    def run(b):
        idx = groups[b]
        return idx, oracle.prefill_sampled(wl, [samples[i] for i in idx], dec)

    with threadpool_limits(1), cf.ThreadPoolExecutor(_oracle_threads()) as ex:
        for idx, r in ex.map(run, sorted(groups)):
            res[idx] = r
    return res


@pytest.mark.timeout(900)
def test_prefill_dsv3_4k_full(B):
    """Every output element of the 4096-token, 128-head prefill against the
    oracle (run in 16-head slices): max-abs and mean-abs over all of them."""
    wl = prefill_recipe("dsv3_prefill_4k")
    _say("prefill dsv3_prefill_4k: running")
    got = _run_prefill(B, wl)
    _say("prefill dsv3_prefill_4k: oracle over all 128 heads")
    ref = _oracle_prefill_by_heads(wl)
    err = _assert_close(got, ref, BF16_MAX, BF16_MEAN)
    _say(f"prefill dsv3_prefill_4k: {got.size} elements, max-abs {err.max():.3e}, "
         f"mean-abs {err.mean():.3e}")


def _dense_sampled_check(B, name, max_abs, mean_abs):
    _say(f"prefill {name}: generating")
    wl = prefill_recipe(name)
    _say(f"prefill {name}: running")
    got = _run_prefill(B, wl)
    assert np.isfinite(got).all()  # every row written (outputs start as NaN)
    pairs = _dense_samples(wl, np.random.default_rng(7))
    _say(f"prefill {name}: oracle on {len(pairs)} sampled rows (every head of every sequence)")
    ref = _oracle_prefill_sampled(wl, pairs)
    g = np.stack([got[t, h] for t, h in pairs])
    err = _assert_close(g, ref, max_abs, mean_abs)
    _say(f"prefill {name}: max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")


@pytest.mark.timeout(900)
def test_prefill_ragged_b16_dense_sampled(B):
    _dense_sampled_check(B, "ragged_b16_cached", BF16_MAX, BF16_MEAN)


@pytest.mark.timeout(900)
def test_prefill_fp8_dense_sampled(B):
    _dense_sampled_check(B, "fp8_ragged_b8_cached", FP8_MAX, None)


def test_prefill_max_chunks_derived_or_rejected(B):
    """The convenience path reads the planner's chunk count: max_chunks None
    plans every chunk the batch needs (tiny_b2 needs 3 chunks of 8 tokens),
    and a max_chunks below that raises instead of leaving queries unwritten."""
    wl = prefill_recipe("tiny_b2")
    _assert_close(_run_prefill(B, wl, max_chunks=None), oracle.prefill(wl), BF16_MAX, BF16_MEAN)
    with pytest.raises(ValueError, match="max_chunks"):
        _run_prefill(B, wl, max_chunks=2)
    t = prefill_tensors(wl)
    with pytest.raises(ValueError, match="max_chunks"):
        B.prefill_decode(t["q"], t["input_row_offsets"], t["cache_lengths"], t["kv_cache"],
                         t["page_table"], t["w_uk"], t["w_uv"], t["kv_norm_gamma"],
                         t["freqs_cis"], int(wl.new_lens.max()), int(wl.cached_lens.max()),
                         wl.scale, wl.eps, w_k=t["w_k"], buffer_token_size=wl.buffer_token_size,
                         max_chunks=1)


def test_prefill_fp8_small_full(B):
    wl = make_prefill("m8", 43, [70, 5, 140], [0, 60, 9], 2, 16, 128, fp8=True)
    _assert_close(_run_prefill(B, wl), oracle.prefill(wl), FP8_MAX)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _run_decode(B, wl, num_partitions=0):
    t = decode_tensors(wl)
    out = B.decode(t["q"], t["context_lengths"], t["kv_cache"], t["page_table"], t["w_uk"],
                   t["w_uv"], int(wl.context_lens.max()), wl.scale,
                   num_partitions=num_partitions,
                   output=_nan_out(wl.batch, wl.num_heads, 128))
    torch.cuda.synchronize()
    return _f64(out)


@pytest.mark.parametrize("parts", [0, 1, 3, 7])
def test_decode_small_full(B, parts):
    wl = make_decode("d", 51, [1, 37, 300, 64, 1000], 8, 16)
    _assert_close(_run_decode(B, wl, parts), oracle.decode(wl), BF16_MAX, BF16_MEAN)


def test_decode_all_heads_full(B):
    wl = make_decode("d128", 52, [5000, 129, 2], 128, 64)
    _assert_close(_run_decode(B, wl), oracle.decode(wl), BF16_MAX, BF16_MEAN)


def _oracle_decode_threaded(wl):
    """oracle.decode over every sequence, one sequence per task of a thread pool."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    dec = oracle.DecodedDecode(wl)
    with threadpool_limits(1), cf.ThreadPoolExecutor(_oracle_threads()) as ex:
        rows = list(ex.map(lambda b: oracle.decode(wl, dec, batch_indices=[b])[0],
                           range(wl.batch)))
    return np.stack(rows)


@pytest.mark.timeout(900)
def test_decode_b64_full(B):
    """All 64 sequences (every key range of the split) against the oracle."""
    _say("decode_b64: generating")
    wl = decode_recipe("decode_b64")
    _say("decode_b64: running")
    got = _run_decode(B, wl)
    _say("decode_b64: oracle on all 64 sequences")
    err = _assert_close(got, _oracle_decode_threaded(wl), BF16_MAX, BF16_MEAN)
    _say(f"decode_b64: max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("parts", [0, 1])
def test_decode_extreme_score_range_recomputed(B, parts, fp8):
    """One late cache row whose rope part is 16 * sign(q_rope) of head 0 (latent
    part zero): its logit for head 0 exceeds the other rows' by ~80 log2 units,
    more than the split kernel's 64-unit range, so with one key range (parts =
    1; the row sits in the 19th tile of its segment) that partial is handed to
    the combine step's recomputation; without it exp2 would overflow fp32. The
    rope half of q enters the scores unrounded, so bf16 bounds apply as usual
    (16 and 0 are exact in e4m3 too)."""
    wl = make_decode("ext", 61, [700, 300], 8, 16, fp8=fp8)
    dec = oracle.DecodedDecode(wl)
    row = np.zeros(576, dtype=np.float32)
    row[512:] = 16.0 * np.sign(dec.q[0, 0, 128:])
    p = 600  # position in sequence 0, well after its first tiles
    slot = int(wl.page_table[0, p // wl.page_size]) * wl.page_size + p % wl.page_size
    wl.pool.reshape(-1, 576)[slot] = f32_to_e4m3fn_codes(row) if fp8 else f32_to_bf16_bits(row)
    got = _run_decode(B, wl, parts)
    ref = oracle.decode(wl)
    if fp8:
        _assert_close(got, ref, FP8_MAX)
    else:
        _assert_close(got, ref, BF16_MAX, BF16_MEAN)


# decode over an e4m3fn cache: rows are widened exactly to bf16 and both
# products run on bf16 MFMA, so only the bf16 roundings of the scores'
# probabilities and of q_lat separate the result from the oracle


@pytest.mark.parametrize("parts", [0, 3])
def test_decode_fp8_small_full(B, parts):
    wl = make_decode("d8", 53, [1, 37, 300, 64, 1000], 8, 16, fp8=True)
    _assert_close(_run_decode(B, wl, parts), oracle.decode(wl), FP8_MAX)


def test_decode_fp8_all_heads_full(B):
    wl = make_decode("d8_128", 54, [5000, 129, 2], 128, 64, fp8=True)
    _assert_close(_run_decode(B, wl), oracle.decode(wl), FP8_MAX)


def test_decode_fp8_single_key_widening_exact(B):
    """Contexts of one key: the softmax weight is exactly 1, so o_lat is the
    stored latent row itself and the output is w_uv times that row, summed in
    fp32 and rounded once to bf16. The rows are set to chosen e4m3fn codes:
    sequences 0..31 hold only subnormal codes (exponent field 0), the others
    every finite code at random, up to +-448. Each output element must be
    within one bf16 rounding (2^-8 relative) plus the fp32 summation bound
    (2^-20 of the sum of |w z|) of the exact value, so a code widened wrongly
    (a subnormal flushed, a wrong exponent bias) fails."""
    wl = make_decode("d8_one", 55, [1] * 64, 8, 16, fp8=True)
    rng = np.random.default_rng(56)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    subn = np.array([c for c in range(256) if (c & 0x78) == 0], dtype=np.uint8)
    rows = wl.pool.reshape(-1, 576)
    for b in range(64):
        slot = int(wl.page_table[b, 0]) * wl.page_size
        rows[slot] = rng.choice(subn if b < 32 else finite, 576)
    got = _run_decode(B, wl)
    ref = oracle.decode(wl)
    dec = oracle.DecodedDecode(wl)
    for b in range(64):
        z = np.abs(dec.pool.reshape(-1, 576)[int(wl.page_table[b, 0]) * wl.page_size, :512])
        sum_abs = np.abs(dec.w_uv) @ z  # [H, 128]
        bound = 2.0 ** -8 * np.abs(ref[b]) + 2.0 ** -20 * sum_abs + 1e-30
        assert np.all(np.abs(got[b] - ref[b]) <= bound), f"sequence {b}"


@pytest.mark.timeout(900)
def test_decode_b64_fp8_full(B):
    _say("decode_b64_fp8: generating")
    wl = decode_recipe("decode_b64_fp8")
    _say("decode_b64_fp8: running")
    got = _run_decode(B, wl)
    _say("decode_b64_fp8: oracle on all 64 sequences")
    err = _assert_close(got, _oracle_decode_threaded(wl), FP8_MAX)
    _say(f"decode_b64_fp8: max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")


# ---------------------------------------------------------------------------
# KV write path: new tokens normalised, rotated and stored in their slots
# ---------------------------------------------------------------------------

def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _dev_pool(pool, fp8):
    if fp8:
        return torch.from_numpy(np.ascontiguousarray(pool)).view(torch.float8_e4m3fn).cuda()
    return _dev_bf16(pool)


def _kv_raw(rng, n):
    x = f32_to_bf16_bits((1.5 * rng.standard_normal((n, 576))).astype(np.float32))
    gamma = f32_to_bf16_bits((1.0 + 0.3 * rng.standard_normal(512)).astype(np.float32))
    return x, gamma


def _stored_bound(r, fp8):
    # one rounding of the fp32 result to the cache dtype (unit roundoff 2^-8
    # for bf16, 2^-4 for e4m3 normals, half the 2^-9 subnormal step) plus the
    # fp32 arithmetic of the norm and the rotation
    if fp8:
        return 2.0 ** -4 * np.abs(r) + 2.0 ** -10 + 1e-5
    return (2.0 ** -8 + 2e-6) * np.abs(r) + 1e-5


@pytest.mark.parametrize("fp8", [False, True])
def test_kv_write_small(B, fp8):
    rng = np.random.default_rng(61)
    ps = 16
    cached, new = [5, 0, 40, 7], [17, 1, 33, 0]
    L = np.asarray(cached) + np.asarray(new)
    maxp = int(((L + ps - 1) // ps).max()) + 1
    num_pages = len(cached) * maxp + 3
    pt = rng.permutation(num_pages)[:len(cached) * maxp].reshape(len(cached), maxp).astype(np.int32)
    pt[2, 3] = -1                              # a missing page: its tokens are skipped
    vals = rng.standard_normal((num_pages, ps, 576)).astype(np.float32)
    pool = f32_to_e4m3fn_codes(vals) if fp8 else f32_to_bf16_bits(vals)
    off = np.concatenate([[0], np.cumsum(new)]).astype(np.uint32)
    x, gamma = _kv_raw(rng, int(off[-1]))
    max_seq_len = int(L.max()) - 3             # the last three positions have no rotation row
    freqs = rope_table_bits(max_seq_len, 64)
    cache = _dev_pool(pool, fp8)
    B.mla_kv_write(cache, torch.from_numpy(pt).cuda(), _dev_bf16(x), _u32(off), _u32(cached),
                   _dev_bf16(gamma), _dev_bf16(freqs), 1e-6)
    torch.cuda.synchronize()
    got_bits = fp8_bits(cache) if fp8 else bf16_bits(cache)
    dec = oracle.e4m3fn_to_f64 if fp8 else oracle.bf16_to_f64
    ref = oracle.kv_write(dec(pool), pt, oracle.bf16_to_f64(x), off, cached,
                          oracle.bf16_to_f64(gamma), oracle.bf16_to_f64(freqs), 1e-6, ps)
    written = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(len(cached)):
        for i in range(new[b]):
            p = cached[b] + i
            if pt[b, p // ps] >= 0 and p < max_seq_len:
                written[pt[b, p // ps], p % ps] = True
    assert 0 < written.sum() < sum(new)       # the hole and the short table removed some
    assert np.array_equal(got_bits[~written], pool[~written])     # nothing else touched
    g, r = dec(got_bits)[written], ref[written]
    assert (np.abs(g - r) <= _stored_bound(r, fp8)).all()


@pytest.mark.parametrize("fp8", [False, True])
def test_kv_write_then_decode(B, fp8):
    # decode reads rows as stored: write each sequence's new token from its raw
    # row, then decode; the oracle decodes the pool the write defines
    wl = make_decode("kvw", 71, [300, 1, 1000, 77], 16, 16, fp8=fp8)
    ctx = wl.context_lens.astype(np.int64)
    rng = np.random.default_rng(72)
    x, gamma = _kv_raw(rng, len(ctx))
    freqs = rope_table_bits(int(ctx.max()), 64)
    off = np.arange(len(ctx) + 1, dtype=np.uint32)
    t = decode_tensors(wl)
    B.mla_kv_write(t["kv_cache"], t["page_table"], _dev_bf16(x), _u32(off), _u32(ctx - 1),
                   _dev_bf16(gamma), _dev_bf16(freqs), 1e-6)
    out = B.decode(t["q"], t["context_lengths"], t["kv_cache"], t["page_table"], t["w_uk"],
                   t["w_uv"], int(ctx.max()), wl.scale)
    torch.cuda.synchronize()
    dec = oracle.e4m3fn_to_f64 if fp8 else oracle.bf16_to_f64
    vals = oracle.kv_write(dec(wl.pool), wl.page_table, oracle.bf16_to_f64(x), off, ctx - 1,
                           oracle.bf16_to_f64(gamma), oracle.bf16_to_f64(freqs), 1e-6,
                           wl.page_size).astype(np.float32)
    stored = f32_to_e4m3fn_codes(vals) if fp8 else f32_to_bf16_bits(vals)
    ref = oracle.decode(dataclasses.replace(wl, pool=stored))
    if fp8:
        _assert_close(_f64(out), ref, FP8_MAX)
    else:
        _assert_close(_f64(out), ref, BF16_MAX, BF16_MEAN)


# ---------------------------------------------------------------------------
# sparse decode: attention over explicit lists of pool rows
# ---------------------------------------------------------------------------

def _sparse_case(wl, lens, seed):
    rng = np.random.default_rng(seed)
    rows = wl.pool.shape[0] * wl.pool.shape[1]
    stride = max(lens) + 3
    idx = rng.integers(0, rows, size=(len(lens), stride)).astype(np.int32)
    idx[0, :] = idx[0, 0]                      # the same row listed over and over
    return idx


def _run_sparse(B, wl, idx, lens):
    t = decode_tensors(wl)
    out = B.decode_sparse(t["q"], torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                          t["kv_cache"], torch.from_numpy(idx).cuda(), t["w_uk"], t["w_uv"],
                          idx.shape[1], wl.scale)
    torch.cuda.synchronize()
    return _f64(out)


def _sparse_ref(wl, idx, lens):
    dec = oracle.DecodedDecode(wl)
    return oracle.decode_sparse(dec.q, dec.pool, idx, lens, dec.w_uk, dec.w_uv, wl.scale,
                                dec.nope, dec.lora)


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_sparse_small(B, fp8):
    wl = make_decode("sp", 81, [2000, 900, 3000, 40, 1500], 16, 16, fp8=fp8)
    lens = [5, 37, 300, 0, 700]
    idx = _sparse_case(wl, lens, 82)
    got = _run_sparse(B, wl, idx, lens)
    ref = _sparse_ref(wl, idx, lens)
    assert np.array_equal(got[3], np.zeros_like(got[3]))      # an empty list gives zeros
    if fp8:
        _assert_close(got, ref, FP8_MAX)
    else:
        _assert_close(got, ref, BF16_MAX, BF16_MEAN)


def test_decode_sparse_over_the_context_in_order_equals_decode(B):
    wl = make_decode("spd", 83, [1, 37, 300, 64, 1000], 128, 16)
    ps = wl.page_size
    ctx = [int(c) for c in wl.context_lens]
    idx = np.zeros((len(ctx), max(ctx)), dtype=np.int32)
    for b, n in enumerate(ctx):
        p = np.arange(n)
        idx[b, :n] = wl.page_table[b, p // ps] * ps + p % ps
    _assert_close(_run_sparse(B, wl, idx, ctx), oracle.decode(wl), BF16_MAX, BF16_MEAN)


# ---------------------------------------------------------------------------
# attention sinks: one more logit per sequence in the softmax denominator
# ---------------------------------------------------------------------------

def _sinks(vals):
    return torch.tensor(vals, dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_sinks_multichunk(B, fp8):
    # sequences split over several chunks: the sink enters once, at the end
    # (e4m3: the cache, q and the score path in e4m3, as the fp8 prefill runs)
    wl = make_prefill("sink", 44, [70, 5, 140], [0, 60, 9], 2, 16, 64, fp8=fp8)
    sinks = [2.5, -np.inf, 0.3]
    t = prefill_tensors(wl)
    out = B.prefill(t["q"], t["input_row_offsets"], t["cache_lengths"], t["kv_cache"],
                    t["page_table"], t["w_k"], t["w_uv"], t["kv_norm_gamma"], t["freqs_cis"],
                    wl.buffer_token_size, wl.max_chunks, int(wl.new_lens.max()), wl.scale,
                    wl.eps, attn_sink=_sinks(sinks))
    torch.cuda.synchronize()
    ref = oracle.prefill(wl, sinks=np.array(sinks))
    if fp8:
        _assert_close(_f64(out), ref, FP8_MAX)
    else:
        _assert_close(_f64(out), ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("parts", [0, 3])
def test_decode_sinks(B, parts):
    wl = make_decode("dsk", 53, [1, 37, 300, 64, 1000], 8, 16)
    sinks = [1.0, 4.0, -np.inf, -3.0, 0.0]
    t = decode_tensors(wl)
    out = B.decode(t["q"], t["context_lengths"], t["kv_cache"], t["page_table"], t["w_uk"],
                   t["w_uv"], int(wl.context_lens.max()), wl.scale, num_partitions=parts,
                   attn_sink=_sinks(sinks))
    torch.cuda.synchronize()
    _assert_close(_f64(out), oracle.decode(wl, sinks=np.array(sinks)), BF16_MAX, BF16_MEAN)


def test_decode_sparse_sinks(B):
    wl = make_decode("spk", 84, [2000, 900, 3000], 16, 16)
    lens = [5, 300, 0]
    idx = _sparse_case(wl, lens, 85)
    sinks = [2.0, -1.0, 5.0]
    t = decode_tensors(wl)
    out = B.decode_sparse(t["q"], torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                          t["kv_cache"], torch.from_numpy(idx).cuda(), t["w_uk"], t["w_uv"],
                          idx.shape[1], wl.scale, attn_sink=_sinks(sinks))
    torch.cuda.synchronize()
    dec = oracle.DecodedDecode(wl)
    ref = oracle.decode_sparse(dec.q, dec.pool, idx, lens, dec.w_uk, dec.w_uv, wl.scale,
                               dec.nope, dec.lora, sinks=np.array(sinks))
    _assert_close(_f64(out), ref, BF16_MAX, BF16_MEAN)


# ---------------------------------------------------------------------------
# the graph op as one call: KV write, then prefill or decode by max_seq_len
# ---------------------------------------------------------------------------

def _round_to_storage(vals, fp8):
    v = np.asarray(vals, dtype=np.float32)
    return f32_to_e4m3fn_codes(v) if fp8 else f32_to_bf16_bits(v)


def _decoded(bits, fp8):
    return oracle.e4m3fn_to_f64(bits) if fp8 else oracle.bf16_to_f64(bits)


@pytest.mark.parametrize("fp8", [False, True])
def test_unified_prefill_writes_then_attends_over_stored_rows(B, fp8):
    # several chunks of 256 tokens, ragged prompts, an empty one, pages of 16;
    # the pool's cached rows are taken as stored rows, the new tokens come in raw
    wl = make_prefill("uni", 91, [300, 77, 0, 129, 1], [0, 250, 33, 1000, 5], 4, 16, 256)
    pool = _round_to_storage(oracle.bf16_to_f64(wl.pool), fp8)
    rng = np.random.default_rng(92)
    x, gamma = _kv_raw(rng, wl.total_q)
    t = prefill_tensors(wl)
    cache = _dev_pool(pool, fp8)
    _say(f"unified prefill fp8_cache={fp8}")
    out = B.prefill_decode(t["q"], t["input_row_offsets"], t["cache_lengths"], cache,
                           t["page_table"], t["w_uk"], t["w_uv"], _dev_bf16(gamma),
                           t["freqs_cis"], int(wl.new_lens.max()), int(wl.cached_lens.max()),
                           wl.scale, wl.eps, kv_input=_dev_bf16(x), w_k=t["w_k"],
                           buffer_token_size=wl.buffer_token_size, max_chunks=wl.max_chunks)
    torch.cuda.synchronize()
    dec = oracle.Decoded(wl)
    written = oracle.kv_write(_decoded(pool, fp8), wl.page_table, oracle.bf16_to_f64(x),
                              wl.input_row_offsets, wl.cache_lengths, oracle.bf16_to_f64(gamma),
                              dec.freqs, wl.eps, wl.page_size)
    stored = _decoded(_round_to_storage(written, fp8), fp8)
    ref, _ = oracle.prefill_decode(dec.q, dec.offs, dec.clen, stored, wl.page_table,
                                   wl.page_size, dec.w_k, dec.w_uk, dec.w_uv, dec.gamma,
                                   dec.freqs, wl.scale, wl.eps, int(wl.new_lens.max()))
    _assert_close(_f64(out), ref, BF16_MAX, BF16_MEAN)
    got_pool = _decoded(fp8_bits(cache) if fp8 else bf16_bits(cache), fp8)
    assert (np.abs(got_pool - written) <= _stored_bound(written, fp8)).all()


@pytest.mark.parametrize("fp8,parts", [(False, 0), (False, 5), (True, 0)])
def test_unified_decode_writes_the_token_then_attends(B, fp8, parts):
    wl = make_decode("udec", 93, [300, 1, 1000, 77, 2500], 16, 16, fp8=fp8)
    ctx = wl.context_lens.astype(np.int64)
    rng = np.random.default_rng(94)
    x, gamma = _kv_raw(rng, len(ctx))
    freqs = rope_table_bits(int(ctx.max()), 64)
    off = np.arange(len(ctx) + 1, dtype=np.uint32)
    t = decode_tensors(wl)
    _say(f"unified decode fp8_cache={fp8} parts={parts}")
    out = B.prefill_decode(t["q"], _u32(off), _u32(ctx - 1), t["kv_cache"], t["page_table"],
                           t["w_uk"], t["w_uv"], _dev_bf16(gamma), _dev_bf16(freqs), 1,
                           int(ctx.max()) - 1, wl.scale, 1e-6, kv_input=_dev_bf16(x),
                           num_partitions=parts)
    # the dense decode entry over the same written pool runs the same kernels
    same = B.decode(t["q"], t["context_lengths"], t["kv_cache"], t["page_table"], t["w_uk"],
                    t["w_uv"], int(ctx.max()), wl.scale, num_partitions=parts)
    torch.cuda.synchronize()
    assert torch.equal(out, same)
    vals = oracle.kv_write(_decoded(wl.pool, fp8), wl.page_table, oracle.bf16_to_f64(x), off,
                           ctx - 1, oracle.bf16_to_f64(gamma), oracle.bf16_to_f64(freqs), 1e-6,
                           wl.page_size)
    ref = oracle.decode(dataclasses.replace(wl, pool=_round_to_storage(vals, fp8)))
    _assert_close(_f64(out), ref, FP8_MAX if fp8 else BF16_MAX, None if fp8 else BF16_MEAN)


def test_unified_sparse_decode_with_sinks(B):
    wl = make_decode("usp", 95, [2000, 900, 3000], 16, 16)
    lens = [5, 300, 0]
    idx = _sparse_case(wl, lens, 96)
    sinks = [1.0, -2.0, 3.0]
    ctx = wl.context_lens.astype(np.int64)
    t = decode_tensors(wl)
    gamma = _dev_bf16(f32_to_bf16_bits(np.ones(512, np.float32)))
    freqs = _dev_bf16(rope_table_bits(int(ctx.max()), 64))
    out = B.prefill_decode(t["q"], _u32(np.arange(len(ctx) + 1)), _u32(ctx - 1), t["kv_cache"],
                           t["page_table"], t["w_uk"], t["w_uv"], gamma, freqs, 1,
                           int(ctx.max()) - 1, wl.scale, 1e-6,
                           d_indices=torch.from_numpy(idx).cuda(),
                           topk_lengths=torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                           attn_sink=_sinks(sinks))
    torch.cuda.synchronize()
    dec = oracle.DecodedDecode(wl)
    ref = oracle.decode_sparse(dec.q, dec.pool, idx, lens, dec.w_uk, dec.w_uv, wl.scale,
                               dec.nope, dec.lora, sinks=np.array(sinks))
    _assert_close(_f64(out), ref, BF16_MAX, BF16_MEAN)


def test_unified_calls_replay_from_a_captured_graph(B):
    # every grid and the partition count are host values: a captured call
    # replays with new device data (queries, cache lengths) and matches the
    # eager call on the same data bit for bit
    wl = make_decode("ugr", 97, [700, 1, 2000, 64], 8, 16)
    ctx = wl.context_lens.astype(np.int64)
    t = decode_tensors(wl)
    Bn, H = wl.batch, wl.num_heads
    off = _u32(np.arange(Bn + 1))
    clen = _u32(ctx - 1)
    gamma = _dev_bf16(f32_to_bf16_bits(np.ones(512, np.float32)))
    freqs = _dev_bf16(rope_table_bits(int(ctx.max()), 64))
    max_cache = int(ctx.max()) - 1
    parts = 7
    nbytes = B.mla_prefill_decode_workspace_size(Bn, Bn, H, 1, 0, max_cache, wl.page_size, 0,
                                                 parts, B.MLA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((Bn, H, 128), dtype=torch.bfloat16, device="cuda")
    ref_out = torch.empty_like(out)

    def call(o, w):
        B.mla_prefill_decode(o, t["q"], off, clen, t["kv_cache"], t["page_table"], t["w_uk"],
                             t["w_uv"], gamma, freqs, 1, max_cache, wl.scale, 1e-6, w,
                             num_partitions=parts)

    call(out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, ws)
    rng = np.random.default_rng(98)
    for rep in range(3):
        qn = f32_to_bf16_bits(rng.standard_normal(wl.q.shape).astype(np.float32))
        t["q"].copy_(_dev_bf16(qn))
        new_ctx = np.maximum(1, ctx - rng.integers(0, 50, size=Bn))
        clen.copy_(_u32(new_ctx - 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        call(ref_out, ws2)
        torch.cuda.synchronize()
        _say(f"graph replay {rep}")
        assert torch.equal(got, ref_out)
        if rep == 0:
            ref = oracle.decode(dataclasses.replace(wl, q=qn,
                                                    context_lens=new_ctx.astype(np.uint32)))
            _assert_close(_f64(got), ref, BF16_MAX, BF16_MEAN)


def test_unified_prefill_with_its_plan_replays_from_a_captured_graph(B):
    wl = make_prefill("ugp", 99, [130, 0, 64], [40, 7, 200], 2, 16, 128)
    t = prefill_tensors(wl)
    Bn, H, Tq = wl.batch, wl.num_heads, wl.total_q
    C, T = wl.max_chunks, wl.buffer_token_size
    bro = torch.empty((C, Bn + 1), dtype=torch.uint32, device="cuda")
    co = torch.empty((C, Bn), dtype=torch.uint32, device="cuda")
    bl = torch.empty((C,), dtype=torch.int32, device="cuda")
    max_rows = Bn * T
    nbytes = B.mla_prefill_decode_workspace_size(Bn, Tq, H, int(wl.new_lens.max()), max_rows,
                                                 int(wl.cached_lens.max()), wl.page_size, 0, 0,
                                                 B.MLA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((Tq, H, 128), dtype=torch.bfloat16, device="cuda")

    def call(o):
        B.mla_prefill_plan(bro, co, bl, t["input_row_offsets"], t["cache_lengths"], T)
        B.mla_prefill_decode(o, t["q"], t["input_row_offsets"], t["cache_lengths"],
                             t["kv_cache"], t["page_table"], t["w_uk"], t["w_uv"],
                             t["kv_norm_gamma"], t["freqs_cis"], int(wl.new_lens.max()),
                             int(wl.cached_lens.max()), wl.scale, wl.eps, ws, w_k=t["w_k"],
                             plan_tensors=(bro, co, bl), max_rows=max_rows)

    call(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    rng = np.random.default_rng(100)
    ref_out = torch.empty_like(out)
    for rep in range(3):
        qn = f32_to_bf16_bits(rng.standard_normal(wl.q.shape).astype(np.float32))
        t["q"].copy_(_dev_bf16(qn))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        call(ref_out)
        torch.cuda.synchronize()
        _say(f"prefill graph replay {rep}")
        assert torch.equal(got, ref_out)
        if rep == 0:
            dec = oracle.Decoded(dataclasses.replace(wl, q=qn))
            ref, _ = oracle.prefill_decode(dec.q, dec.offs, dec.clen, dec.pool, wl.page_table,
                                           wl.page_size, dec.w_k, dec.w_uk, dec.w_uv,
                                           dec.gamma, dec.freqs, wl.scale, wl.eps,
                                           int(wl.new_lens.max()))
            _assert_close(_f64(got), ref, BF16_MAX, BF16_MEAN)


def test_decode_many_sequences_ragged_batch(B):
    # 130 sequences: three 64-sequence blocks of the absorb grid (the last one
    # ragged), prefix sums over more than one 256-entry scan block of ranges
    # when the partition count is raised, contexts from 1 to 300 keys
    rng = np.random.default_rng(121)
    ctx = rng.integers(1, 301, size=130)
    ctx[[0, 64, 129]] = [1, 300, 2]
    wl = make_decode("many", 122, list(ctx), 4, 16)
    _say("decode 130 sequences")
    for parts in (0, 300):
        _assert_close(_run_decode(B, wl, parts), oracle.decode(wl), BF16_MAX, BF16_MEAN)


def test_unified_decode_at_full_size_matches_the_decode_entry(B):
    # decode_b64 as the benchmark runs it through the graph op: each new
    # token's raw row written, then the decode over cache_len + 1 rows; the
    # dense decode entry over the written pool must agree bit for bit (its
    # parity at this size is checked above), and sampled written rows must
    # equal the oracle's normalised and rotated rows within one rounding
    wl = decode_recipe("decode_b64")
    ctx = wl.context_lens.astype(np.int64)
    rng = np.random.default_rng(131)
    x, gamma = _kv_raw(rng, len(ctx))
    freqs = rope_table_bits(int(ctx.max()), 64)
    t = decode_tensors(wl)
    _say("unified decode, decode_b64")
    out = B.prefill_decode(t["q"], _u32(np.arange(len(ctx) + 1)), _u32(ctx - 1), t["kv_cache"],
                           t["page_table"], t["w_uk"], t["w_uv"], _dev_bf16(gamma),
                           _dev_bf16(freqs), 1, int(ctx.max()) - 1, wl.scale, 1e-6,
                           kv_input=_dev_bf16(x))
    same = B.decode(t["q"], t["context_lengths"], t["kv_cache"], t["page_table"], t["w_uk"],
                    t["w_uv"], int(ctx.max()), wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, same)
    pool = t["kv_cache"]
    for b in (0, 17, 63):
        p = int(ctx[b]) - 1
        slot = int(wl.page_table[b, p // wl.page_size]) * wl.page_size + p % wl.page_size
        got = oracle.bf16_to_f64(bf16_bits(pool.reshape(-1, 576)[slot]))
        latn, kr = oracle.norm_rope_rows(oracle.bf16_to_f64(x[b:b + 1]), [p],
                                         oracle.bf16_to_f64(gamma), oracle.bf16_to_f64(freqs),
                                         1e-6, 512)
        ref = np.concatenate([latn[0], kr[0]])
        assert (np.abs(got - ref) <= _stored_bound(ref, False)).all()


def test_hbm_read_probe_folds_every_word(B):
    """The measurement helper reads every 16-byte word once: each workgroup's
    XOR equals the XOR of the words the grid-stride loop assigns to it."""
    rng = np.random.default_rng(141)
    for n16, groups in ((1000, 3), (256 * 40 + 7, 8), (1 << 16, 64)):
        words = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
        src = torch.from_numpy(words.view(np.int32)).cuda()
        out = torch.zeros(groups, dtype=torch.uint32, device="cuda")
        B.mla_hbm_read(src, out, groups)
        torch.cuda.synchronize()
        owner = (np.arange(n16) % (groups * 256)) // 256
        per_word = np.bitwise_xor.reduce(words, axis=1)
        want = [int(np.bitwise_xor.reduce(per_word[owner == w])) if (owner == w).any() else 0
                for w in range(groups)]
        assert out.cpu().numpy().astype(np.int64).tolist() == want
