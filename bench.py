"""Benchmark: MLA chunked prefill (and absorbed decode) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S]
                [--phases prefill,ragged,decode,sparse,kvwrite,unified,hbm,cpu]
                [--no-decode] [--no-cpu]

A step is one pass of the prefill path over the DeepSeek-V3-shaped batch (one
4096-token prompt, no cache, 128 heads): mla_prefill_plan, then for every chunk
slot mla_gather_norm_rope, mla_up_project and mla_prefill_attention, all
through the C ABI on torch's current stream. Inputs are resident in HBM before
the timed region. HIP events recorded on that stream around every call give
per-call durations; the attention call is the dominant kernel. "value" is the
end-to-end prefill rate in algorithmic attention TFLOP/s (attention FLOPs /
whole step time); "roofline" is the attention call alone against the bf16
dense MFMA peak, with HBM traffic and MFMA-busy figures from committed counter
summaries taken on the same kernel source (else null).

Further phases, each reported under its own key:
- ragged: the two ragged batches with cached prefixes and three chunks
  (ragged_b16_cached in bf16, fp8_ragged_b8_cached with q and the pool in
  e4m3): per chunk gather (timed after a cache flush), up-projection and
  attention in pipeline order, and the whole mla_prefill call; attention
  against the bf16 peak, or the fp8 peak and the mixed fp8/bf16 roofline.
- decode: mla_decode on the 64-sequence absorbed-decode batch (contexts
  U{4096..32768}) with a bf16 and an e4m3 cache, in HBM GB/s.
- sparse: mla_decode_sparse with every sequence listing 2048 rows.
- kvwrite: mla_kv_write of the prompt's 4096 new tokens.
- unified: mla_prefill_decode in its prefill and decode branches.
- hbm: the practical HBM rates of torch's own read and copy kernels.
- cpu: the fp64 oracle timed on bounded samples of every workload (and the
  scalar tier on the tiny one), on this host's cores.
Every timed rep of an HBM-bound call (decode, sparse decode, KV write,
gather) is preceded by reading a 1 GiB buffer, so that neither L2 nor the
256 MiB MALL still holds its inputs (the decode is also timed after writing
the buffer, and back to back without a flush).

Before the W warm-up steps, about S seconds (default 1) of the same work run
untimed, so that the GPU clock has left its idle state; the K timed steps are
exactly K. One JSON line is printed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA prefill attn TFLOP/s & % bf16 MFMA peak; decode HBM GB/s & % peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def visible_pairs(new_lens, cached_lens) -> int:
    """(query, key) pairs under the cache-shifted causal mask: query i of a
    sequence with c cached tokens sees c + i + 1 keys."""
    return int(sum(int(n) * int(c) + int(n) * (int(n) + 1) // 2
                   for n, c in zip(new_lens, cached_lens)))


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mla_chunked_prefill_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file: str, name: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current source of the kernel; else None."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(kernel_file):
        return None
    return d.get("traffic_bytes_per_launch")


def warm_clock(fn, seconds: float, torch):
    """Run fn back to back for about `seconds` so that the GPU clock has left
    its idle state before anything is timed (the first milliseconds of work
    otherwise run measurably slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def graph_ms(fn, per_graph: int, reps: int, torch):
    """Capture per_graph back-to-back calls of fn into one HIP graph, replay
    it reps times between two events; returns ms per call. For calls whose
    kernels take less time than the host needs to launch them."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per_graph)


class Flusher:
    """Evicts the caches before a timed rep of an HBM-bound call: reads a 1 GiB
    device buffer (written once here), so that neither L2 nor the 256 MiB MALL
    still holds the call's inputs. Reading leaves clean lines behind; a flush
    that writes the buffer leaves dirty lines whose write-back lands inside
    the timed call (mode "write", kept for comparison)."""

    def __init__(self, torch, mode: str = "read"):
        self.torch = torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        self.mode = mode
        self.k = 0

    def __call__(self):
        if self.mode == "read":
            self.buf.sum()
        elif self.mode == "write":
            self.k = (self.k + 1) & 0x7F
            self.buf.fill_(float(self.k))


def flushed_ms(fn, steps: int, flush, torch):
    """Per-call durations (ms) of fn between two events, each call preceded by
    a cache flush outside the events; returns (mean, median, min)."""
    evs = []
    for _ in range(steps):
        flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return sum(ms) / len(ms), ms[len(ms) // 2], ms[0]


def hbm_ceiling(binding, torch, reps: int = 10):
    """Practical HBM rates: the library's plain streaming-read kernel over
    4 GiB (best of a few grid sizes), torch's sum over the same 4 GiB (reads
    only) and a 2 GiB torch device copy (reads + writes)."""
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def rate(fn, nbytes):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    probe = {}
    for groups in (1024, 2048, 4096, 8192):
        out = torch.empty(groups, dtype=torch.uint32, device="cuda")
        probe[groups] = rate(lambda: binding.mla_hbm_read(x, out, groups), 4 << 30)
    best = max(probe, key=probe.get)
    tsum = rate(lambda: x.sum(), 4 << 30)
    del x
    src = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy = rate(lambda: dst.copy_(src), 4 << 30)
    del src, dst
    return dict(read_gbps=round(probe[best], 1), read_groups=best,
                read_gbps_by_groups={str(k): round(v, 1) for k, v in probe.items()},
                torch_sum_read_gbps=round(tsum, 1), torch_copy_gbps=round(copy, 1),
                how="mla_hbm_read (16-byte streaming loads, 256-thread workgroups) over 4 GiB; "
                    "torch.sum over the same 4 GiB; 2 GiB torch device copy counted as "
                    "read + write")


def event_ms(fn, steps: int, torch):
    """Mean duration of fn between two events on the current stream."""
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / len(evs)


def bench_prefill(args, binding, torch):
    from workloads import prefill_recipe
    from workloads.device import prefill_tensors

    # chunk slots as the plan sizes them (one: the 4096-token prompt fits a
    # 8192-token chunk); the parity tests also run the recipe's spare slot
    wl = prefill_recipe("dsv3_prefill_4k", C=None)
    t = prefill_tensors(wl)
    B, H, T, C = wl.batch, wl.num_heads, wl.buffer_token_size, wl.max_chunks
    Tq = wl.total_q
    lens = wl.seq_lens
    # host bound on any chunk's rows (the host knows the lengths here)
    max_rows = int(min(B * T, sum(min(int(L), T) for L in lens)))
    max_rows = (max_rows + 63) // 64 * 64
    dev = "cuda"
    bro = torch.empty((C, B + 1), dtype=torch.uint32, device=dev)
    co = torch.empty((C, B), dtype=torch.uint32, device=dev)
    bl = torch.empty((C,), dtype=torch.int32, device=dev)
    latn = torch.empty((max_rows, 512), dtype=torch.bfloat16, device=dev)
    krope = torch.empty((max_rows, 64), dtype=torch.bfloat16, device=dev)
    k_nope = torch.empty((H, max_rows, 128), dtype=torch.bfloat16, device=dev)
    v_t = torch.empty((H, 128, max_rows), dtype=torch.bfloat16, device=dev)
    out = torch.empty((Tq, H, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.mla_prefill_attention_workspace_size(B, Tq, H), dtype=torch.uint8,
                     device=dev)
    max_prompt = int(wl.new_lens.max())

    calls = ["plan", "gather", "up_project", "attention"]

    def step(ev):
        def rec(name, fn):
            if ev is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                ev.setdefault(name, []).append((e0, e1))
            else:
                fn()

        rec("plan", lambda: binding.mla_prefill_plan(bro, co, bl, t["input_row_offsets"],
                                                     t["cache_lengths"], T))
        for c in range(C):
            rec("gather", lambda: binding.mla_gather_norm_rope(
                latn, krope, t["kv_cache"], t["page_table"], bro[c], co[c], bl[c:c + 1],
                t["kv_norm_gamma"], t["freqs_cis"], wl.eps))
            rec("up_project", lambda: binding.mla_up_project(k_nope, v_t, latn, t["w_k"],
                                                             t["w_uv"], bl[c:c + 1]))
            rec("attention", lambda: binding.mla_prefill_attention(
                out, t["q"], k_nope, v_t, krope, t["input_row_offsets"], t["cache_lengths"],
                bro[c], co[c], bl[c:c + 1], max_prompt, wl.scale, ws))

    warm_clock(lambda: step(None), args.warm_seconds, torch)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    ev = {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(ev)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    per_call_ms = {}
    for name in calls:
        tot = sum(a.elapsed_time(b) for a, b in ev.get(name, []))
        per_call_ms[name] = tot / args.steps  # ms per step, summed over chunk slots
    # the attention call of the used chunk: C slots, only chunk 0 has rows here
    attn_launch_ms = [a.elapsed_time(b) for a, b in ev["attention"]]
    used = [x for i, x in enumerate(attn_launch_ms) if i % C == 0]
    attn_ms = sum(used) / len(used)
    pairs = visible_pairs(wl.new_lens, wl.cached_lens)
    attn_flop = 2 * (192 + 128) * H * pairs
    rows = int(sum(lens))
    gemm_flop = 2 * rows * 512 * 2 * H * 128
    return dict(
        wl=wl, wall_ms=wall * 1e3, per_call_ms=per_call_ms, attn_ms=attn_ms,
        attn_flop=attn_flop, gemm_flop=gemm_flop, pairs=pairs, max_rows=max_rows)


PEAK_FP8_TFLOPS = 5000.0


def chunk_pairs(bro, co, new_lens, cached_lens, c: int) -> int:
    """Visible (query, key) pairs whose key lies in chunk c: query i of
    sequence b sits at position cached + i and sees the chunk's keys at
    positions co .. co + rows - 1 that are not after it."""
    import numpy as np

    tot = 0
    for b in range(len(new_lens)):
        rows = int(bro[c, b + 1]) - int(bro[c, b])
        n, cb, k0 = int(new_lens[b]), int(cached_lens[b]), int(co[c, b])
        if rows == 0 or n == 0:
            continue
        P = cb + np.arange(n, dtype=np.int64)
        tot += int(np.clip(P - k0 + 1, 0, rows).sum())
    return tot


def bench_prefill_ragged(args, binding, torch, flush, name):
    """A ragged batch with cached prefixes over several chunks (all 128 heads):
    per-call times of every chunk's gather (after a cache flush), up-projection
    and attention, run in pipeline order, and of the whole mla_prefill call."""
    import numpy as np
    from workloads import prefill_recipe
    from workloads.device import prefill_tensors

    wl = prefill_recipe(name)
    t = prefill_tensors(wl)
    B, H, T, C, Tq = wl.batch, wl.num_heads, wl.buffer_token_size, wl.max_chunks, wl.total_q
    fp8 = bool(wl.fp8)
    kdt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    max_rows = (int(min(B * T, sum(min(int(L), T) for L in wl.seq_lens))) + 63) // 64 * 64
    bro, co, bl, _ = binding.plan(t["input_row_offsets"], t["cache_lengths"], T, C)
    bro_h, co_h, bl_h = bro.cpu().numpy(), co.cpu().numpy(), bl.cpu().numpy()
    chunks = [c for c in range(C) if bl_h[c] > 0]
    dev = "cuda"
    latn = torch.empty((max_rows, 512), dtype=torch.bfloat16, device=dev)
    krope = torch.empty((max_rows, 64), dtype=kdt, device=dev)
    k_nope = torch.empty((H, max_rows, 128), dtype=kdt, device=dev)
    v_t = torch.empty((H, 128, max_rows), dtype=torch.bfloat16, device=dev)
    out = torch.empty((Tq, H, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.mla_prefill_attention_workspace_size(B, Tq, H), dtype=torch.uint8,
                     device=dev)
    max_prompt = int(wl.new_lens.max())
    bro_c = [bro[c].contiguous() for c in range(C)]
    co_c = [co[c].contiguous() for c in range(C)]

    def gather(c):
        binding.mla_gather_norm_rope(latn, krope, t["kv_cache"], t["page_table"], bro_c[c],
                                     co_c[c], bl[c:c + 1], t["kv_norm_gamma"], t["freqs_cis"],
                                     wl.eps)

    def up(c):
        binding.mla_up_project(k_nope, v_t, latn, t["w_k"], t["w_uv"], bl[c:c + 1])

    def attn(c):
        binding.mla_prefill_attention(out, t["q"], k_nope, v_t, krope, t["input_row_offsets"],
                                      t["cache_lengths"], bro_c[c], co_c[c], bl[c:c + 1],
                                      max_prompt, wl.scale, ws)

    def pipeline(ev):
        for c in chunks:
            for nm, fn in (("gather", gather), ("up_project", up), ("attention", attn)):
                if ev is None:
                    fn(c)
                    continue
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn(c)
                e1.record()
                ev.setdefault((nm, c), []).append((e0, e1))

    warm_clock(lambda: pipeline(None), args.warm_seconds / 2, torch)
    for _ in range(args.warmup):
        pipeline(None)
    torch.cuda.synchronize()
    ev = {}
    for _ in range(args.steps):
        pipeline(ev)
    torch.cuda.synchronize()
    ms = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in ev.items()}
    # the gather alone after a cache flush (HBM-bound)
    gather_ms = {c: flushed_ms(lambda: gather(c), args.steps, flush, torch)[0] for c in chunks}
    # the whole call (plan given)
    pws = torch.empty(binding.mla_prefill_workspace_size(B, Tq, H, max_rows,
                                                         binding.MLA_FP8_E4M3FN if fp8
                                                         else binding.MLA_BF16),
                      dtype=torch.uint8, device=dev)

    def full():
        binding.mla_prefill(out, t["q"], t["input_row_offsets"], t["cache_lengths"],
                            t["kv_cache"], t["page_table"], bro, co, bl, max_rows, t["w_k"],
                            t["w_uv"], t["kv_norm_gamma"], t["freqs_cis"], max_prompt, wl.scale,
                            wl.eps, pws)

    for _ in range(args.warmup):
        full()
    full_ms = event_ms(full, args.steps, torch)
    pairs = {c: chunk_pairs(bro_h, co_h, wl.new_lens, wl.cached_lens, c) for c in chunks}
    tot_pairs = sum(pairs.values())
    assert tot_pairs == visible_pairs(wl.new_lens, wl.cached_lens)
    f_qk, f_pv = 2 * 192 * H * tot_pairs, 2 * 128 * H * tot_pairs
    attn_ms = sum(ms[("attention", c)] for c in chunks)
    attn_tf = (f_qk + f_pv) / (attn_ms * 1e-3) / 1e12
    rows = {c: int(bl_h[c]) for c in chunks}
    row_bytes = (576 if fp8 else 1152) + 128 + 1024 + (64 if fp8 else 128)
    g_bytes = sum(rows[c] * row_bytes for c in chunks)
    g_ms = sum(gather_ms.values())
    up_flop = sum(2 * rows[c] * 512 * 2 * H * 128 for c in chunks)
    up_ms = sum(ms[("up_project", c)] for c in chunks)
    res = dict(
        batch=B, total_q=Tq, chunks=len(chunks), rows_per_chunk=[rows[c] for c in chunks],
        visible_pairs=tot_pairs, attn_flop=f_qk + f_pv,
        mla_prefill_ms=round(full_ms, 4),
        mla_prefill_attn_tflops=round((f_qk + f_pv) / (full_ms * 1e-3) / 1e12, 2),
        attention_ms_per_chunk=[round(ms[("attention", c)], 4) for c in chunks],
        attention_ms=round(attn_ms, 4), attention_tflops=round(attn_tf, 2),
        up_project_ms=round(up_ms, 4),
        up_project_tflops=round(up_flop / (up_ms * 1e-3) / 1e12, 2),
        gather_ms_per_chunk_flushed=[round(gather_ms[c], 4) for c in chunks],
        gather_bytes=g_bytes, gather_gbps=round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
        gather_frac_hbm=round(g_bytes / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4))
    if fp8:
        # scores on fp8 MFMA, the value product on bf16 MFMA
        t_mixed = f_qk / (PEAK_FP8_TFLOPS * 1e12) + f_pv / (PEAK_BF16_TFLOPS * 1e12)
        res.update(attention_frac_fp8_peak=round(attn_tf / PEAK_FP8_TFLOPS, 4),
                   attention_frac_mixed_roofline=round(t_mixed / (attn_ms * 1e-3), 4),
                   mixed_roofline="t = F_QK / 5.0 PFLOP/s (fp8) + F_PV / 2.5 PFLOP/s (bf16)")
    else:
        res.update(attention_frac_bf16_peak=round(attn_tf / PEAK_BF16_TFLOPS, 4))
    del t, latn, krope, k_nope, v_t, out, ws, pws
    return wl, res


def bench_decode(args, binding, torch, flush, recipe="decode_b64", sinks=False):
    from workloads import decode_recipe
    from workloads.device import decode_tensors

    wl = decode_recipe(recipe)
    t = decode_tensors(wl)
    B, H = wl.batch, wl.num_heads
    max_ctx = int(wl.context_lens.max())
    code = binding.MLA_FP8_E4M3FN if wl.fp8 else binding.MLA_BF16
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(binding.mla_decode_workspace_size(B, H, max_ctx, wl.page_size, 0, code),
                     dtype=torch.uint8, device="cuda")

    sink = torch.linspace(-2.0, 2.0, B, device="cuda", dtype=torch.float32) if sinks else None

    def call():
        binding.mla_decode(out, t["q"], t["context_lengths"], t["kv_cache"], t["page_table"],
                           t["w_uk"], t["w_uv"], max_ctx, wl.scale, ws, attn_sink=sink)

    warm_clock(call, args.warm_seconds / 2, torch)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms, med, mn = flushed_ms(call, args.steps, flush, torch)
    ctx_rows = int(wl.context_lens.astype("int64").sum())
    row_bytes = 576 * (1 if wl.fp8 else 2)
    bytes_alg = (ctx_rows * row_bytes + 2 * H * 512 * 128 * 2 + B * H * 192 * 2 + B * H * 128 * 2)
    flop = 2 * (576 + 512) * H * ctx_rows
    return dict(ms=ms, median_ms=med, min_ms=mn, bytes=bytes_alg, flop=flop, ctx_rows=ctx_rows,
                wl=wl)


def bench_decode_sparse(args, binding, torch, flush, topk=2048):
    """mla_decode_sparse on decode_b64's pool, queries and weights: every
    sequence lists `topk` distinct rows of its own context (uniform positions,
    sorted, mapped through its page table)."""
    import numpy as np
    from workloads import decode_recipe
    from workloads.device import decode_tensors

    wl = decode_recipe("decode_b64")
    t = decode_tensors(wl)
    B, H = wl.batch, wl.num_heads
    rng = np.random.default_rng(10)
    ps = wl.page_size
    idx = np.zeros((B, topk), dtype=np.int32)
    for b in range(B):
        pos = np.sort(rng.choice(int(wl.context_lens[b]), size=topk, replace=False))
        idx[b] = wl.page_table[b, pos // ps] * ps + pos % ps
    d_idx = torch.from_numpy(idx).cuda()
    lens = torch.full((B,), topk, dtype=torch.int32, device="cuda")
    rows = t["kv_cache"].reshape(-1, 576)
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(binding.mla_decode_sparse_workspace_size(B, H, topk, 0, binding.MLA_BF16),
                     dtype=torch.uint8, device="cuda")

    def call():
        binding.mla_decode_sparse(out, t["q"], lens, rows, d_idx, t["w_uk"], t["w_uv"], topk,
                                  wl.scale, ws)

    warm_clock(call, args.warm_seconds / 4, torch)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms, med, mn = flushed_ms(call, args.steps, flush, torch)
    nrows = B * topk
    bytes_alg = nrows * 576 * 2 + 2 * H * 512 * 128 * 2 + B * H * 192 * 2 + B * H * 128 * 2 + nrows * 4
    flop = 2 * (576 + 512) * H * nrows
    return dict(ms=ms, median_ms=med, min_ms=mn, bytes=bytes_alg, flop=flop)


def bench_kv_write(args, binding, torch, flush):
    """mla_kv_write on the prompt of dsv3_prefill_4k: 4096 new tokens' raw
    576-wide rows normalised, rotated and stored in a bf16 pool of 128-row
    pages (shuffled page table). Timed per call after a cache flush (the
    flush keeps the GPU busy while the host issues the call), and as replays
    of a HIP graph of 20 back-to-back calls over the same, cached, buffers."""
    import numpy as np
    from workloads import f32_to_bf16_bits
    from workloads.gen import rope_table_bits

    rng = np.random.default_rng(9)
    n, ps = 4096, 128
    pages = n // ps
    num_pages = pages + 8
    pt = torch.from_numpy(rng.permutation(num_pages)[:pages].reshape(1, pages).astype(np.int32)).cuda()
    bf = lambda a: torch.from_numpy(f32_to_bf16_bits(a.astype(np.float32)).view(np.int16)).view(
        torch.bfloat16).cuda()
    x = bf(rng.standard_normal((n, 576)))
    gamma = bf(1.0 + 0.1 * rng.standard_normal(512))
    freqs = torch.from_numpy(rope_table_bits(n, 64).view(np.int16)).view(torch.bfloat16).cuda()
    cache = torch.zeros((num_pages, ps, 576), dtype=torch.bfloat16, device="cuda")
    offs = torch.tensor([0, n], dtype=torch.uint32, device="cuda")
    clen = torch.tensor([0], dtype=torch.uint32, device="cuda")

    def call():
        binding.mla_kv_write(cache, pt, x, offs, clen, gamma, freqs, 1e-6)

    warm_clock(call, args.warm_seconds / 4, torch)
    ms, med, mn = flushed_ms(call, args.steps, flush, torch)
    gms = graph_ms(call, 20, max(1, args.steps // 2), torch)
    bytes_alg = n * (576 * 2 + 576 * 2 + 64 * 2) + 512 * 2
    return dict(ms=ms, median_ms=med, min_ms=mn, graph_ms=gms, bytes=bytes_alg)


def bench_unified(args, binding, torch):
    """mla_prefill_decode, the graph op as one call, in both branches:
    prefill: dsv3_prefill_4k's prompt arrives as 4096 raw rows (kv_input),
    is written into the pool, and the planned prefill reads every row as
    stored; decode: decode_b64's 64 new tokens arrive raw, are written, and
    each sequence attends over its cache_len + 1 rows. The decode call is
    also timed as a replay of a captured HIP graph."""
    import numpy as np
    from workloads import decode_recipe, f32_to_bf16_bits, prefill_recipe
    from workloads.device import decode_tensors, prefill_tensors
    from workloads.gen import rope_table_bits

    rng = np.random.default_rng(11)

    def bf(a):
        return torch.from_numpy(f32_to_bf16_bits(a.astype(np.float32)).view(np.int16)).view(
            torch.bfloat16).cuda()

    gamma = bf(1.0 + 0.1 * rng.standard_normal(512))
    res = {}

    wl = prefill_recipe("dsv3_prefill_4k")
    t = prefill_tensors(wl)
    Bp, H, T, C, Tq = wl.batch, wl.num_heads, wl.buffer_token_size, wl.max_chunks, wl.total_q
    x = bf(rng.standard_normal((Tq, 576)))
    max_rows = (min(Bp * T, int(sum(min(int(L), T) for L in wl.seq_lens))) + 63) // 64 * 64
    plan_t = binding.plan(t["input_row_offsets"], t["cache_lengths"], T, C)
    max_new, max_cache = int(wl.new_lens.max()), int(wl.cached_lens.max())
    ws = torch.empty(binding.mla_prefill_decode_workspace_size(
        Bp, Tq, H, max_new, max_rows, max_cache, wl.page_size, 0, 0, binding.MLA_BF16),
        dtype=torch.uint8, device="cuda")
    out = torch.empty((Tq, H, 128), dtype=torch.bfloat16, device="cuda")

    def pcall():
        binding.mla_prefill_decode(out, t["q"], t["input_row_offsets"], t["cache_lengths"],
                                   t["kv_cache"], t["page_table"], t["w_uk"], t["w_uv"], gamma,
                                   t["freqs_cis"], max_new, max_cache, wl.scale, wl.eps, ws,
                                   kv_input=x, w_k=t["w_k"], plan_tensors=plan_t,
                                   max_rows=max_rows)

    warm_clock(pcall, args.warm_seconds / 2, torch)
    for _ in range(args.warmup):
        pcall()
    torch.cuda.synchronize()
    res["prefill_ms"] = event_ms(pcall, args.steps, torch)
    del t, ws, out

    dl = decode_recipe("decode_b64")
    d = decode_tensors(dl)
    Bd = dl.batch
    ctx = dl.context_lens.astype(np.int64)
    xd = bf(rng.standard_normal((Bd, 576)))
    freqs = torch.from_numpy(rope_table_bits(int(ctx.max()), 64).view(np.int16)).view(
        torch.bfloat16).cuda()
    offs = torch.arange(Bd + 1, dtype=torch.int64).to(torch.uint32).cuda()
    clen = torch.from_numpy((ctx - 1).astype(np.uint32)).cuda()
    max_cache = int(ctx.max()) - 1
    wsd = torch.empty(binding.mla_prefill_decode_workspace_size(
        Bd, Bd, dl.num_heads, 1, 0, max_cache, dl.page_size, 0, 0, binding.MLA_BF16),
        dtype=torch.uint8, device="cuda")
    outd = torch.empty((Bd, dl.num_heads, 128), dtype=torch.bfloat16, device="cuda")

    def dcall():
        binding.mla_prefill_decode(outd, d["q"], offs, clen, d["kv_cache"], d["page_table"],
                                   d["w_uk"], d["w_uv"], gamma, freqs, 1, max_cache, dl.scale,
                                   1e-6, wsd, kv_input=xd)

    warm_clock(dcall, args.warm_seconds / 2, torch)
    for _ in range(args.warmup):
        dcall()
    torch.cuda.synchronize()
    res["decode_ms"] = event_ms(dcall, args.steps, torch)
    res["decode_graph_ms"] = graph_ms(dcall, 4, max(1, args.steps // 2), torch)
    res["decode_bytes"] = (int(ctx.sum()) * 576 * 2 + 2 * dl.num_heads * 512 * 128 * 2 +
                           Bd * dl.num_heads * (192 + 128) * 2 + Bd * (576 * 2 + 576 * 2))
    return res


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def _head_slice(wl, sel):
    """The prefill workload restricted to the heads in sel (their q, w_k,
    w_uv and w_uk slices)."""
    import dataclasses

    import numpy as np

    d, H = wl.dims, wl.num_heads
    w = dataclasses.replace(wl)
    w.q = np.ascontiguousarray(wl.q[:, sel])
    w.w_k = np.ascontiguousarray(wl.w_k.reshape(H, d.nope, d.lora)[sel].reshape(-1, d.lora))
    w.w_uv = np.ascontiguousarray(wl.w_uv[sel])
    w.w_uk = np.ascontiguousarray(wl.w_uk[sel])
    w.num_heads = len(sel)
    return w


def cpu_baseline(full_wl, heads: int):
    """The oracle as it stands on `heads` of the 128 heads of the same prefill
    workload; returns (attention TFLOP/s on the sample, seconds, threads)."""
    import numpy as np

    from oracle import oracle

    wl = _head_slice(full_wl, list(range(heads)))
    threads = _blas_threads()
    t0 = time.perf_counter()
    out = oracle.prefill(wl)
    sec = time.perf_counter() - t0
    assert np.isfinite(out).all()
    flop = 2 * (192 + 128) * heads * visible_pairs(wl.new_lens, wl.cached_lens)
    return flop / sec / 1e12, sec, threads


def oracle_timings(ragged, dec_wl):
    """The oracle (and, on the tiny batch, the scalar tier) timed on bounded
    samples of the other workloads; rates in algorithmic FLOPs of the sample."""
    import numpy as np

    from oracle import brute, oracle
    from workloads import prefill_recipe

    res = {}
    wl0 = prefill_recipe("tiny_b2")
    f0 = 2 * (192 + 128) * wl0.num_heads * visible_pairs(wl0.new_lens, wl0.cached_lens)
    t0 = time.perf_counter()
    oracle.prefill(wl0)
    s0 = time.perf_counter() - t0
    t0 = time.perf_counter()
    brute.prefill(wl0)
    sb = time.perf_counter() - t0
    res["tiny_b2"] = dict(sample="whole workload", oracle_seconds=round(s0, 4),
                          oracle_gflops=round(f0 / s0 / 1e9, 3),
                          brute_seconds=round(sb, 3), brute_gflops=round(f0 / sb / 1e9, 5),
                          brute_cores=1)
    for name, wl in ragged.items():
        w = _head_slice(wl, [0])
        f = 2 * (192 + 128) * visible_pairs(w.new_lens, w.cached_lens)
        t0 = time.perf_counter()
        out = oracle.prefill(w)
        sec = time.perf_counter() - t0
        assert np.isfinite(out).all()
        res[name] = dict(sample="whole prefill (gather, RMSNorm, RoPE, up-projection, "
                                "attention) of every sequence, head 0 of 128",
                         oracle_seconds=round(sec, 2), oracle_gflops=round(f / sec / 1e9, 3))
    idx = list(range(8))
    f = 2 * (576 + 512) * dec_wl.num_heads * int(dec_wl.context_lens[idx].astype(np.int64).sum())
    t0 = time.perf_counter()
    oracle.decode(dec_wl, batch_indices=idx)
    sec = time.perf_counter() - t0
    res[dec_wl.name] = dict(sample="absorbed decode of sequences 0..7 of 64, all 128 heads",
                            oracle_seconds=round(sec, 2), oracle_gflops=round(f / sec / 1e9, 3))
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_counters(name: str, kernel_file: str):
    """A committed counter summary, if it was taken on the current source of
    its kernel; else None."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(kernel_file):
        return None
    return d


PHASES = ("prefill", "ragged", "decode", "sparse", "kvwrite", "unified", "hbm", "cpu")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="untimed run of the same work before the warm-up steps")
    ap.add_argument("--phases", default=",".join(PHASES),
                    help="comma-separated subset of " + ",".join(PHASES) +
                         " (prefill, the headline, always runs)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode, sparse and unified phases")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timings")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    phases = set(x.strip() for x in args.phases.split(",") if x.strip())
    if args.no_decode:
        phases -= {"decode", "sparse", "unified"}
    if args.no_cpu:
        phases.discard("cpu")

    import torch

    from mla_chunked_prefill_amd import binding

    binding.load()
    torch.cuda.init()
    if args.copy_calib:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flush = Flusher(torch)
    p = bench_prefill(args, binding, torch)
    attn_tflops = p["attn_flop"] / (p["attn_ms"] * 1e-3) / 1e12
    value = p["attn_flop"] / (p["wall_ms"] * 1e-3) / 1e12
    traffic = load_traffic("attn.hip", "attn_dsv3_prefill_4k_counters.json")
    mfma = load_counters("attn_dsv3_prefill_4k_counters.json", "attn.hip")
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q and latent cache, N(0,1/sqrt(512)) weights)",
        "config": {"workload": "dsv3_prefill_4k: batch 1, 4096 new tokens, no cache, "
                               "128 heads, q 192 = 128 nope + 64 rope, v 128, latent 512, "
                               "page 128, buffer_token_size 8192 (one chunk slot), causal",
                   "global_batch": 1, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_attn_kernel<bf16> (mla_prefill_attention)",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flop_per_launch": p["attn_flop"],
            "avg_launch_ms": round(p["attn_ms"], 4),
            "mfma_busy": None if mfma is None else mfma.get("mfma_busy"),
            "valu_per_mfma": None if mfma is None else mfma.get("valu_per_mfma"),
            # the shader clock the counters saw (GRBM cycles over the kernel's
            # duration): the 2.5 PFLOP/s peak assumes 2.4 GHz
            "clock_ghz": None if mfma is None else mfma.get("clock_ghz"),
        },
        "prefill_breakdown_ms": {k: round(v, 4) for k, v in p["per_call_ms"].items()},
        "prefill_end_to_end_tflops": round((p["attn_flop"] + p["gemm_flop"]) /
                                           (p["wall_ms"] * 1e-3) / 1e12, 2),
    }
    ragged = {}
    if "ragged" in phases:
        for key, name in (("prefill_ragged_b16", "ragged_b16_cached"),
                          ("prefill_fp8_ragged_b8", "fp8_ragged_b8_cached")):
            wl, r = bench_prefill_ragged(args, binding, torch, flush, name)
            r["workload"] = (f"{name}: {wl.batch} prompts, new U{{128..4096}}, cached "
                             f"U{{0..8192}}, 128 heads, page 128, buffer_token_size 8192"
                             + (", q and pool float8_e4m3fn" if wl.fp8 else ", bf16"))
            line[key] = r
            ragged[name] = wl
            torch.cuda.empty_cache()
    dec_wl = None
    if "decode" in phases:
        dd = bench_decode(args, binding, torch, flush)
        dec_wl = dd["wl"]
        gbps = dd["bytes"] / (dd["ms"] * 1e-3) / 1e9
        line["decode"] = {
            "workload": "decode_b64: 64 sequences, one new token each, contexts "
                        "U{4096..32768}, 128 heads, 576-wide bf16 latent cache, page 64",
            "ms": round(dd["ms"], 4), "median_ms": round(dd["median_ms"], 4),
            "min_ms": round(dd["min_ms"], 4),
            "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes": dd["bytes"],
            "tflops": round(dd["flop"] / (dd["ms"] * 1e-3) / 1e12, 2),
            "timing": "each call after reading a 1 GiB buffer (cache flush)",
            "split_kernel_traffic": load_traffic("decode.hip", "decode_split_decode_b64_counters.json"),
        }
        d8 = bench_decode(args, binding, torch, flush, "decode_b64_fp8")
        gbps = d8["bytes"] / (d8["ms"] * 1e-3) / 1e9
        line["decode_fp8"] = {
            "workload": "decode_b64_fp8: as decode_b64 with the cache stored float8_e4m3fn "
                        "(unit amax)",
            "ms": round(d8["ms"], 4), "median_ms": round(d8["median_ms"], 4),
            "min_ms": round(d8["min_ms"], 4),
            "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes": d8["bytes"],
            "tflops": round(d8["flop"] / (d8["ms"] * 1e-3) / 1e12, 2),
            "split_kernel_traffic": load_traffic("decode.hip",
                                                 "decode_split_decode_b64_fp8_counters.json"),
        }
        dk = bench_decode(args, binding, torch, flush, sinks=True)
        line["decode"]["ms_with_sinks"] = round(dk["ms"], 4)
        flush.mode = "write"
        dw = bench_decode(args, binding, torch, flush)
        flush.mode = "none"
        dn = bench_decode(args, binding, torch, flush)
        flush.mode = "read"
        line["decode"]["ms_after_write_flush"] = round(dw["ms"], 4)
        line["decode"]["ms_back_to_back_no_flush"] = round(dn["ms"], 4)
    if "sparse" in phases:
        ds = bench_decode_sparse(args, binding, torch, flush)
        gbps = ds["bytes"] / (ds["ms"] * 1e-3) / 1e9
        line["decode_sparse"] = {
            "workload": "mla_decode_sparse: decode_b64's 64 sequences, each attending over "
                        "2048 distinct rows of its own context listed by physical index",
            "ms": round(ds["ms"], 4), "median_ms": round(ds["median_ms"], 4),
            "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes": ds["bytes"],
            "tflops": round(ds["flop"] / (ds["ms"] * 1e-3) / 1e12, 2),
            "timing": "each call after reading a 1 GiB buffer (cache flush)",
        }
    if "kvwrite" in phases:
        kw = bench_kv_write(args, binding, torch, flush)
        gbps = kw["bytes"] / (kw["ms"] * 1e-3) / 1e9
        line["kv_write"] = {
            "workload": "mla_kv_write: the 4096 new tokens of dsv3_prefill_4k, raw 576-wide "
                        "rows normalised, rotated and stored into a bf16 pool of 128-row pages",
            "ms": round(kw["ms"], 5), "median_ms": round(kw["median_ms"], 5),
            "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes": kw["bytes"],
            "timing": "each call after reading a 1 GiB buffer (cache flush); a 10 MB call is latency-bound",
            "graph_replay_ms_cached": round(kw["graph_ms"], 5),
        }
    if "unified" in phases:
        un = bench_unified(args, binding, torch)
        gbps = un["decode_bytes"] / (un["decode_ms"] * 1e-3) / 1e9
        line["prefill_decode"] = {
            "workload": "mla_prefill_decode, the graph op as one call: prefill branch on "
                        "dsv3_prefill_4k with its 4096 raw rows written first and every row "
                        "read as stored; decode branch on decode_b64 with each new token's "
                        "raw row written first",
            "prefill_ms": round(un["prefill_ms"], 4),
            "prefill_attn_tflops": round(p["attn_flop"] / (un["prefill_ms"] * 1e-3) / 1e12, 2),
            "decode_ms": round(un["decode_ms"], 4),
            "decode_graph_replay_ms": round(un["decode_graph_ms"], 4),
            "decode_achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "decode_frac": round(gbps / PEAK_HBM_GBPS, 4),
        }
    if "hbm" in phases:
        del flush
        torch.cuda.empty_cache()
        line["hbm_ceiling"] = hbm_ceiling(binding, torch)
        line["hbm_ceiling"]["spec_gbps"] = PEAK_HBM_GBPS
    if "cpu" in phases:
        tf, sec, threads = cpu_baseline(p["wl"], args.cpu_heads)
        line["cpu_baseline"] = {
            "value": round(tf, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 NumPy oracle, whole prefill (gather, RMSNorm, RoPE, up-projection, "
                      f"attention) of dsv3_prefill_4k restricted to {args.cpu_heads} of 128 "
                      f"heads; {sec:.1f} s; rate in attention FLOPs of the sample",
            "seconds": round(sec, 2),
            "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
        }
        if ragged and dec_wl is not None:
            line["cpu_baseline"]["other_workloads"] = oracle_timings(ragged, dec_wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
