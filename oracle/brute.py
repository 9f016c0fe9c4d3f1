"""Scalar pure-Python tier of the oracle, for tiny inputs.

TEST INFRASTRUCTURE. Only tests/ call this module. Every step is an explicit
loop over Python floats (IEEE double), written independently of oracle.py so
that the two tiers pin each other: on tiny inputs they must agree to rounding.

The planner here walks tokens one at a time instead of using the closed form:
position p of sequence b belongs to chunk p // T, since T caps the tokens a
sequence contributes to any one chunk (mla_prefill_plan page, Args
"buffer_token_size"), and the plan arrays are read off that assignment.
"""
from __future__ import annotations

import math
import struct


def bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e4m3fn(code: int) -> float:
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)        # m/8 * 2^-6
    return s * math.ldexp(8 + m, e - 10)    # (1 + m/8) * 2^(e-7)


def _val(x, fp8: bool) -> float:
    return e4m3fn(x) if fp8 else bf16(x)


# --------------------------------------------------------------------------
# Token-walk planner
# --------------------------------------------------------------------------


def plan_walk(input_row_offsets, cache_lengths, T: int, C: int):
    """Plan by assigning every token to its chunk and counting.

    Returns plain lists: buffer_row_offsets [C][B+1], cache_offsets [C][B],
    buffer_lengths [C]. A sequence with no token in a chunk gets cache offset
    L_b if all its tokens are in earlier chunks (there are no later ones).
    """
    offs = [int(x) for x in input_row_offsets]
    clen = [int(x) for x in cache_lengths]
    B = len(clen)
    counts = [[0] * B for _ in range(C)]
    first = [[None] * B for _ in range(C)]
    L = [offs[b + 1] - offs[b] + clen[b] for b in range(B)]
    for b in range(B):
        for p in range(L[b]):
            c = p // T
            if c >= C:
                raise ValueError("max_chunks too small for this batch")
            counts[c][b] += 1
            if first[c][b] is None:
                first[c][b] = p
    bro, co, bl = [], [], []
    for c in range(C):
        row = [0]
        for b in range(B):
            row.append(row[-1] + counts[c][b])
        bro.append(row)
        co.append([first[c][b] if first[c][b] is not None else L[b] for b in range(B)])
        bl.append(row[-1] if row[-1] > 0 else -1)
    return bro, co, bl


# --------------------------------------------------------------------------
# Attention, loops only
# --------------------------------------------------------------------------


def prefill(wl):
    """out[t][h][d] as nested lists, by scalar loops over the definitions."""
    d = wl.dims
    fp8 = wl.fp8
    H = wl.num_heads
    ps = wl.page_size
    offs = [int(x) for x in wl.input_row_offsets]
    clen = [int(x) for x in wl.cache_lengths]
    depth = d.lora + d.rope
    pool = wl.pool.reshape(-1, depth)
    gamma = [bf16(x) for x in wl.gamma]
    out = []
    for b in range(len(clen)):
        n = offs[b + 1] - offs[b]
        L = n + clen[b]
        # processed keys of every position of this sequence
        xs, ys = [], []
        for p in range(L):
            slot = int(wl.page_table[b][p // ps]) * ps + p % ps
            raw = [_val(v, fp8) for v in pool[slot]]
            x = raw[:d.lora]
            y = raw[d.lora:]
            ss = 0.0
            for v in x:
                ss += v * v
            inv = 1.0 / math.sqrt(ss / d.lora + wl.eps)
            xs.append([x[l] * gamma[l] * inv for l in range(d.lora)])
            f = [bf16(v) for v in wl.freqs[p]]
            yt = [0.0] * d.rope
            for i in range(d.rope // 2):
                a, bb = y[2 * i], y[2 * i + 1]
                c, s = f[2 * i], f[2 * i + 1]
                yt[2 * i] = a * c - bb * s
                yt[2 * i + 1] = a * s + bb * c
            ys.append(yt)
        # up-projected keys and values of every position, per head
        kn = [[None] * L for _ in range(H)]
        vv = [[None] * L for _ in range(H)]
        for h in range(H):
            for p in range(L):
                kv = []
                for e in range(d.nope):
                    w = wl.w_k[h * d.nope + e]
                    acc = 0.0
                    for l in range(d.lora):
                        acc += bf16(w[l]) * xs[p][l]
                    kv.append(acc)
                kn[h][p] = kv
                vrow = []
                for e in range(d.v):
                    w = wl.w_uv[h][e]
                    acc = 0.0
                    for l in range(d.lora):
                        acc += bf16(w[l]) * xs[p][l]
                    vrow.append(acc)
                vv[h][p] = vrow
        for i in range(n):
            t = offs[b] + i
            P = clen[b] + i
            row = []
            for h in range(H):
                qv = [_val(v, fp8) for v in wl.q[t][h]]
                scores = []
                for p in range(P + 1):
                    s = 0.0
                    for e in range(d.nope):
                        s += qv[e] * kn[h][p][e]
                    for e in range(d.rope):
                        s += qv[d.nope + e] * ys[p][e]
                    scores.append(s * wl.scale)
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                tot = sum(ex)
                o = [0.0] * d.v
                for p in range(P + 1):
                    a = ex[p] / tot
                    for e in range(d.v):
                        o[e] += a * vv[h][p][e]
                row.append(o)
            out.append(row)
    return out


def decode(wl):
    """Absorbed decode out[b][h][d] by scalar loops."""
    d = wl.dims
    fp8 = wl.fp8
    H = wl.num_heads
    ps = wl.page_size
    depth = d.lora + d.rope
    pool = wl.pool.reshape(-1, depth)
    out = []
    for b in range(len(wl.context_lens)):
        ctx = int(wl.context_lens[b])
        Z = []
        for p in range(ctx):
            slot = int(wl.page_table[b][p // ps]) * ps + p % ps
            Z.append([_val(v, fp8) for v in pool[slot]])
        row = []
        for h in range(H):
            qv = [bf16(v) for v in wl.q[b][h]]
            qlat = []
            for l in range(d.lora):
                acc = 0.0
                for e in range(d.nope):
                    acc += bf16(wl.w_uk[h][l][e]) * qv[e]
                qlat.append(acc)
            scores = []
            for p in range(ctx):
                s = 0.0
                for l in range(d.lora):
                    s += qlat[l] * Z[p][l]
                for e in range(d.rope):
                    s += qv[d.nope + e] * Z[p][d.lora + e]
                scores.append(s * wl.scale)
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            tot = sum(ex)
            olat = [0.0] * d.lora
            for p in range(ctx):
                a = ex[p] / tot
                for l in range(d.lora):
                    olat[l] += a * Z[p][l]
            o = []
            for e in range(d.v):
                acc = 0.0
                for l in range(d.lora):
                    acc += bf16(wl.w_uv[h][e][l]) * olat[l]
                o.append(acc)
            row.append(o)
        out.append(row)
    return out
