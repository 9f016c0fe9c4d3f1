"""The C ABI library loads, exports every declared symbol, and rejects bad
host arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from mla_chunked_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mla_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmla.so is not built (run python -m mla_chunked_prefill_amd.build)")
    return binding.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(binding.EXPORTED) == names


def test_status_strings(lib):
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(-1) == b"invalid argument"
    assert lib.mla_status_string(-3) == b"workspace missing or too small"


def test_invalid_arguments_are_rejected_on_the_host(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    # null output pointer
    st = lib.mla_prefill_plan(None, fake, fake, None, fake, fake, 2, 3, 8, None)
    assert st == -1 and b"null" in lib.mla_last_error()
    # zero buffer_token_size
    assert lib.mla_prefill_plan(fake, fake, fake, None, fake, fake, 2, 3, 0, None) == -1
    # batch * T overflows 31 bits
    assert lib.mla_prefill_plan(fake, fake, fake, None, fake, fake, 4096, 1, 1 << 20, None) == -1
    # unsupported dtype
    assert lib.mla_up_project(fake, fake, 7, fake, fake, fake, fake, 2, 128, None) == -2
    # a tensor pointer that is not 16-byte aligned
    odd = P(0x1008)
    assert lib.mla_up_project(fake, odd, 0, fake, fake, fake, fake, 2, 128, None) == -1
    assert b"aligned" in lib.mla_last_error()
    assert lib.mla_decode(fake, fake, fake, odd, 0, fake, fake, fake, 4, 8, 16, 100, 50, 1000, 0,
                          0.1, None, fake, 1 << 40, None) == -1
    # KV write: null input, unsupported cache dtype, misaligned cache
    assert lib.mla_kv_write(fake, 0, fake, None, fake, fake, fake, fake, 2, 10, 16, 4, 8, 64,
                            1e-6, None) == -1
    assert lib.mla_kv_write(fake, 7, fake, fake, fake, fake, fake, fake, 2, 10, 16, 4, 8, 64,
                            1e-6, None) == -2
    assert lib.mla_kv_write(odd, 0, fake, fake, fake, fake, fake, fake, 2, 10, 16, 4, 8, 64,
                            1e-6, None) == -1
    # no new tokens: nothing to do, nothing enqueued
    assert lib.mla_kv_write(fake, 0, fake, fake, fake, fake, fake, fake, 2, 0, 16, 4, 8, 64,
                            1e-6, None) == 0
    # sparse decode: max_topk beyond the index stride; no index list
    need = lib.mla_decode_sparse_workspace_size(4, 8, 100, 0, 0)
    assert need > 0
    assert lib.mla_decode_sparse(fake, fake, fake, fake, 0, fake, 64, fake, fake, 4, 8, 1000, 100,
                                 0, 0.1, None, fake, need, None) == -1
    assert lib.mla_decode_sparse(fake, fake, fake, fake, 0, None, 128, fake, fake, 4, 8, 1000, 100,
                                 0, 0.1, None, fake, need, None) == -1
    # max_rows not a multiple of 64
    assert lib.mla_up_project(fake, fake, 0, fake, fake, fake, fake, 2, 100, None) == -1
    # workspace too small
    need = lib.mla_decode_workspace_size(4, 8, 1000, 16, 0, 0)
    assert need > 0
    st = lib.mla_decode(fake, fake, fake, fake, 0, fake, fake, fake, 4, 8, 16, 100, 50, 1000, 0,
                        0.1, None, fake, need - 1, None)
    assert st == -3
    # heads beyond what decode supports
    assert lib.mla_decode(fake, fake, fake, fake, 0, fake, fake, fake, 4, 256, 16, 100, 50, 1000,
                          0, 0.1, None, fake, 1 << 40, None) == -1


def test_noalloc_decode_rejects_before_any_launch(lib):
    fake = ctypes.c_void_p(0x1000)
    args = [fake, fake, fake, fake, 0, fake, fake, fake, 64, 128, 64, 512, 10000, 32768]
    # null input
    assert lib.mla_decode_noalloc(fake, None, *args[2:], 0, 0.1, None, None) == -1
    # a decode whose workspace exceeds the fixed scratch array (128 MiB): the
    # size check comes before the device is touched
    need = lib.mla_decode_workspace_size(64, 128, 32768, 64, 65536, 0)
    assert need > (128 << 20)
    assert lib.mla_decode_noalloc(*args, 65536, 0.1, None, None) == -3
    assert b"scratch" in lib.mla_last_error()
    # the default partition count of a 64 x 32k, 128-head decode fits
    assert lib.mla_decode_workspace_size(64, 128, 32768, 64, 0, 0) <= (128 << 20)


def test_workspace_sizes_grow_with_problem(lib):
    a = lib.mla_prefill_workspace_size(2, 100, 4, 256, 0)
    b = lib.mla_prefill_workspace_size(2, 100, 4, 512, 0)
    c = lib.mla_prefill_workspace_size(2, 100, 4, 512, 1)
    assert 0 < a < b and c < b
    assert lib.mla_prefill_workspace_size(0, 100, 4, 512, 0) == 0
    assert lib.mla_prefill_attention_workspace_size(2, 100, 4) < a


def _unified_call(lib, **over):
    """mla_prefill_decode with fake device pointers (never dereferenced: every
    case below fails, or has nothing to do, before the first launch)."""
    fake = ctypes.c_void_p(0x1000)
    a = dict(output=fake, q=fake, kv_input=None, offs=fake, clen=fake, cache=fake, cache_dtype=0,
             page_table=fake, bro=fake, co=fake, bl=fake, max_chunks=2, max_rows=512, w_k=fake,
             w_uk=fake, w_uv=fake, gamma=fake, freqs=fake, B=4, total_q=4, H=8, max_seq_len=1,
             ps=16, maxp=64, num_pages=100, max_cache_len=900, freqs_len=1024, scale=0.1,
             eps=1e-6, d_indices=None, stride=0, topk=None, sink=None, num_partitions=0,
             ws=fake, ws_bytes=1 << 40, stream=None)
    a.update(over)
    return lib.mla_prefill_decode(*a.values())


def test_unified_entry_checks_and_workspace(lib):
    fake = ctypes.c_void_p(0x1000)
    # decode takes one token per sequence
    assert _unified_call(lib, total_q=5) == -1
    assert b"one new token" in lib.mla_last_error()
    # max_seq_len 0 goes with total_q 0; then there is nothing to do
    assert _unified_call(lib, max_seq_len=0) == -1
    assert _unified_call(lib, max_seq_len=0, total_q=0, ws=None, ws_bytes=0) == 0
    # prefill needs the plan and w_k
    assert _unified_call(lib, max_seq_len=7, total_q=20, bro=None) == -1
    assert _unified_call(lib, max_seq_len=7, total_q=20, w_k=None) == -1
    # sparse decode needs the lengths and a positive stride
    assert _unified_call(lib, d_indices=fake, stride=64) == -1
    assert _unified_call(lib, d_indices=fake, topk=fake, stride=0) == -1
    # a KV write needs gamma and freqs
    assert _unified_call(lib, kv_input=fake, gamma=None) == -1
    # workspaces: the selected branch's, and too small is rejected
    dec = lib.mla_prefill_decode_workspace_size(4, 4, 8, 1, 0, 900, 16, 0, 0, 0)
    assert dec == lib.mla_decode_workspace_size(4, 8, 901, 16, 0, 0) > 0
    sp = lib.mla_prefill_decode_workspace_size(4, 4, 8, 1, 0, 900, 16, 64, 0, 1)
    assert sp == lib.mla_decode_sparse_workspace_size(4, 8, 64, 0, 1) > 0
    pf = lib.mla_prefill_decode_workspace_size(4, 20, 8, 7, 512, 900, 16, 0, 0, 0)
    assert pf == lib.mla_prefill_workspace_size(4, 20, 8, 512, 0) > 0
    assert lib.mla_prefill_decode_workspace_size(0, 4, 8, 1, 0, 900, 16, 0, 0, 0) == 0
    assert _unified_call(lib, ws_bytes=dec - 1) == -3
    assert _unified_call(lib, max_seq_len=7, total_q=20, ws_bytes=pf - 1) == -3
