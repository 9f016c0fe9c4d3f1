"""The allocation-free decode entry (mla_decode_noalloc, scratch in a fixed
array inside the library) against the decode entry with a caller workspace:
the same kernels, so the outputs must agree bit for bit, and both must meet
the oracle's bf16 bounds. Two calls in a row, the second on a smaller batch,
so the second runs over what the first left in the shared array."""
import numpy as np
import pytest
import torch

from oracle import oracle
from workloads import decode_recipe, make_decode
from workloads.device import bf16_bits, decode_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mla_chunked_prefill_amd import binding
    binding.load()
    return binding


def _both(B, wl, parts, sink=None):
    t = decode_tensors(wl)
    Bn, H = wl.batch, wl.num_heads
    max_ctx = int(wl.context_lens.max())
    nan = lambda: torch.full((Bn, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    a, b = nan(), nan()
    B.mla_decode_noalloc(a, t["q"], t["context_lengths"], t["kv_cache"], t["page_table"],
                         t["w_uk"], t["w_uv"], max_ctx, wl.scale, num_partitions=parts,
                         attn_sink=sink)
    B.decode(t["q"], t["context_lengths"], t["kv_cache"], t["page_table"], t["w_uk"], t["w_uv"],
             max_ctx, wl.scale, num_partitions=parts, output=b, attn_sink=sink)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_decode_matches_decode_on_two_calls(B):
    print("noalloc: decode_b64", flush=True)
    big = decode_recipe("decode_b64")
    a, b = _both(B, big, 0)
    assert torch.equal(a, b)
    assert torch.isfinite(a.float()).all()
    print("noalloc: smaller batch after it", flush=True)
    small = make_decode("na", 71, [1, 37, 300, 64, 1000], 8, 16)
    sink = torch.tensor([0.5, -1.0, 2.0, 0.0, 1.5], dtype=torch.float32, device="cuda")
    a, b = _both(B, small, 3, sink)
    assert torch.equal(a, b)
    ref = oracle.decode(small, sinks=sink.cpu().numpy().astype(np.float64))
    got = oracle.bf16_to_f64(bf16_bits(a))
    err = np.abs(got - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, err.max()


def test_noalloc_decode_rejects_an_oversized_decode(B):
    wl = make_decode("na2", 72, [40, 50], 8, 16)
    t = decode_tensors(wl)
    out = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MlaError) as e:
        # 65536 partitions of partial states: far beyond the 128 MiB array
        B.mla_decode_noalloc(out, t["q"], t["context_lengths"], t["kv_cache"],
                             t["page_table"], t["w_uk"], t["w_uv"], 50, wl.scale,
                             num_partitions=65536)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert (out == 0).all()
