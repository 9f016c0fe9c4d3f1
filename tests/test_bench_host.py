"""Host-side checks of the benchmark script (no GPU needed).

- it refuses more than one GPU, with the reason, before touching a device;
- its count of (query, key) pairs under the cache-shifted causal mask, the
  denominator of every attention TFLOP/s it reports, equals a brute-force
  count over small batches;
- the committed counter summaries it reads (`profiles/*_counters.json`) were
  taken on the current kernel sources, so its roofline object carries their
  traffic, MFMA-busy and clock figures instead of nulls.
"""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402  (module level imports no GPU library)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["n_gpus"] == 2 and "one GPU" in d["error"]


def test_visible_pairs_matches_a_brute_force_count():
    rng = np.random.default_rng(5)
    for _ in range(40):
        B = int(rng.integers(1, 6))
        new = rng.integers(0, 30, B)
        cached = rng.integers(0, 50, B)
        # query i of a sequence sits at position c + i and sees keys 0 .. c + i
        brute = sum(1 for n, c in zip(new, cached)
                    for i in range(int(n)) for j in range(int(c) + int(n)) if j <= int(c) + i)
        assert bench.visible_pairs(new, cached) == brute


def test_counter_summaries_were_taken_on_the_current_sources():
    names = sorted(f for f in os.listdir(bench.PROFILES) if f.endswith("_counters.json"))
    assert names, "no counter summaries committed"
    for f in names:
        with open(os.path.join(bench.PROFILES, f)) as fh:
            d = json.load(fh)
        assert d["source_hash"] == bench.source_hash(*d["source_files"]), f
        assert d["traffic_bytes_per_launch"] > 0 and 0.0 <= d["mfma_busy"] <= 1.0, f
