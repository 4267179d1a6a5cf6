"""Host logic of bench.py, on the CPU: the algorithmic byte and flop counts
behind every roofline fraction, the match of counter summaries to kernel
sources, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_relative_bias_amd import inputs  # noqa: E402


def _brute_counts(b):
    """The same quantities counted key by key from the visibility rule
    (0 <= p - j < W, any p - j >= 0 without a window) and the bias clamp
    (distance d reads entry min(d, R - 1))."""
    e = 2 if b.dtype == "bf16" else 4
    Hq, Hkv, D, W, R = b.num_q_heads, b.num_kv_heads, b.head_dim, b.window, b.rel_len
    pairs = 0
    entries = 0
    keys = 0
    pages = 0
    for s in range(b.num_seqs):
        n, L = int(b.q_lens[s]), int(b.seq_lens[s])
        seen = set()
        for t in range(n):
            p = L - n + t
            vis = [j for j in range(L) if p - j >= 0 and (W <= 0 or p - j < W)]
            pairs += len(vis)
            entries += len({min(p - j, R - 1) for j in vis})
            seen.update(vis)
        keys += len(seen)
        pages += len({j // 16 for j in seen})
    return {"flops": 4 * D * Hq * pairs,
            "bytes": keys * Hkv * D * e * 2 + entries * Hq * e + b.total_q * Hq * D * e * 2
            + 4 * pages}


@pytest.mark.parametrize("L,n,W,R", [
    ([300, 77, 1], [300, 77, 1], 64, 64),      # windowed prefill, L = 1
    ([500, 90], [1, 40], 0, 128),              # causal, clamp active, chunk on a cache
    ([40, 17], [40, 17], 0, 64),               # causal, no clamp
    ([1000, 33], [1, 1], 100, 100),            # decode rows with a window
])
def test_algorithmic_matches_brute_force(L, n, W, R):
    b = inputs.make_batch(np.random.default_rng(0), np.array(L), np.array(n), num_q_heads=6,
                          num_kv_heads=2, head_dim=64, window=W, rel_len=R,
                          max_blocks_per_seq=64)
    got = bench.algorithmic(b)
    want = _brute_counts(b)
    assert got["flops"] == want["flops"]
    assert got["bytes"] == want["bytes"]


def test_traffic_summaries_match_only_their_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    rel = os.path.relpath(str(src), bench.ROOT)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_w.json").write_text(json.dumps({
        "kernel_sources_sha256_16": {rel: bench.source_hash(str(src))},
        "hbm_bytes_per_step": 1234}))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.traffic_from_profiles("w", [str(src)]) == 1234
    assert bench.traffic_from_profiles("missing", [str(src)]) is None
    src.write_text("kernel v2\n")                         # the source moved on
    assert bench.traffic_from_profiles("w", [str(src)]) is None


def test_committed_summaries_name_the_kernels_each_record_runs():
    # Every committed traffic summary lists the kernel source(s) of its
    # record and device.hpp, so that bench.py can tell when it is stale.
    names = [f for f in os.listdir(bench.PROFILES) if f.startswith("traffic_") and f.endswith(".json")]
    assert names
    for f in names:
        with open(os.path.join(bench.PROFILES, f)) as fh:
            rec = json.load(fh)
        srcs = set(rec["kernel_sources_sha256_16"])
        assert "paged_relative_bias_amd/csrc/device.hpp" in srcs, f
        want = set()
        if "decode" in f or "split" in f:
            want.add("paged_relative_bias_amd/csrc/decode.hip")
        if "prefill" in f or "mixed" in f:
            want.add("paged_relative_bias_amd/csrc/prefill_bf16.hip")
        assert want <= srcs, f
        assert rec["hbm_bytes_per_step"] > 0


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
