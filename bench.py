#!/usr/bin/env python3
"""Throughput of relative-bias paged attention on one MI355X (gfx950).

One step is one call of the library's hot path on one synthetic batch, with
its inputs already resident in HBM:
  * decode workloads: inkling_rel_attn_decode (split-KV decode kernel, plus
    the log-sum-exp merge kernel when it uses more than one split);
  * prefill workloads: inkling_rel_attn_prefill;
  * global_mixed_split: prefill of the 4 chunks, then decode of the 48 rows,
    back to back on one stream.

The JSON line's headline (`value`, `roofline`, `cpu_baseline`) is the
local-layer decode batch (64 sequences, contexts U[1024, 8192], 48 query /
16 KV heads, head_dim 128, window 512, bf16).  Without --workload the line
also carries `workloads`: one record of the same fields for every other
serving configuration (global decode at the library's split count and at 1,
8 and 32 splits, and replayed from a HIP graph; local prefill; the global
mixed batch as one call and split; long-context global decode; and the
smaller model's shapes).

Timing: a settle phase of back-to-back steps covering at least
--settle-ms of GPU time (the clocks and the memory system reach their
steady state only after tens of ms of sustained work: local decode runs
3-4% slower over its first few ms), then W untimed warm-up steps, then
exactly K steps bracketed by torch.cuda.synchronize(); two HIP events on the launch stream around the
timed region give the back-to-back mean launch time, from which the
roofline fractions are computed, and a separate pass with an event pair
around every step (at least 50) gives the median and p10/p90 launch
durations, reported beside it.  Consecutive steps read
different device copies of the inputs (replicas rotated round-robin, at
least 512 MB apart) so no step finds its data in the 256 MB Infinity Cache
left behind by the previous one, as in a real forward where consecutive
attention calls belong to different layers.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s & HBM GB/s fraction; prefill tokens/s & MFMA util fraction"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20
DECODE_KERNEL_SRC = os.path.join(ROOT, "paged_relative_bias_amd", "csrc", "decode.hip")
PREFILL_KERNEL_SRC = os.path.join(ROOT, "paged_relative_bias_amd", "csrc", "prefill.hip")
# bf16 with head_dim 128 and no append (every bench workload without --append).
PREFILL_BF16_KERNEL_SRC = os.path.join(ROOT, "paged_relative_bias_amd", "csrc", "prefill_bf16.hip")
DEVICE_HELPERS_SRC = os.path.join(ROOT, "paged_relative_bias_amd", "csrc", "device.hpp")
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "local_decode"
# The other records: generator -> [(record name, decode split count (0 =
# the library's choice)[, launched as HIP graph replays])]; each generated
# batch serves all of its records.
SECONDARY = [
    ("global_decode", [("global_decode", 0), ("global_decode_s1", 1),
                       ("global_decode_s8", 8), ("global_decode_s32", 32),
                       ("global_decode_graph", 0, True)]),
    ("local_prefill", [("local_prefill", 0)]),
    ("global_mixed", [("global_mixed", 0), ("global_mixed_split", 0)]),
    ("long_global_decode", [("long_global_decode", 0)]),
    ("long_global_prefill", [("long_global_prefill", 0)]),
    ("small_local_decode", [("small_local_decode", 0)]),
    ("small_global_decode", [("small_global_decode", 0)]),
    ("small_local_prefill", [("small_local_prefill", 0)]),
]
WORKLOAD_CHOICES = ["local_decode", "global_decode", "local_prefill", "global_mixed",
                    "global_mixed_split", "tiny_prefill", "long_global_decode",
                    "long_global_prefill",
                    "small_local_decode", "small_global_decode", "small_local_prefill"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(batch):
    """Bytes the method must move and flops it must do for one call.

    Per sequence b with query positions [L_b - n_b, L_b):
      keys_read_b  = keys visible to at least one of its queries
      pairs_b      = sum over its queries of visible keys (per head)
      entries_b    = sum over its queries of distinct bias entries read,
                     min(visible keys, R) (distances >= R - 1 share entry R - 1)
    bytes = sum_b keys_read_b * Hkv * D * e * 2     (K and V, once per KV head)
          + sum_b entries_b * Hq * e                (bias entries used)
          + total_q * Hq * D * e * 2                (q in, out)
          + 4 * sum_b ceil(L_b / 16)-pages touched  (block table)
    flops = 4 * D * Hq * sum_b pairs_b              (QK^T and PV)
    e = element size (2 for bf16).  Masked, padded and split work excluded.
    """
    e = 2 if batch.dtype == "bf16" else 4
    Hq, Hkv, D, W = batch.num_q_heads, batch.num_kv_heads, batch.head_dim, batch.window
    R = batch.rel_len
    kv = pages = 0
    pairs = entries = 0
    for b in range(batch.num_seqs):
        n, L = int(batch.q_lens[b]), int(batch.seq_lens[b])
        if n == 0:
            continue
        p = np.arange(L - n, L, dtype=np.int64)
        vis = np.minimum(p + 1, W) if W > 0 else p + 1
        pairs += int(vis.sum())
        entries += int(np.minimum(vis, R).sum())
        lo = max(0, L - n - W + 1) if W > 0 else 0
        keys = L - lo
        kv += keys * Hkv * D * e * 2
        pages += (L - 1) // 16 - lo // 16 + 1
    bias = entries * Hq * e
    qo = batch.total_q * Hq * D * e * 2
    total = kv + bias + qo + 4 * pages
    return {"bytes": total, "kv": kv, "bias": bias, "qo": qo,
            "block_table": 4 * pages, "flops": 4 * D * Hq * pairs, "pairs": pairs}


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(record, kernel_srcs):
    """HBM bytes per step from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"traffic_{record}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    want = rec.get("kernel_sources_sha256_16") or {}
    if not want:
        return None
    for src in kernel_srcs:
        rel = os.path.relpath(src, ROOT)
        if want.get(rel) != source_hash(src):
            return None
    return rec.get("hbm_bytes_per_step")


def cpu_baseline(batch, budget_s):
    """The fp64 oracle as it stands, on the host cores, over the whole batch
    (decode) or over a bounded, seeded subset of (row, head) pairs (prefill),
    scaled to query tokens per second."""
    import oracle

    threads = oracle.max_threads()
    Hq = batch.num_q_heads
    total_rows = batch.total_q * Hq
    rng = np.random.default_rng(0)
    probe = rng.choice(total_rows, size=min(256, total_rows), replace=False)
    t0 = time.perf_counter()
    oracle.run_batch(batch, rows=probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    if per_row * total_rows <= budget_s:
        rows = None
        frac = 1.0
        sample = f"whole batch: {batch.total_q} rows x {Hq} heads"
    else:
        n = int(min(total_rows, max(256, budget_s / max(per_row, 1e-9))))
        rows = rng.choice(total_rows, size=n, replace=False)
        frac = n / total_rows
        sample = f"{n} random (row, head) pairs of {total_rows} ({100 * frac:.2f}%)"
    # Repeat short runs until at least ~2 s have been timed (mean per run).
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.run_batch(batch, rows=rows)
        runs += 1
        if time.perf_counter() - t0 >= min(2.0, budget_s):
            break
    dt = (time.perf_counter() - t0) / runs
    tokens = batch.total_q * frac
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds_per_run": round(dt, 4),
            "runs": runs}


def spike_bias(batch, amount=60.0):
    """+amount on the distance-0 bias entry of every row: the query's own key
    then has a logit far above every other, which sends every workgroup of
    the fixed-reference softmax into its second pass."""
    import dataclasses
    import torch
    rel = batch.rel_logits.clone()
    rel[:, :, 0] = (rel[:, :, 0].float() + amount).to(rel.dtype)
    return dataclasses.replace(batch, rel_logits=rel)


class Workload:
    """Device replicas of one configuration and the pre-marshalled calls of
    one step on each."""

    def __init__(self, name, batch, *, splits, append, graph, replicas, dev):
        import torch
        from paged_relative_bias_amd import binding, inputs

        self.name = name
        self.batch = batch
        split_mixed = name == "global_mixed_split"
        parts = list(inputs.split_mixed(batch)) if split_mixed else [batch]
        self.parts = [p for p in parts if p.num_seqs > 0]
        alg = [algorithmic(p) for p in self.parts]
        self.step_bytes = sum(a["bytes"] for a in alg)
        if append:
            # k_new and v_new read once, and the same rows written to the cache.
            self.step_bytes += 2 * 2 * batch.total_q * batch.num_kv_heads * batch.head_dim * (
                2 if batch.dtype == "bf16" else 4)
        self.step_flops = sum(a["flops"] for a in alg)
        self.tokens = sum(p.total_q for p in self.parts)
        self.replicas = replicas or max(2, math.ceil(2 * MALL_BYTES / self.step_bytes) + 1)
        self.stream = torch.cuda.current_stream()
        self.launch_stream = torch.cuda.Stream() if graph else self.stream
        self.kernel_srcs = {DEVICE_HELPERS_SRC}
        self.splits_used = []
        calls, self.keep = [], []
        for r in range(self.replicas):
            rc = []
            for p in self.parts:
                q = p.q.to(dev)
                k, v = p.k_cache.to(dev), p.v_cache.to(dev)
                rel = p.rel_logits.to(dev)
                bt = torch.from_numpy(p.block_table).to(dev)
                sl = torch.from_numpy(p.seq_lens).to(dev)
                out = torch.empty_like(q)
                if p.is_decode() and name != "global_mixed":
                    d = binding.dims_for(q, k, bt, rel, num_seqs=p.num_seqs, max_q_len=1,
                                         max_seq_len=p.max_seq_len)
                    s = splits or binding.num_splits(d, p.window, 0)
                    need = binding.decode_workspace_bytes(d, p.window, s)
                    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
                    a, dims = binding.decode_args(q, k, v, bt, sl, rel, p.window, p.scale, out,
                                                  max_seq_len=p.max_seq_len, num_splits=s,
                                                  workspace=ws, stream=self.launch_stream)
                    if append:
                        # The new token's rows are the ones already at key L - 1.
                        kn = torch.stack([p.k_logical[i][int(p.seq_lens[i]) - 1]
                                          for i in range(p.num_seqs)]).to(dev)
                        vn = torch.stack([p.v_logical[i][int(p.seq_lens[i]) - 1]
                                          for i in range(p.num_seqs)]).to(dev)
                        a = a[:1] + (binding._ptr(kn), binding._ptr(vn)) + a[1:]
                        self.keep += [kn, vn]
                    rc.append(("inkling_rel_attn_decode_append" if append
                               else "inkling_rel_attn_decode", a))
                    self.keep += [q, k, v, rel, bt, sl, out, ws, dims]
                    self.kernel_srcs.add(DECODE_KERNEL_SRC)
                    if r == 0:
                        self.splits_used.append(s)
                else:
                    cu = torch.from_numpy(p.cu_q_lens).to(dev)
                    a, dims = binding.prefill_args(q, k, v, bt, sl, cu, rel, p.window, p.scale,
                                                   out, max_q_len=p.max_q_len,
                                                   max_seq_len=p.max_seq_len,
                                                   stream=self.launch_stream)
                    if append:
                        rows = [(i, pos) for i in range(p.num_seqs)
                                for pos in range(int(p.seq_lens[i]) - int(p.q_lens[i]),
                                                 int(p.seq_lens[i]))]
                        kn = torch.stack([p.k_logical[i][pos] for i, pos in rows]).to(dev)
                        vn = torch.stack([p.v_logical[i][pos] for i, pos in rows]).to(dev)
                        a = a[:1] + (binding._ptr(kn), binding._ptr(vn)) + a[1:]
                        self.keep += [kn, vn]
                    rc.append(("inkling_rel_attn_prefill_append" if append
                               else "inkling_rel_attn_prefill", a))
                    self.keep += [q, k, v, rel, bt, sl, cu, out, dims]
                    fast = p.dtype == "bf16" and p.head_dim == 128 and not append
                    self.kernel_srcs.add(PREFILL_BF16_KERNEL_SRC if fast else PREFILL_KERNEL_SRC)
            calls.append(rc)
        torch.cuda.synchronize()
        lib = binding.load()
        self.fns = [[(getattr(lib, n), a) for n, a in rc] for rc in calls]
        self.step = self._eager
        if graph:
            # One eager run per replica on the capture stream (kernel
            # attributes are set on first use), then one capture per replica.
            with torch.cuda.stream(self.launch_stream):
                for r in range(self.replicas):
                    self._eager(r)
            self.launch_stream.synchronize()
            self.graphs = []
            for r in range(self.replicas):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=self.launch_stream):
                    self._eager(r)
                self.graphs.append(g)
            torch.cuda.synchronize()
            self.step = lambda i: self.graphs[i % self.replicas].replay()

    def _eager(self, i):
        from paged_relative_bias_amd import binding
        for fn, a in self.fns[i % self.replicas]:
            st = fn(*a)
            if st != 0:
                raise binding.InklingError(st, "step")

    def time(self, steps, warmup, settle_ms=0.0):
        import torch
        # Settle: a short probe estimates the step time, then enough
        # back-to-back steps to cover settle_ms of GPU time, with no
        # synchronisation between them.
        n0 = 0
        if settle_ms > 0:
            for i in range(4):
                self.step(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(8):
                self.step(i)
            torch.cuda.synchronize()
            est_ms = max((time.perf_counter() - t0) * 1e3 / 8, 1e-3)
            n0 = int(min(20000, math.ceil(settle_ms / est_ms)))
            for i in range(n0):
                self.step(i)
        for i in range(warmup):
            self.step(n0 + i)
        torch.cuda.synchronize()
        # Timed region: K back-to-back steps, HIP events on the launch stream
        # at its two ends only (an event between launches adds its own gap).
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(steps):
            self.step(warmup + i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        mean_ms = e0.elapsed_time(e1) / steps
        # Per-step durations, from a separate pass with an event pair per step.
        n = max(50, min(steps, 200))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (a, b) in enumerate(ev):
            a.record(self.stream)
            self.step(i)
            b.record(self.stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in ev])
        return {"ms_per_step": 1e3 * wall / steps, "mean_ms": mean_ms,
                "median_ms": float(np.median(per)), "p10_ms": float(np.percentile(per, 10)),
                "p90_ms": float(np.percentile(per, 90)), "per_step_n": n}


def record_for(name, batch, wl, t, record_name, cpu):
    # The launch duration is the mean over the timed region's back-to-back
    # launches (HIP events on the launch stream at its two ends).
    mean = t["mean_ms"]
    median = t["median_ms"]
    achieved = wl.step_bytes / (mean * 1e-3) / 1e9
    tflops = wl.step_flops / (mean * 1e-3) / 1e12
    peak_tf = BF16_PEAK_TFLOPS if batch.dtype == "bf16" else FP32_PEAK_TFLOPS
    # A graph-replayed record runs the same kernels as its eager form.
    traffic = traffic_from_profiles(record_name.removesuffix("_graph"), sorted(wl.kernel_srcs))
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": wl.step_bytes,
            "algorithmic_flops_per_launch": wl.step_flops,
            "launch_ms_median": round(median, 5),
            "launch_ms_p10": round(t["p10_ms"], 5),
            "launch_ms_p90": round(t["p90_ms"], 5),
            "launch_ms_mean_back_to_back": round(t["mean_ms"], 5),
            "launch_note": ("achieved and frac from the mean launch time of the timed region; "
                            f"median, p10 and p90 from a later pass of {t['per_step_n']} "
                            "per-step event pairs"),
            "mfma_tflops": round(tflops, 2),
            "mfma_peak_tflops": peak_tf,
            "mfma_frac": round(tflops / peak_tf, 4)}
    if traffic:
        roof["traffic_over_algorithmic"] = round(traffic / wl.step_bytes, 3)
    # The binding roofline is the one the launch comes closer to: HBM for
    # decode and short-context prefill, the bf16 MFMA peak for long-context
    # prefill.  The HBM figures stay in hbm_gbs / hbm_frac either way.
    roof["hbm_gbs"], roof["hbm_frac"] = roof["achieved"], roof["frac"]
    if roof["mfma_frac"] > roof["frac"]:
        roof.update({"bound": "mfma", "achieved": roof["mfma_tflops"], "peak": peak_tf,
                     "unit": "TFLOP/s", "frac": roof["mfma_frac"]})
    cfg = {"workload": name, "num_seqs": int(batch.num_seqs), "total_q": int(batch.total_q),
           "num_q_heads": batch.num_q_heads, "num_kv_heads": batch.num_kv_heads,
           "head_dim": batch.head_dim, "window": batch.window, "rel_len": batch.rel_len,
           "block_size": batch.block_size, "seq_lens_sum": int(batch.seq_lens.sum()),
           "max_seq_len": int(batch.max_seq_len), "num_splits": wl.splits_used or None,
           "replicas": wl.replicas}
    return {"value": round(wl.tokens / (t["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(t["ms_per_step"], 5), "dtype": batch.dtype,
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def make_batch_for(gen_name, args, seed):
    from paged_relative_bias_amd import inputs

    t0 = time.perf_counter()
    gen = inputs.WORKLOADS[gen_name]
    batch = gen(seed=seed, batch=args.batch) if args.batch else gen(seed=seed)
    if args.spike:
        batch = spike_bias(batch)
    log(f"generated {gen_name} in {time.perf_counter() - t0:.1f}s: B={batch.num_seqs} "
        f"total_q={batch.total_q} Hq={batch.num_q_heads} Hkv={batch.num_kv_heads} "
        f"D={batch.head_dim} W={batch.window} R={batch.rel_len}")
    return batch


def run_record(record_name, batch, splits, args, dev, steps, warmup, cpu, graph=None):
    """Time one record on an already generated batch (graph: replay HIP graphs
    of the step; None follows --graph)."""
    import torch

    graph = args.graph if graph is None else graph
    kind = "global_mixed_split" if record_name == "global_mixed_split" else batch.name
    wl = Workload(kind, batch, splits=splits, append=args.append, graph=graph,
                  replicas=args.replicas, dev=dev)
    t = wl.time(steps, warmup, args.settle_ms)
    rec = record_for(kind, batch, wl, t, record_name, cpu)
    rec["config"]["settle_ms"] = args.settle_ms
    rec["config"]["seed"] = args.seed
    rec["config"]["launch"] = "hip_graph" if graph else "eager"
    rec["config"]["append"] = bool(args.append)
    rec["config"]["bias_spike"] = bool(args.spike)
    r = rec["roofline"]
    log(f"{record_name}: {t['ms_per_step'] * 1e3:.1f} us/step wall; launch median "
        f"{r['launch_ms_median'] * 1e3:.1f} us (p10 {r['launch_ms_p10'] * 1e3:.1f}, p90 "
        f"{r['launch_ms_p90'] * 1e3:.1f}, back-to-back mean "
        f"{r['launch_ms_mean_back_to_back'] * 1e3:.1f}); {r['hbm_gbs']:.0f} GB/s = "
        f"{100 * r['hbm_frac']:.1f}% HBM; {r['mfma_tflops']:.1f} TFLOP/s = "
        f"{100 * r['mfma_frac']:.2f}% MFMA; {rec['value'] / 1e6:.3f} M tokens/s; "
        f"splits={wl.splits_used} replicas={wl.replicas}")
    del wl
    gc.collect()
    torch.cuda.empty_cache()
    return rec


def baseline(batch, args, budget):
    if args.no_cpu_baseline:
        return None
    cpu = cpu_baseline(batch, budget)
    log(f"  cpu baseline ({batch.name}): {cpu}")
    return cpu


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Prefill launches (~0.7 ms) need about 20 ms of back-to-back work before
    # their duration settles; 50 untimed steps cover that for every workload.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="back-to-back steps covering this much GPU time before the warm-up steps")
    ap.add_argument("--workload", default=None, choices=WORKLOAD_CHOICES,
                    help="time only this workload (default: the headline and every other)")
    ap.add_argument("--headline-only", action="store_true",
                    help="without --workload: skip the other workloads' records")
    ap.add_argument("--splits", type=int, default=0, help="decode num_splits (0 = library)")
    ap.add_argument("--replicas", type=int, default=0, help="input copies rotated (0 = auto)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences in a decode workload (0 = the workload's own)")
    ap.add_argument("--append", action="store_true",
                    help="the *_append entry points: the step's new K/V rows are stored "
                         "into the cache in the same launch")
    ap.add_argument("--graph", action="store_true",
                    help="capture each replica's step once in a HIP graph and time replays")
    ap.add_argument("--spike", action="store_true",
                    help="+60 on every row's distance-0 bias entry (forces the second pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work for the headline's CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(attention shards by KV head with no exchange between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_relative_bias_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    st, msg = binding.check_device(0)
    if st != binding.OK:
        print(msg, file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        # A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # counters calibrate the counter units, and its rate is the
        # practical streaming bandwidth of the box.
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = 2 * nbytes / (ms * 1e-3) / 1e9
        log(f"copy 1 GiB: {ms * 1e3:.1f} us, {gbs:.0f} GB/s read+write")
        print(json.dumps({"copy_bytes": nbytes, "launches": 3 + reps, "copy_us": round(ms * 1e3, 2),
                          "copy_read_plus_write_gbs": round(gbs, 1)}))
        return

    if args.batch and args.workload and not args.workload.endswith("decode"):
        log("--batch applies to the decode workloads only")
        sys.exit(2)
    head_name = args.workload or HEADLINE
    gen_name = "global_mixed" if head_name == "global_mixed_split" else head_name
    batch = make_batch_for(gen_name, args, args.seed)
    cpu = baseline(batch, args, args.cpu_budget)
    rec = run_record(head_name, batch, args.splits, args, dev, args.steps, args.warmup, cpu)
    line = {"metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": rec["dtype"], "data": "synthetic (seeded N(0,1), shuffled page pool)",
            "config": rec["config"], "roofline": rec["roofline"],
            "cpu_baseline": rec["cpu_baseline"]}
    del batch
    gc.collect()
    if args.workload is None and not args.headline_only:
        # Every other configuration: at most 100 timed steps each and a
        # shorter oracle sample; one generated batch serves all its records.
        others = {}
        for gname, recs in SECONDARY:
            try:
                b = make_batch_for(gname, args, args.seed)
                cpu = baseline(b, args, min(args.cpu_budget, 10.0))
                for rname, splits, *graph in recs:
                    others[rname] = run_record(rname, b, splits, args, dev,
                                               min(args.steps, 100), args.warmup, cpu,
                                               graph=graph[0] if graph else None)
                del b
            except Exception as e:  # keep the headline and the other records
                log(f"{gname}: failed: {e!r}")
                for rname, *_ in recs:
                    others.setdefault(rname, {"error": repr(e)})
            gc.collect()
        line["workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
