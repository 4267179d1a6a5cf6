#!/usr/bin/env python3
"""Throughput of relative-bias paged attention on one MI355X (gfx950).

One step is one call of the library's hot path on one synthetic batch, with
its inputs already resident in HBM:
  * decode workloads: inkling_rel_attn_decode (split-KV decode kernel, plus
    the log-sum-exp merge kernel when it uses more than one split);
  * prefill workloads: inkling_rel_attn_prefill.
The default workload is the local-layer decode batch (64 sequences, contexts
U[1024, 8192], 48 query / 16 KV heads, head_dim 128, window 512, bf16).

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize(); HIP events on the launch stream around every step
give the per-launch duration used for the roofline.  Consecutive steps read
different device copies of the inputs (replicas rotated round-robin, at
least 512 MB apart) so no step finds its data in the 256 MB Infinity Cache
left behind by the previous one, as in a real forward where consecutive
attention calls belong to different layers.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
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
PROFILES = os.path.join(ROOT, "profiles")


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
    kv = bias = pages = 0
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


def traffic_from_profiles(workload, kernel_src, launches_per_step=1):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if
    they were taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != source_hash(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(batch, budget_s=20.0):
    """The fp64 oracle as it stands, on the host cores, over the whole batch
    (decode) or over a bounded, seeded subset of (row, head) pairs (prefill),
    scaled to query tokens per second."""
    import oracle

    threads = oracle.max_threads()
    Hq = batch.num_q_heads
    total_rows = batch.total_q * Hq
    if batch.is_decode():
        rows = None
        sample = f"whole batch: {batch.num_seqs} sequences x {Hq} heads"
        frac = 1.0
    else:
        # Size the subset from a quick probe so the run takes ~budget_s.
        rng = np.random.default_rng(0)
        probe = rng.choice(total_rows, size=min(256, total_rows), replace=False)
        t0 = time.perf_counter()
        oracle.run_batch(batch, rows=probe)
        per_row = (time.perf_counter() - t0) / len(probe)
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
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds_per_run": round(dt, 4),
            "runs": runs}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Prefill launches (~0.7 ms) need about 20 ms of back-to-back work before
    # their duration settles; 50 untimed steps cover that for every workload.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="local_decode",
                    choices=["local_decode", "global_decode", "local_prefill",
                             "global_mixed", "global_mixed_split", "tiny_prefill",
                             "long_global_decode"])
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(attention shards by head with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_relative_bias_amd import binding, inputs

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

    wl = args.workload
    split_mixed = wl == "global_mixed_split"
    gen = inputs.WORKLOADS["global_mixed" if split_mixed else wl]
    t0 = time.perf_counter()
    if args.batch and not wl.endswith("decode"):
        log("--batch applies to the decode workloads only")
        sys.exit(2)
    batch = gen(seed=args.seed, batch=args.batch) if args.batch else gen(seed=args.seed)
    log(f"generated {batch.name} in {time.perf_counter() - t0:.1f}s: B={batch.num_seqs} "
        f"total_q={batch.total_q} Hq={batch.num_q_heads} Hkv={batch.num_kv_heads} "
        f"D={batch.head_dim} W={batch.window} R={batch.rel_len}")
    parts = list(inputs.split_mixed(batch)) if split_mixed else [batch]
    parts = [p for p in parts if p.num_seqs > 0]
    alg = [algorithmic(p) for p in parts]
    step_bytes = sum(a["bytes"] for a in alg)
    if args.append:
        # k_new and v_new read once, and the same rows written to the cache.
        step_bytes += 2 * 2 * batch.total_q * batch.num_kv_heads * batch.head_dim * (
            2 if batch.dtype == "bf16" else 4)
    step_flops = sum(a["flops"] for a in alg)
    replicas = args.replicas or max(2, math.ceil(2 * MALL_BYTES / step_bytes) + 1)

    # With --graph the calls are issued on a side stream that is captured;
    # the replays then run on the current stream.
    stream = torch.cuda.current_stream()
    launch_stream = torch.cuda.Stream() if args.graph else stream
    calls = []       # per replica: list of (fn_name, args)
    keep = []        # tensors and dims that must stay alive
    splits_used = []
    for r in range(replicas):
        rc = []
        for p in parts:
            q = p.q.to(dev)
            k, v = p.k_cache.to(dev), p.v_cache.to(dev)
            rel = p.rel_logits.to(dev)
            bt = torch.from_numpy(p.block_table).to(dev)
            sl = torch.from_numpy(p.seq_lens).to(dev)
            out = torch.empty_like(q)
            if p.is_decode() and wl != "global_mixed":
                d = binding.dims_for(q, k, bt, rel, num_seqs=p.num_seqs, max_q_len=1,
                                     max_seq_len=p.max_seq_len)
                s = args.splits or binding.num_splits(d, p.window, 0)
                need = binding.decode_workspace_bytes(d, p.window, s)
                ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
                a, dims = binding.decode_args(q, k, v, bt, sl, rel, p.window, p.scale, out,
                                              max_seq_len=p.max_seq_len, num_splits=s,
                                              workspace=ws, stream=launch_stream)
                if args.append:
                    # The new token's rows are the ones already at key L - 1.
                    kn = torch.stack([p.k_logical[i][int(p.seq_lens[i]) - 1]
                                      for i in range(p.num_seqs)]).to(dev)
                    vn = torch.stack([p.v_logical[i][int(p.seq_lens[i]) - 1]
                                      for i in range(p.num_seqs)]).to(dev)
                    a = a[:1] + (binding._ptr(kn), binding._ptr(vn)) + a[1:]
                    keep += [kn, vn]
                rc.append(("inkling_rel_attn_decode_append" if args.append
                           else "inkling_rel_attn_decode", a))
                keep += [q, k, v, rel, bt, sl, out, ws, dims]
                if r == 0:
                    splits_used.append(s)
            else:
                cu = torch.from_numpy(p.cu_q_lens).to(dev)
                a, dims = binding.prefill_args(q, k, v, bt, sl, cu, rel, p.window, p.scale,
                                               out, max_q_len=p.max_q_len,
                                               max_seq_len=p.max_seq_len, stream=launch_stream)
                if args.append:
                    # The new tokens' rows are the ones already at their keys.
                    rows = [(i, pos) for i in range(p.num_seqs)
                            for pos in range(int(p.seq_lens[i]) - int(p.q_lens[i]),
                                             int(p.seq_lens[i]))]
                    kn = torch.stack([p.k_logical[i][pos] for i, pos in rows]).to(dev)
                    vn = torch.stack([p.v_logical[i][pos] for i, pos in rows]).to(dev)
                    a = a[:1] + (binding._ptr(kn), binding._ptr(vn)) + a[1:]
                    keep += [kn, vn]
                rc.append(("inkling_rel_attn_prefill_append" if args.append
                           else "inkling_rel_attn_prefill", a))
                keep += [q, k, v, rel, bt, sl, cu, out, dims]
        calls.append(rc)
    torch.cuda.synchronize()
    lib = binding.load()
    fns = [[(getattr(lib, name), a) for name, a in rc] for rc in calls]

    def eager_step(i):
        for fn, a in fns[i % replicas]:
            st = fn(*a)
            if st != 0:
                raise binding.InklingError(st, "step")

    step = eager_step
    if args.graph:
        # One eager run per replica on the capture stream (kernel attributes
        # are set on first use), then one capture per replica.
        with torch.cuda.stream(launch_stream):
            for r in range(replicas):
                eager_step(r)
        launch_stream.synchronize()
        graphs = []
        for r in range(replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=launch_stream):
                eager_step(r)
            graphs.append(g)
        torch.cuda.synchronize()

        def step(i):
            graphs[i % replicas].replay()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K back-to-back steps, HIP events on the launch stream at
    # its two ends only (an event between launches would add its own gap).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    # Mean launch duration over the timed region (includes the short gaps
    # between back-to-back launches, so it never flatters the kernel).
    launch_ms = e0.elapsed_time(e1) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    # Spread, from a separate untimed pass with an event pair per step.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 50))]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in ev])  # ms
    tokens = sum(p.total_q for p in parts)
    value = tokens / (ms_per_step * 1e-3)

    achieved = step_bytes / (launch_ms * 1e-3) / 1e9
    tflops = step_flops / (launch_ms * 1e-3) / 1e12
    kernel_src = (DECODE_KERNEL_SRC if wl in ("local_decode", "global_decode", "long_global_decode")
                  else PREFILL_KERNEL_SRC)
    traffic = traffic_from_profiles(wl, kernel_src)
    peak_tf = BF16_PEAK_TFLOPS if batch.dtype == "bf16" else FP32_PEAK_TFLOPS
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": step_bytes,
            "launch_ms_mean": round(launch_ms, 5),
            "launch_ms_p10": round(float(np.percentile(per, 10)), 5),
            "launch_ms_p90": round(float(np.percentile(per, 90)), 5),
            "launch_note": "mean over the timed region; p10/p90 from a separate per-step pass",
            "mfma_tflops": round(tflops, 2),
            "mfma_frac": round(tflops / peak_tf, 4)}
    log(f"{wl}: {ms_per_step * 1e3:.1f} us/step wall, {launch_ms * 1e3:.1f} us/launch "
        f"(p10 {roof['launch_ms_p10'] * 1e3:.1f}, p90 {roof['launch_ms_p90'] * 1e3:.1f}); "
        f"{achieved:.0f} GB/s = {100 * achieved / HBM_PEAK_GBS:.1f}% HBM; "
        f"{tflops:.1f} TFLOP/s = {100 * tflops / peak_tf:.2f}% MFMA; "
        f"{value / 1e6:.3f} M tokens/s; replicas={replicas} splits={splits_used}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(batch)
        log(f"cpu baseline: {cpu}")

    cfg = {"workload": wl, "num_seqs": int(batch.num_seqs), "total_q": int(batch.total_q),
           "num_q_heads": batch.num_q_heads, "num_kv_heads": batch.num_kv_heads,
           "head_dim": batch.head_dim, "window": batch.window, "rel_len": batch.rel_len,
           "block_size": batch.block_size, "seq_lens_sum": int(batch.seq_lens.sum()),
           "max_seq_len": int(batch.max_seq_len), "num_splits": splits_used or None,
           "replicas": replicas, "seed": args.seed, "launch": "hip_graph" if args.graph else "eager",
           "append": bool(args.append)}
    rec = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": batch.dtype, "data": "synthetic (seeded N(0,1), shuffled page pool)",
           "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
