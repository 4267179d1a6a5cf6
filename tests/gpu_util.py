"""Helpers for the GPU parity tests: move a batch to the device, call the
library through its C ABI binding, compare with the oracle."""
import numpy as np
import torch

import oracle
from paged_relative_bias_amd import binding

# Tolerances.  bf16: the stated bar, max-abs 1e-2 and mean-abs 1e-3 against
# the unrounded fp64 oracle.  Where |ref| >= 4 the spacing of bf16 values is
# at least 1/32, so the correctly rounded result alone can sit up to 1/64 >
# 1e-2 away.  There the per-element bar is half a bf16 ulp of |ref| (the
# rounding of the output) plus COMPUTE_SLACK, the share of the 1e-2 bar that
# is left for arithmetic error where |ref| is in [2, 4) (1e-2 minus half an
# ulp there, 2^-7 = 0.0078).  Every element that passes only through this
# relaxed bar is counted and reported.  The mean-abs bar covers every element.
# fp32: every step is fp32 (fp32 MFMA, fp32 P), so errors are ~1e-6; 1e-4
# leaves two orders of margin.
TOL = {"bf16": (1e-2, 1e-3), "fp32": (1e-4, 1e-5)}
BF16_RELAXED_FROM = 4.0
COMPUTE_SLACK = 2.2e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.exp2(e - 7)


def bf16_bar(ref: np.ndarray) -> np.ndarray:
    """Per-element max-abs bar for bf16 outputs (see TOL above)."""
    bar = np.full(ref.shape, TOL["bf16"][0])
    big = np.abs(ref) >= BF16_RELAXED_FROM
    bar[big] = 0.5 * bf16_ulp(ref[big]) + COMPUTE_SLACK
    return bar


class Dev:
    """Device copies of a batch's tensors."""

    def __init__(self, batch, device="cuda"):
        self.batch = batch
        self.q = batch.q.to(device)
        self.k = batch.k_cache.to(device)
        self.v = batch.v_cache.to(device)
        self.rel = batch.rel_logits.to(device)
        self.bt = torch.from_numpy(batch.block_table).to(device)
        self.sl = torch.from_numpy(batch.seq_lens).to(device)
        self.cu = torch.from_numpy(batch.cu_q_lens).to(device)


def prefill(dev: Dev, out=None, stream=None):
    b = dev.batch
    if out is None:
        out = torch.full_like(dev.q, float("nan"))
    binding.prefill(dev.q, dev.k, dev.v, dev.bt, dev.sl, dev.cu, dev.rel,
                    b.window, b.scale, out, max_q_len=b.max_q_len,
                    max_seq_len=b.max_seq_len, stream=stream)
    return out


def decode(dev: Dev, splits=0, out=None, workspace=None, stream=None):
    b = dev.batch
    if out is None:
        out = torch.full_like(dev.q, float("nan"))
    binding.decode(dev.q, dev.k, dev.v, dev.bt, dev.sl, dev.rel, b.window,
                   b.scale, out, max_seq_len=b.max_seq_len, num_splits=splits,
                   workspace=workspace, stream=stream)
    return out


def compare(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "",
            rows=None):
    """Element-wise check against the oracle; returns (max_abs, mean_abs,
    n_relaxed), n_relaxed being the elements above 1e-2 that pass only
    through the bar for |ref| >= 4."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g.reshape(-1, g.shape[-1])[rows]
    ref = ref.reshape(g.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    mx, mean = float(err.max()), float(err.mean())
    tol_max, tol_mean = TOL[dtype]
    if dtype == "bf16":
        bar = bf16_bar(ref)
    else:
        bar = np.full(err.shape, tol_max)
    relaxed = err > tol_max
    n_relaxed = int(relaxed.sum())
    worst_rel = ""
    if n_relaxed:
        k = np.unravel_index(np.where(relaxed, err, -1.0).argmax(), err.shape)
        worst_rel = f" worst_relaxed: err={err[k]:.3e} ref={ref[k]:.4f} bar={bar[k]:.3e}"
    n_big = int((np.abs(ref) >= BF16_RELAXED_FROM).sum()) if dtype == "bf16" else 0
    print(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} n={err.size} "
          f"n_|ref|>=4={n_big} n_over_1e-2={n_relaxed}{worst_rel}", flush=True)
    worst = np.unravel_index((err - bar).argmax(), err.shape)
    assert np.all(err <= bar) and mean <= tol_mean, (
        f"{what}: max_abs {mx:.3e} (bar {tol_max}; half an ulp + {COMPUTE_SLACK} where "
        f"|ref|>=4) mean_abs {mean:.3e} (tol {tol_mean}); worst at {worst}: "
        f"got {g[worst]} ref {ref[worst]}")
    # Only elements with |ref| >= 4 may exceed 1e-2.
    assert n_relaxed <= n_big
    return mx, mean, n_relaxed


def sample_rows(batch, n_random: int, seed: int = 0, first_positions: int = 3):
    """Flat (row * Hq + h) indices: a seeded random subset plus every head of
    the first `first_positions` positions of each sequence (where few keys
    make bf16 rounding matter most)."""
    rng = np.random.default_rng(seed)
    Hq = batch.num_q_heads
    total = batch.total_q * Hq
    pick = set(rng.choice(total, size=min(n_random, total), replace=False).tolist())
    for s in range(batch.num_seqs):
        n, L = int(batch.q_lens[s]), int(batch.seq_lens[s])
        for t in range(n):
            if L - n + t < first_positions:
                r = int(batch.cu_q_lens[s]) + t
                pick.update(range(r * Hq, (r + 1) * Hq))
    return np.array(sorted(pick), dtype=np.int64)


def oracle_rows(batch, rows, threads=0):
    out, _ = oracle.run_batch(batch, rows=rows, threads=threads)
    return out
