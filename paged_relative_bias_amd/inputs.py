"""Seeded synthetic inputs for paged relative-bias attention.

This module only *creates* inputs: sequence lengths, a shuffled page pool, the
block table and N(0,1) tensors.  It holds none of the attention arithmetic, so
both sides of a parity check (the fp64 oracle and the HIP library) may read
what it returns.

Shapes follow the serving setup described on the TensorRT-LLM Inkling page
(section "Architecture": local layers with window 512 and 16 KV heads, global
full-causal layers with 8 KV heads; hidden size 6144 there and in the ONESHOT
all-reduce note) and the 8-GPU H200 gist (max model length 8192 in its run
command).  48 query heads of dimension 128 give the hidden size 6144.

Generation recipe (fixed, so every machine draws the same values):
  * ``numpy.random.default_rng(seed)``;
  * draw order: lengths, page permutation, q, k, v, rel_logits;
  * values are float32 N(0,1), cast round-to-nearest-even to the batch dtype;
  * the pool holds ``sum(ceil(L_b / block_size))`` used pages plus ``spare``
    unreferenced pages; physical page ids are a random permutation;
  * block-table rows are padded with -1;
  * with ``poison=True`` every byte the method must never read is NaN:
    unreferenced pages, the slots past ``L_b`` in each sequence's last page,
    every ``rel_logits`` entry no visible (query, key) pair indexes and
    (with a window, unless ``poison_stale=False``) the K/V rows of keys older
    than the window of every query of the sequence.  The NaN values replace
    drawn ones after all draws, so they never shift the random stream.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BLOCK_SIZE = 16


@dataclasses.dataclass
class Batch:
    """One call's worth of inputs, on the host (torch CPU tensors)."""

    dtype: str                  # "bf16" or "fp32"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    window: int                 # > 0 sliding window; <= 0 full causal
    scale: float
    seq_lens: np.ndarray        # int32 [B]  KV length including new tokens
    q_lens: np.ndarray          # int32 [B]  new tokens per sequence
    cu_q_lens: np.ndarray       # int32 [B+1]
    q: torch.Tensor             # [total_q, Hq, D]
    k_cache: torch.Tensor       # [num_blocks, block_size, Hkv, D]
    v_cache: torch.Tensor       # [num_blocks, block_size, Hkv, D]
    block_table: np.ndarray     # int32 [B, max_blocks_per_seq], -1 padded
    rel_logits: torch.Tensor    # [total_q, Hq, R]
    k_logical: list             # per sequence [L_b, Hkv, D] (same dtype)
    v_logical: list
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    @property
    def rel_len(self) -> int:
        return int(self.rel_logits.shape[-1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def make_batch(rng: np.random.Generator, seq_lens, q_lens, *, num_q_heads: int,
               num_kv_heads: int, head_dim: int, window: int, rel_len: int,
               dtype: str = "bf16", block_size: int = BLOCK_SIZE,
               max_blocks_per_seq: int | None = None, spare_pages: int = 64,
               poison: bool = True, scale: float | None = None,
               name: str = "", poison_stale: bool = True) -> Batch:
    """Lay out one batch given its lengths; draws pages, q, k, v, rel in order."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(-1)
    q_lens = np.asarray(q_lens, dtype=np.int32).reshape(-1)
    assert seq_lens.shape == q_lens.shape
    assert np.all(q_lens >= 0) and np.all(seq_lens >= q_lens)
    B = seq_lens.shape[0]
    Hq, Hkv, D, bs = num_q_heads, num_kv_heads, head_dim, block_size
    pages_per_seq = [(int(L) + bs - 1) // bs for L in seq_lens]
    used_pages = int(sum(pages_per_seq))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max([1] + pages_per_seq)
    assert max_blocks_per_seq >= max([0] + pages_per_seq)
    num_blocks = used_pages + spare_pages

    # 2. page permutation: logical page k of sequence b -> physical id
    perm = rng.permutation(num_blocks).astype(np.int32)
    block_table = np.full((B, max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        n = pages_per_seq[b]
        block_table[b, :n] = perm[pos:pos + n]
        pos += n

    cu_q_lens = np.zeros(B + 1, dtype=np.int32)
    cu_q_lens[1:] = np.cumsum(q_lens)
    total_q = int(cu_q_lens[-1])
    total_kv = int(seq_lens.sum())

    # 3-6. tensors, in the fixed order
    q = _normal(rng, (total_q, Hq, D), dtype)
    k_all = _normal(rng, (total_kv, Hkv, D), dtype)
    v_all = _normal(rng, (total_kv, Hkv, D), dtype)
    rel = _normal(rng, (total_q, Hq, rel_len), dtype)

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    fill = float("nan") if poison else 0.0
    k_cache = torch.full((num_blocks, bs, Hkv, D), fill, dtype=tdt)
    v_cache = torch.full((num_blocks, bs, Hkv, D), fill, dtype=tdt)
    k_logical, v_logical = [], []
    off = 0
    for b in range(B):
        L = int(seq_lens[b])
        kb = k_all[off:off + L]
        vb = v_all[off:off + L]
        off += L
        k_logical.append(kb)
        v_logical.append(vb)
        n = pages_per_seq[b]
        if n == 0:
            continue
        if poison and poison_stale and window > 0 and int(q_lens[b]) > 0:
            # Keys before the window of the sequence's earliest query.
            stale = max(0, L - int(q_lens[b]) - int(window) + 1)
            if stale:
                kb = kb.clone()
                vb = vb.clone()
                kb[:stale] = float("nan")
                vb[:stale] = float("nan")
        pad = n * bs - L
        if pad:
            kb = torch.cat([kb, torch.full((pad, Hkv, D), fill, dtype=tdt)])
            vb = torch.cat([vb, torch.full((pad, Hkv, D), fill, dtype=tdt)])
        ids = torch.from_numpy(block_table[b, :n].astype(np.int64))
        k_cache[ids] = kb.reshape(n, bs, Hkv, D)
        v_cache[ids] = vb.reshape(n, bs, Hkv, D)

    if poison:
        _poison_unused_bias(rel, seq_lens, q_lens, cu_q_lens, window)

    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Batch(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                 block_size=bs, window=int(window), scale=float(scale),
                 seq_lens=seq_lens, q_lens=q_lens, cu_q_lens=cu_q_lens, q=q,
                 k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                 rel_logits=rel, k_logical=k_logical, v_logical=v_logical,
                 name=name)


def _poison_unused_bias(rel: torch.Tensor, seq_lens, q_lens, cu_q_lens, window):
    """NaN every rel_logits entry that no visible (query, key) pair indexes.

    A query at position p sees distances 0..p (and, with a window W > 0, only
    those below W); distance d reads entry min(d, R-1).  So the entries in use
    are 0..min(p, W-1, R-1) and the rest are never read.
    """
    R = rel.shape[-1]
    idx = torch.arange(R)
    for b in range(len(seq_lens)):
        n = int(q_lens[b])
        if n == 0:
            continue
        L = int(seq_lens[b])
        p = torch.arange(L - n, L)
        lim = p.clone()
        if window > 0:
            lim = torch.clamp(lim, max=window - 1)
        lim = torch.clamp(lim, max=R - 1)
        dead = idx[None, :] > lim[:, None]            # [n, R]
        i0 = int(cu_q_lens[b])
        blk = rel[i0:i0 + n]
        blk.masked_fill_(dead[:, None, :], float("nan"))


# ---------------------------------------------------------------------------
# Named workloads (the serving shapes); each draws lengths first.
# ---------------------------------------------------------------------------
HQ, HKV_LOCAL, HKV_GLOBAL, HEAD_DIM, WINDOW_LOCAL = 48, 16, 8, 128, 512
MAX_CONTEXT = 8192
MAX_BLOCKS = MAX_CONTEXT // BLOCK_SIZE


def tiny(seed: int = 0, poison: bool = True) -> Batch:
    """1 sequence of 64 tokens, Hq=4, Hkv=2, D=64, window 32, R=32, fp32."""
    rng = np.random.default_rng(seed)
    return make_batch(rng, [64], [64], num_q_heads=4, num_kv_heads=2,
                      head_dim=64, window=32, rel_len=32, dtype="fp32",
                      spare_pages=4, poison=poison, name="tiny_prefill")


def local_decode(seed: int = 0, batch: int = 64, lo: int = 1024,
                 hi: int = 8192, poison: bool = True) -> Batch:
    """64 sequences, contexts U[1024, 8192], Hq=48, Hkv=16, W=512, R=512."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi + 1, size=batch)
    return make_batch(rng, L, np.ones_like(L), num_q_heads=HQ,
                      num_kv_heads=HKV_LOCAL, head_dim=HEAD_DIM,
                      window=WINDOW_LOCAL, rel_len=WINDOW_LOCAL,
                      max_blocks_per_seq=MAX_BLOCKS, poison=poison,
                      name="local_decode")


def global_decode(seed: int = 0, batch: int = 32, lo: int = 4096,
                  hi: int = 8192, poison: bool = True) -> Batch:
    """32 sequences, contexts U[4096, 8192], Hq=48, Hkv=8, full causal, R=8192."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi + 1, size=batch)
    return make_batch(rng, L, np.ones_like(L), num_q_heads=HQ,
                      num_kv_heads=HKV_GLOBAL, head_dim=HEAD_DIM, window=0,
                      rel_len=MAX_CONTEXT, max_blocks_per_seq=MAX_BLOCKS,
                      poison=poison, name="global_decode")


def local_prefill(seed: int = 0, batch: int = 8, lo: int = 2048,
                  hi: int = 4096, poison: bool = True) -> Batch:
    """8 sequences from an empty cache, lengths U[2048, 4096], W=512, Hkv=16."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi + 1, size=batch)
    return make_batch(rng, L, L, num_q_heads=HQ, num_kv_heads=HKV_LOCAL,
                      head_dim=HEAD_DIM, window=WINDOW_LOCAL,
                      rel_len=WINDOW_LOCAL, max_blocks_per_seq=MAX_BLOCKS,
                      poison=poison, name="local_prefill")


def global_mixed(seed: int = 0, n_decode: int = 48, n_chunks: int = 4,
                 chunk: int = 1024, poison: bool = True) -> Batch:
    """48 decode rows (contexts U[512, 8192]) then 4 chunks of 1024 new tokens
    on U[0, 7168] cached tokens; Hkv=8, full causal, R=8192."""
    rng = np.random.default_rng(seed)
    Ld = rng.integers(512, MAX_CONTEXT + 1, size=n_decode)
    cached = rng.integers(0, MAX_CONTEXT - chunk + 1, size=n_chunks)
    L = np.concatenate([Ld, cached + chunk])
    n = np.concatenate([np.ones(n_decode, dtype=np.int64),
                        np.full(n_chunks, chunk, dtype=np.int64)])
    return make_batch(rng, L, n, num_q_heads=HQ, num_kv_heads=HKV_GLOBAL,
                      head_dim=HEAD_DIM, window=0, rel_len=MAX_CONTEXT,
                      max_blocks_per_seq=MAX_BLOCKS, poison=poison,
                      name="global_mixed")


def long_global_decode(seed: int = 0, batch: int = 4, lo: int = 32768,
                       hi: int = 240000, poison: bool = True) -> Batch:
    """4 sequences, contexts U[32768, 240000], Hq=48, Hkv=8, full causal,
    R=8192 (distances past 8191 read the last entry)."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi + 1, size=batch)
    return make_batch(rng, L, np.ones_like(L), num_q_heads=HQ,
                      num_kv_heads=HKV_GLOBAL, head_dim=HEAD_DIM, window=0,
                      rel_len=MAX_CONTEXT, max_blocks_per_seq=(hi + BLOCK_SIZE - 1) // BLOCK_SIZE,
                      poison=poison, name="long_global_decode")


def long_global_prefill(seed: int = 0, batch: int = 2, chunk: int = 1024,
                        lo: int = 32768, hi: int = 98304, poison: bool = True) -> Batch:
    """Chunked prefill at long context on a global layer: 2 chunks of 1024 new
    tokens on U[32768, 98304] cached tokens; Hq=48, Hkv=8, full causal,
    R=8192 (distances past 8191 read the last entry)."""
    rng = np.random.default_rng(seed)
    cached = rng.integers(lo, hi + 1, size=batch)
    L = cached + chunk
    return make_batch(rng, L, np.full(batch, chunk, dtype=np.int64), num_q_heads=HQ,
                      num_kv_heads=HKV_GLOBAL, head_dim=HEAD_DIM, window=0,
                      rel_len=MAX_CONTEXT,
                      max_blocks_per_seq=(hi + chunk + BLOCK_SIZE - 1) // BLOCK_SIZE,
                      poison=poison, name="long_global_prefill")


# The smaller model of the same family (TensorRT-LLM Inkling page, commit
# list: the Inkling-Small accuracy commit gives 42 layers and hidden size
# 4096, and no head counts).  Reading: head_dim stays 128, so 32 query heads,
# and the KV head counts the Architecture section gives for the family (16
# local, 8 global) are kept, i.e. grouped-query ratios 2:1 and 4:1.
HQ_SMALL = 32


def small_local_decode(seed: int = 0, batch: int = 64, poison: bool = True) -> Batch:
    """The local decode batch at the smaller model's 32 query heads."""
    rng = np.random.default_rng(seed)
    L = rng.integers(1024, MAX_CONTEXT + 1, size=batch)
    return make_batch(rng, L, np.ones_like(L), num_q_heads=HQ_SMALL,
                      num_kv_heads=HKV_LOCAL, head_dim=HEAD_DIM,
                      window=WINDOW_LOCAL, rel_len=WINDOW_LOCAL,
                      max_blocks_per_seq=MAX_BLOCKS, poison=poison,
                      name="small_local_decode")


def small_global_decode(seed: int = 0, batch: int = 32, poison: bool = True) -> Batch:
    """The global decode batch at the smaller model's 32 query heads."""
    rng = np.random.default_rng(seed)
    L = rng.integers(4096, MAX_CONTEXT + 1, size=batch)
    return make_batch(rng, L, np.ones_like(L), num_q_heads=HQ_SMALL,
                      num_kv_heads=HKV_GLOBAL, head_dim=HEAD_DIM, window=0,
                      rel_len=MAX_CONTEXT, max_blocks_per_seq=MAX_BLOCKS,
                      poison=poison, name="small_global_decode")


def small_local_prefill(seed: int = 0, batch: int = 8, poison: bool = True) -> Batch:
    """The local varlen prefill batch at the smaller model's 32 query heads."""
    rng = np.random.default_rng(seed)
    L = rng.integers(2048, 4096 + 1, size=batch)
    return make_batch(rng, L, L, num_q_heads=HQ_SMALL, num_kv_heads=HKV_LOCAL,
                      head_dim=HEAD_DIM, window=WINDOW_LOCAL,
                      rel_len=WINDOW_LOCAL, max_blocks_per_seq=MAX_BLOCKS,
                      poison=poison, name="small_local_prefill")


WORKLOADS = {
    "tiny_prefill": tiny,
    "local_decode": local_decode,
    "global_decode": global_decode,
    "local_prefill": local_prefill,
    "global_mixed": global_mixed,
    "long_global_decode": long_global_decode,
    "long_global_prefill": long_global_prefill,
    "small_local_decode": small_local_decode,
    "small_global_decode": small_global_decode,
    "small_local_prefill": small_local_prefill,
}


def split_mixed(batch: Batch):
    """Split a mixed batch into (decode rows, prefill chunks) as two batches
    over the same page pool.  Pure re-indexing of already drawn tensors."""
    dec = np.nonzero(batch.q_lens == 1)[0]
    pre = np.nonzero(batch.q_lens != 1)[0]

    def sub(idx):
        rows = np.concatenate([np.arange(batch.cu_q_lens[b],
                                         batch.cu_q_lens[b + 1])
                               for b in idx]) if len(idx) else np.zeros(0, np.int64)
        rows_t = torch.from_numpy(rows.astype(np.int64))
        ql = batch.q_lens[idx]
        cu = np.zeros(len(idx) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(ql)
        return dataclasses.replace(
            batch, seq_lens=batch.seq_lens[idx].copy(), q_lens=ql.copy(),
            cu_q_lens=cu, q=batch.q[rows_t].contiguous(),
            block_table=batch.block_table[idx].copy(),
            rel_logits=batch.rel_logits[rows_t].contiguous(),
            k_logical=[batch.k_logical[b] for b in idx],
            v_logical=[batch.v_logical[b] for b in idx])

    return sub(dec), sub(pre)
