"""The seeded input generator lays data out as documented (CPU only)."""
import numpy as np
import torch

from paged_relative_bias_amd import inputs


def test_pages_hold_logical_keys_and_poison_elsewhere():
    W = 6
    b = inputs.make_batch(np.random.default_rng(0), [37, 5, 16], [3, 5, 1],
                          num_q_heads=4, num_kv_heads=2, head_dim=8, window=W,
                          rel_len=8, dtype="bf16", spare_pages=5)
    used = set()
    for s in range(b.num_seqs):
        L, n = int(b.seq_lens[s]), int(b.q_lens[s])
        npg = (L + 15) // 16
        assert np.all(b.block_table[s, npg:] == -1)
        stale = max(0, L - n - W + 1)      # keys older than every query's window
        for j in range(L):
            blk = int(b.block_table[s, j // 16])
            used.add(blk)
            if j < stale:
                assert torch.isnan(b.k_cache[blk, j % 16].float()).all()
                assert torch.isnan(b.v_cache[blk, j % 16].float()).all()
                continue
            assert torch.equal(b.k_cache[blk, j % 16], b.k_logical[s][j])
            assert torch.equal(b.v_cache[blk, j % 16], b.v_logical[s][j])
        last = int(b.block_table[s, npg - 1])
        assert torch.isnan(b.k_cache[last, (L - 1) % 16 + 1:].float()).all()
    spare = [p for p in range(b.num_blocks) if p not in used]
    assert len(spare) == 5
    assert torch.isnan(b.v_cache[spare].float()).all()


def test_bias_poison_marks_exactly_the_unread_entries():
    W, R = 6, 8
    b = inputs.make_batch(np.random.default_rng(1), [37, 5, 16], [3, 5, 1],
                          num_q_heads=4, num_kv_heads=2, head_dim=8, window=W,
                          rel_len=R, dtype="fp32")
    for s in range(b.num_seqs):
        n, L = int(b.q_lens[s]), int(b.seq_lens[s])
        for t in range(n):
            p = L - n + t
            used = {min(d, R - 1) for d in range(p + 1) if d < W}
            row = b.rel_logits[b.cu_q_lens[s] + t]
            for e in range(R):
                assert bool(torch.isnan(row[:, e]).all()) == (e not in used)


def test_workloads_are_deterministic_and_shaped():
    a, b = inputs.tiny(), inputs.tiny()
    assert torch.equal(a.q, b.q) and np.array_equal(a.block_table, b.block_table)
    assert a.q.dtype == torch.float32 and tuple(a.rel_logits.shape) == (64, 4, 32)
    assert a.window == 32 and a.num_kv_heads == 2 and a.head_dim == 64
    d = inputs.local_decode(batch=4)
    assert d.q.dtype == torch.bfloat16 and d.is_decode()
    assert d.max_blocks_per_seq == 512 and tuple(d.rel_logits.shape) == (4, 48, 512)
    assert np.all((d.seq_lens >= 1024) & (d.seq_lens <= 8192))


def test_mixed_split_reindexes_without_copying_arithmetic():
    rng = np.random.default_rng(2)
    b = inputs.make_batch(rng, [9, 40, 3, 20], [1, 17, 1, 20], num_q_heads=2,
                          num_kv_heads=1, head_dim=8, window=0, rel_len=40)
    dec, pre = inputs.split_mixed(b)
    assert list(dec.seq_lens) == [9, 3] and list(pre.seq_lens) == [40, 20]
    assert torch.equal(dec.q[1], b.q[18])
    assert torch.equal(pre.q[17], b.q[19])
