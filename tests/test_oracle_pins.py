"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes part of the definition (TensorRT-LLM Inkling page, section
'Architecture': learned per-(query token, head, distance) bias added to the
scaled logits before the softmax; sliding-window local layers and full-causal
global layers; grouped KV heads; vLLM page, section 'Purpose': keys and
values live in a paged cache) so that a plausible slip in the oracle - a
dropped term, a wrong sign or index, a transposed operand - fails one of them:

  * hand-derived closed forms (tests/golden/hand_cases.json);
  * a dense brute force on unpaged logical K/V (tests/bruteforce.py);
  * the library special case: zero bias reduces to torch's
    scaled_dot_product_attention with an explicit causal mask;
  * invariants: constant bias, page permutation, NaN poison, head subsets,
    chunked prefill, prefill-vs-decode, split + log-sum-exp merge;
  * closed forms: a single visible key returns V, a uniform window returns
    the mean position, a +40 one-hot bias selects one key.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_relative_bias_amd import inputs
from tests.bruteforce import dense_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _arr(x):
    """Nested JSON lists -> float64 array; null -> NaN."""
    def conv(v):
        if isinstance(v, list):
            return [conv(u) for u in v]
        return np.nan if v is None else v
    return np.array(conv(x), dtype=np.float64)


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    f32 = lambda k: torch.from_numpy(_arr(case[k]).astype(np.float32))
    out, lse = oracle.attention(
        dtype="fp32", q=f32("q"), k_cache=f32("k_cache"), v_cache=f32("v_cache"),
        block_table=np.array(case["block_table"], dtype=np.int32),
        seq_lens=np.array(case["seq_lens"], dtype=np.int32),
        cu_q_lens=np.array(case["cu_q_lens"], dtype=np.int32),
        rel_logits=f32("rel_logits"), window=case["window"], scale=case["scale"])
    np.testing.assert_allclose(out, np.array(case["expected_out"]), rtol=1e-6, atol=0)
    np.testing.assert_allclose(lse, np.array(case["expected_lse"]), rtol=1e-6, atol=0)


def _random_batch(rng, *, B, Hq, Hkv, D, W, R, dtype="fp32", poison=True,
                  decode=False, bs=16):
    L = rng.integers(1, 71, size=B)
    if decode:
        n = np.ones_like(L)
    else:
        n = np.array([rng.integers(1, l + 1) for l in L])
    return inputs.make_batch(rng, L, n, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=D, window=W, rel_len=R, dtype=dtype,
                             poison=poison, block_size=bs,
                             max_blocks_per_seq=int(np.ceil(70 / bs)) + 1,
                             spare_pages=3)


CASES = [(B, Hq, Hkv, D, W, R, bs)
         for (B, Hq, Hkv) in [(1, 2, 1), (3, 4, 2), (2, 6, 3), (2, 6, 1)]
         for D in (8, 64)
         for (W, R) in [(1, 4), (3, 3), (16, 16), (32, 8), (0, 70), (0, 5)]
         for bs in (16, 5)]


@pytest.mark.parametrize("B,Hq,Hkv,D,W,R,bs", CASES[::3])
def test_bruteforce_agreement(B, Hq, Hkv, D, W, R, bs):
    rng = np.random.default_rng(1000 + B * 7 + Hq * 3 + D + W + R + bs)
    batch = _random_batch(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, R=R, bs=bs)
    out, lse = oracle.run_batch(batch)
    ref, ref_lse = dense_attention(batch)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_bruteforce_bf16_and_tiny_workload():
    batch = inputs.tiny()
    out, lse = oracle.run_batch(batch)
    ref, ref_lse = dense_attention(batch)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    rng = np.random.default_rng(7)
    b16 = _random_batch(rng, B=3, Hq=6, Hkv=2, D=64, W=16, R=16, dtype="bf16")
    out, lse = oracle.run_batch(b16)
    ref, ref_lse = dense_attention(b16)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_bf16_read_matches_torch_widening():
    """The oracle's bf16 decoding equals torch's exact bf16 -> fp32 cast."""
    rng = np.random.default_rng(3)
    b16 = _random_batch(rng, B=2, Hq=4, Hkv=2, D=8, W=0, R=70, dtype="bf16")
    f32 = inputs.Batch(**{**b16.__dict__})
    f32.dtype = "fp32"
    f32.q = b16.q.float()
    f32.k_cache = b16.k_cache.float()
    f32.v_cache = b16.v_cache.float()
    f32.rel_logits = b16.rel_logits.float()
    a, la = oracle.run_batch(b16)
    b, lb = oracle.run_batch(f32)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("W", [0, 200])
def test_zero_bias_reduces_to_sdpa(W):
    """Zero bias and W >= L: plain causal attention (torch SDPA, fp64)."""
    rng = np.random.default_rng(11)
    batch = _random_batch(rng, B=3, Hq=6, Hkv=2, D=16, W=W, R=70, poison=False)
    batch.rel_logits.zero_()
    out, _ = oracle.run_batch(batch)
    G = batch.num_q_heads // batch.num_kv_heads
    for b in range(batch.num_seqs):
        n, L = int(batch.q_lens[b]), int(batch.seq_lens[b])
        i0 = int(batch.cu_q_lens[b])
        q = batch.q[i0:i0 + n].double().permute(1, 0, 2)[None]
        k = batch.k_logical[b].double().repeat_interleave(G, 1).permute(1, 0, 2)[None]
        v = batch.v_logical[b].double().repeat_interleave(G, 1).permute(1, 0, 2)[None]
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=mask, scale=batch.scale)[0].permute(1, 0, 2)
        np.testing.assert_allclose(out[i0:i0 + n], ref.numpy(), rtol=0, atol=1e-12)


def test_constant_bias_is_invisible():
    rng = np.random.default_rng(12)
    batch = _random_batch(rng, B=2, Hq=4, Hkv=2, D=16, W=9, R=9, poison=False)
    c = torch.randn(batch.total_q, batch.num_q_heads, 1) * 5
    batch.rel_logits = c.expand_as(batch.rel_logits).contiguous()
    out_c, lse_c = oracle.run_batch(batch)
    batch.rel_logits = torch.zeros_like(batch.rel_logits)
    out_0, lse_0 = oracle.run_batch(batch)
    np.testing.assert_allclose(out_c, out_0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_c - lse_0, c[..., 0].double().numpy(),
                               rtol=0, atol=1e-12)


def test_page_permutation_is_invisible():
    rng = np.random.default_rng(13)
    batch = _random_batch(rng, B=3, Hq=4, Hkv=2, D=8, W=0, R=70, bs=5)
    out, lse = oracle.run_batch(batch)
    perm = rng.permutation(batch.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    pt = torch.from_numpy(inv)
    k2 = torch.empty_like(batch.k_cache)
    v2 = torch.empty_like(batch.v_cache)
    k2[pt] = batch.k_cache
    v2[pt] = batch.v_cache
    bt = np.where(batch.block_table >= 0, inv[np.maximum(batch.block_table, 0)], -1)
    batch.k_cache, batch.v_cache, batch.block_table = k2, v2, bt.astype(np.int32)
    out2, lse2 = oracle.run_batch(batch)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_poison_is_invisible():
    """NaN in every never-read byte leaves the output finite and bit-equal."""
    seeds = dict(B=3, Hq=4, Hkv=2, D=8, W=7, R=9)
    a = _random_batch(np.random.default_rng(14), poison=True, **seeds)
    b = _random_batch(np.random.default_rng(14), poison=False, **seeds)
    assert torch.isnan(a.k_cache).any() and torch.isnan(a.rel_logits).any()
    oa, la = oracle.run_batch(a)
    ob, lb = oracle.run_batch(b)
    assert np.all(np.isfinite(oa))
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_single_visible_key_returns_v():
    rng = np.random.default_rng(15)
    for W in (1, 0):
        batch = _random_batch(rng, B=3, Hq=4, Hkv=2, D=8, W=W, R=4)
        out, lse = oracle.run_batch(batch)
        G = batch.num_q_heads // batch.num_kv_heads
        for b in range(batch.num_seqs):
            n, L = int(batch.q_lens[b]), int(batch.seq_lens[b])
            for t in range(n):
                p = L - n + t
                if W == 1 or p == 0:
                    v = batch.v_logical[b][p].double().repeat_interleave(G, 0)
                    assert np.array_equal(out[batch.cu_q_lens[b] + t], v.numpy())


@pytest.mark.parametrize("W", [1, 5, 16, 0])
def test_uniform_window_mean_position(W):
    """q = 0, bias = 0, V[j] = j: out = mean of [max(0, p-W+1), p]."""
    rng = np.random.default_rng(16)
    batch = _random_batch(rng, B=3, Hq=2, Hkv=1, D=4, W=W, R=4)
    batch.q.zero_()
    batch.rel_logits.zero_()
    for b in range(batch.num_seqs):
        L = int(batch.seq_lens[b])
        code = torch.arange(L, dtype=torch.float32)[:, None, None].expand(L, 1, 4)
        blocks = batch.block_table[b]
        for j in range(L):
            batch.v_cache[blocks[j // 16], j % 16] = code[j]
    out, _ = oracle.run_batch(batch)
    for b in range(batch.num_seqs):
        n, L = int(batch.q_lens[b]), int(batch.seq_lens[b])
        for t in range(n):
            p = L - n + t
            lo = max(0, p - W + 1) if W > 0 else 0
            assert np.all(out[batch.cu_q_lens[b] + t] == (lo + p) / 2.0)


def test_onehot_bias_selects_distance():
    """+40 at distance d*: weight on key p - d* is >= 1 - L e^-40."""
    rng = np.random.default_rng(17)
    batch = _random_batch(rng, B=2, Hq=2, Hkv=1, D=4, W=0, R=70, decode=True,
                          poison=False)
    batch.q.zero_()
    for dstar in (0, 1, 5):
        batch.rel_logits.zero_()
        batch.rel_logits[:, :, dstar] = 40.0
        out, _ = oracle.run_batch(batch)
        for b in range(batch.num_seqs):
            L = int(batch.seq_lens[b])
            if L - 1 - dstar < 0:
                continue
            v = batch.v_logical[b][L - 1 - dstar, 0].double().numpy()
            np.testing.assert_allclose(out[b, 0], v, rtol=0, atol=1e-14 * 70)


def test_onehot_clamp_entry_covers_far_keys():
    """R < L: +40 at entry R-1 weighs every key with d >= R-1 equally."""
    rng = np.random.default_rng(18)
    R = 6
    batch = inputs.make_batch(rng, [40, 23], [1, 1], num_q_heads=2,
                              num_kv_heads=1, head_dim=4, window=0, rel_len=R,
                              dtype="fp32", poison=False)
    batch.q.zero_()
    batch.rel_logits.zero_()
    batch.rel_logits[:, :, R - 1] = 40.0
    out, _ = oracle.run_batch(batch)
    for b in range(2):
        L = int(batch.seq_lens[b])
        far = batch.v_logical[b][: L - 1 - (R - 1) + 1, 0].double().mean(0).numpy()
        np.testing.assert_allclose(out[b, 0], far, rtol=0, atol=1e-12)


def test_gqa_probe_selects_query_heads():
    """Only the G query heads of the one non-zero KV head see non-uniform
    attention (contiguous groups: h / (Hq / Hkv))."""
    rng = np.random.default_rng(19)
    batch = _random_batch(rng, B=2, Hq=6, Hkv=3, D=8, W=0, R=70, decode=True,
                          poison=False)
    batch.rel_logits.zero_()
    batch.k_cache.zero_()
    hot = 1
    for b in range(batch.num_seqs):
        L = int(batch.seq_lens[b])
        for j in range(L):
            batch.k_cache[batch.block_table[b][j // 16], j % 16, hot] = \
                batch.k_logical[b][j, hot] * 8
    out, _ = oracle.run_batch(batch)
    for b in range(batch.num_seqs):
        L = int(batch.seq_lens[b])
        if L < 3:
            continue
        for h in range(6):
            g = h // 2
            mean = batch.v_logical[b][:, g].double().mean(0).numpy()
            uniform = np.allclose(out[b, h], mean, atol=1e-12)
            assert uniform == (g != hot), (b, h)


def test_split_merge_equals_whole():
    rng = np.random.default_rng(20)
    batch = _random_batch(rng, B=3, Hq=4, Hkv=2, D=8, W=0, R=70, decode=True)
    out, lse = oracle.run_batch(batch)
    for S in (1, 2, 3, 8):
        cuts = [np.sort(np.concatenate([[0, int(L)], rng.integers(0, int(L) + 1, S - 1)]))
                for L in batch.seq_lens]
        o_s, l_s = [], []
        for s in range(S):
            lo = np.array([c[s] for c in cuts], dtype=np.int32)
            hi = np.array([c[s + 1] for c in cuts], dtype=np.int32)
            o, l = oracle.run_batch(batch, key_lo=lo, key_hi=hi)
            o_s.append(o.reshape(-1, 8))
            l_s.append(l.reshape(-1))
        m, ml = oracle.lse_combine(np.stack(o_s), np.stack(l_s))
        np.testing.assert_allclose(m.reshape(out.shape), out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml.reshape(lse.shape), lse, rtol=0, atol=1e-12)


def test_prefill_last_row_equals_decode_and_chunking():
    rng = np.random.default_rng(21)
    full = inputs.make_batch(rng, [50, 33], [20, 33], num_q_heads=4,
                             num_kv_heads=2, head_dim=8, window=12, rel_len=12,
                             dtype="fp32")
    out, lse = oracle.run_batch(full)
    # decode of each sequence at its last position: same pages, q row, rel row
    last = full.cu_q_lens[1:] - 1
    dec = inputs.Batch(**{**full.__dict__})
    dec.q_lens = np.ones(2, np.int32)
    dec.cu_q_lens = np.arange(3, dtype=np.int32)
    dec.q = full.q[torch.from_numpy(last.astype(np.int64))]
    dec.rel_logits = full.rel_logits[torch.from_numpy(last.astype(np.int64))]
    od, ld = oracle.run_batch(dec)
    assert np.array_equal(od, out[last]) and np.array_equal(ld, lse[last])
    # chunked: first k tokens of sequence 0 on fewer keys, then the rest
    k = 7
    c1 = inputs.Batch(**{**full.__dict__})
    c1.seq_lens = np.array([50 - 20 + k], np.int32)
    c1.q_lens = np.array([k], np.int32)
    c1.cu_q_lens = np.array([0, k], np.int32)
    c1.block_table = full.block_table[:1]
    c1.q, c1.rel_logits = full.q[:k], full.rel_logits[:k]
    o1, _ = oracle.run_batch(c1)
    assert np.array_equal(o1, out[:k])
    c2 = inputs.Batch(**{**c1.__dict__})
    c2.seq_lens = np.array([50], np.int32)
    c2.q_lens = np.array([20 - k], np.int32)
    c2.cu_q_lens = np.array([0, 20 - k], np.int32)
    c2.q, c2.rel_logits = full.q[k:20], full.rel_logits[k:20]
    o2, _ = oracle.run_batch(c2)
    assert np.array_equal(o2, out[k:20])


def test_row_subset_equals_slice():
    rng = np.random.default_rng(22)
    batch = _random_batch(rng, B=3, Hq=6, Hkv=2, D=8, W=5, R=5)
    out, lse = oracle.run_batch(batch)
    rows = rng.choice(batch.total_q * 6, size=17, replace=False)
    o, l = oracle.run_batch(batch, rows=rows)
    assert np.array_equal(o, out.reshape(-1, 8)[rows])
    assert np.array_equal(l, lse.reshape(-1)[rows])


def test_empty_visible_set_is_zero():
    """R9: no visible key (only reachable through a key range) -> 0, -inf."""
    rng = np.random.default_rng(23)
    batch = _random_batch(rng, B=2, Hq=2, Hkv=1, D=4, W=0, R=70, decode=True)
    z = np.zeros(2, np.int32)
    o, l = oracle.run_batch(batch, key_lo=z, key_hi=z)
    assert np.all(o == 0) and np.all(l == -np.inf)
