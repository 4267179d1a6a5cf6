"""Dense brute force used only to pin the oracle.

It never touches the page pool: it works on the per-sequence *logical* K/V
kept by the input generator, builds the whole [n, L] distance matrix, the mask
and the gathered bias as dense arrays, and applies a numpy softmax.  So it
shares neither the paged gather nor the row loop of the oracle and catches
mistakes in either (page/slot indexing, the position formula, the clamp).
"""
import numpy as np
import torch


def _f64(t) -> np.ndarray:
    return t.detach().to(torch.float64).numpy()


def dense_attention(batch):
    """Return (out [total_q, Hq, D], lse [total_q, Hq]) in float64."""
    Hq, Hkv, D = batch.num_q_heads, batch.num_kv_heads, batch.head_dim
    G = Hq // Hkv
    W, R = batch.window, batch.rel_len
    out = np.zeros((batch.total_q, Hq, D))
    lse = np.full((batch.total_q, Hq), -np.inf)
    q = _f64(batch.q)
    rel = _f64(batch.rel_logits)
    for b in range(batch.num_seqs):
        n, L = int(batch.q_lens[b]), int(batch.seq_lens[b])
        if n == 0:
            continue
        i0 = int(batch.cu_q_lens[b])
        Q = q[i0:i0 + n]                                        # [n, Hq, D]
        K = np.repeat(_f64(batch.k_logical[b]), G, axis=1)      # [L, Hq, D]
        V = np.repeat(_f64(batch.v_logical[b]), G, axis=1)
        pos_q = np.arange(L - n, L)
        pos_k = np.arange(L)
        dist = pos_q[:, None] - pos_k[None, :]                  # [n, L]
        mask = dist >= 0
        if W > 0:
            mask &= dist < W
        idx = np.clip(dist, 0, R - 1)
        bias = np.take_along_axis(
            rel[i0:i0 + n], np.broadcast_to(idx[:, None, :], (n, Hq, L)), axis=2)
        with np.errstate(invalid="ignore"):
            S = batch.scale * np.einsum("nhd,lhd->nhl", Q, K) + bias
        S = np.where(mask[:, None, :], S, -np.inf)
        M = S.max(axis=-1, keepdims=True)
        empty = ~np.isfinite(M)
        Ms = np.where(empty, 0.0, M)
        P = np.exp(S - Ms)
        Z = P.sum(axis=-1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            O = np.einsum("nhl,lhd->nhd", P, V) / Z
            ls = (Ms + np.log(Z))[..., 0]
        O = np.where(empty, 0.0, O)
        ls = np.where(empty[..., 0], -np.inf, ls)
        out[i0:i0 + n] = O
        lse[i0:i0 + n] = ls
    return out, lse
