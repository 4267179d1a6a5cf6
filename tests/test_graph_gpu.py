"""Decode captured once in a HIP graph and replayed with new device-side
metadata (sequence lengths, block table) between replays.

The launch reads `seq_lens` and `block_table` from device memory and takes
only host bounds (max_seq_len, num_splits) as arguments, so one capture
serves every step whose lengths stay within the captured bound.  Each replay
is checked against an eager call on the same metadata (bit-equal) and
against the fp64 oracle; lengths cross page boundaries between replays.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_relative_bias_amd import binding, inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st, msg = binding.check_device(0)
    assert st == binding.OK, msg
    yield
    torch.cuda.synchronize()


def _say(*a):
    print(*a, flush=True)


# Lengths per replay: every sequence moves across a page boundary (16 keys)
# at least once, and one sequence steps through 15 -> 16 -> 17 -> 33.
LENGTH_STEPS = [
    [15, 700, 2049, 4000],
    [16, 701, 2048, 4001],
    [17, 512, 2050, 3999],
    [33, 513, 2047, 4096],
]


def _batch(W, R, Hq, Hkv, seed):
    Lmax = np.max(np.array(LENGTH_STEPS), axis=0).tolist()
    rng = np.random.default_rng(seed)
    # Replays use shorter lengths than the batch is drawn with, so keys
    # older than the longest lengths' windows stay finite.
    return inputs.make_batch(rng, Lmax, [1] * len(Lmax), num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=128, window=W, rel_len=R, dtype="bf16",
                             poison_stale=False)


def _permute_pages(d: U.Dev, b, seed):
    """Moves every cache page to a new physical slot (in place on the
    device) and rewrites the block table to match."""
    perm = np.random.default_rng(seed).permutation(b.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    idx = torch.from_numpy(inv).to(d.k.device)
    k2 = torch.empty_like(d.k)
    v2 = torch.empty_like(d.v)
    k2[idx] = d.k
    v2[idx] = d.v
    d.k.copy_(k2)
    d.v.copy_(v2)
    bt = d.bt.cpu().numpy()
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    d.bt.copy_(torch.from_numpy(bt2))


@pytest.mark.parametrize("W,R,Hq,Hkv,splits", [(512, 512, 48, 16, 1), (0, 8192, 48, 8, 4),
                                               (0, 8192, 12, 2, 0)])
def test_decode_graph_replay_with_new_metadata(W, R, Hq, Hkv, splits):
    b = _batch(W, R, Hq, Hkv, seed=60 + Hkv)
    d = U.Dev(b)
    dims = binding.dims_for(d.q, d.k, d.bt, d.rel, num_seqs=b.num_seqs, max_q_len=1,
                            max_seq_len=b.max_seq_len)
    need = binding.decode_workspace_bytes(dims, W, splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    out = torch.full_like(d.q, float("nan"))
    stream = torch.cuda.Stream()

    def launch(o, s):
        binding.decode(d.q, d.k, d.v, d.bt, d.sl, d.rel, W, b.scale, o,
                       max_seq_len=b.max_seq_len, num_splits=splits, workspace=ws, stream=s)

    # Warm-up on the capture stream (sets kernel attributes once).
    d.sl.copy_(torch.tensor(LENGTH_STEPS[0], dtype=torch.int32))
    with torch.cuda.stream(stream):
        launch(out, stream)
    stream.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        launch(out, torch.cuda.current_stream())

    eager = torch.empty_like(out)
    for step, lens in enumerate(LENGTH_STEPS + LENGTH_STEPS[::-1]):
        _say(f"graph decode W={W} Hkv={Hkv} splits={splits} step {step} lens={lens}")
        d.sl.copy_(torch.tensor(lens, dtype=torch.int32))
        if step == 3:
            _permute_pages(d, b, seed=step)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        # Eager call on the same metadata, between replays.
        launch(eager, None)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"step {step}"
        ref, _ = oracle.run_batch(dataclasses.replace(b, seq_lens=np.array(lens, np.int32)))
        U.compare(out, ref, "bf16", f"graph/{W}/{Hkv}/s{splits}/step{step}")
