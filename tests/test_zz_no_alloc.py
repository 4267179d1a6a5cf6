"""inkling_rel_attn_decode_noalloc (the decode that allocates nothing and
keeps its split partials in the library's per-GPU buffer) against
inkling_rel_attn_decode with a caller workspace: two calls in a row, the
second on a smaller batch, both through the C ABI; each bit-equal to the
workspace form and within the bar of the oracle."""
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


def _noalloc(d, splits):
    b = d.batch
    out = torch.full_like(d.q, float("nan"))
    binding.decode_noalloc(d.q, d.k, d.v, d.bt, d.sl, d.rel, b.window, b.scale, out,
                           max_seq_len=b.max_seq_len, num_splits=splits)
    return out


@pytest.mark.parametrize("splits", [0, 8, 1])
def test_noalloc_matches_workspace_decode_twice(splits):
    big = inputs.make_batch(np.random.default_rng(90), [4000, 7000, 33, 1500, 6000, 900],
                            [1] * 6, num_q_heads=48, num_kv_heads=8, head_dim=128,
                            window=0, rel_len=8192, dtype="bf16")
    small = inputs.make_batch(np.random.default_rng(91), [700, 20], [1, 1], num_q_heads=48,
                              num_kv_heads=8, head_dim=128, window=0, rel_len=8192,
                              dtype="bf16")
    for name, b in (("big", big), ("small", small)):
        print(f"noalloc decode {name}: L={b.seq_lens.tolist()} splits={splits}", flush=True)
        d = U.Dev(b)
        got = _noalloc(d, splits)
        want = U.decode(d, splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name
        ref, _ = oracle.run_batch(b)
        U.compare(got, ref, "bf16", f"noalloc/{name}/s{splits}")


def test_noalloc_rejects_oversized_split_workspace():
    b = inputs.make_batch(np.random.default_rng(92), [9000] * 64, [1] * 64, num_q_heads=48,
                          num_kv_heads=8, head_dim=128, window=0, rel_len=8192,
                          dtype="bf16", spare_pages=1)
    d = U.Dev(b)
    out = torch.zeros_like(d.q)
    with pytest.raises(binding.InklingError) as e:
        binding.decode_noalloc(d.q, d.k, d.v, d.bt, d.sl, d.rel, b.window, b.scale, out,
                               max_seq_len=b.max_seq_len, num_splits=128)
    assert e.value.status == 5   # INKLING_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0   # nothing launched
