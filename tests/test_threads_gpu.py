"""The library's first calls made from two host threads at once.

Each kernel raises its LDS limit once per process, under std::call_once; a
fresh process whose first prefill and decode calls come from two threads
concurrently must launch correctly from both.  The calls run in a child
process so that they really are the process's first.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

_CHILD = r"""
import sys, threading
import numpy as np
import torch
sys.path.insert(0, ROOT)
from paged_relative_bias_amd import binding, inputs
from tests import gpu_util as U

st, msg = binding.check_device(0)
assert st == binding.OK, msg
pre = inputs.make_batch(np.random.default_rng(5), [300, 200], [300, 40], num_q_heads=12,
                        num_kv_heads=4, head_dim=128, window=64, rel_len=64)
dec = inputs.make_batch(np.random.default_rng(6), [900, 300], [1, 1], num_q_heads=12,
                        num_kv_heads=4, head_dim=128, window=0, rel_len=512)
dp, dd = U.Dev(pre), U.Dev(dec)
torch.cuda.synchronize()
start = threading.Barrier(2)
outs, errs = [None, None], []


def work(i):
    try:
        s = torch.cuda.Stream()
        start.wait()
        o1 = U.prefill(dp, stream=s)
        o2 = U.decode(dd, splits=3, stream=s)
        s.synchronize()
        outs[i] = (o1, o2)
    except Exception as e:  # reported by the parent
        errs.append(repr(e))


ts = [threading.Thread(target=work, args=(i,)) for i in range(2)]
for t in ts:
    t.start()
for t in ts:
    t.join()
assert not errs, errs
r1, r2 = U.prefill(dp), U.decode(dd, splits=3)
torch.cuda.synchronize()
for o1, o2 in outs:
    assert torch.equal(o1.view(torch.int16), r1.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), r2.view(torch.int16))
print("two-thread first calls: ok", flush=True)
"""


def test_first_calls_from_two_threads():
    code = "ROOT = " + repr(ROOT) + "\n" + _CHILD
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
