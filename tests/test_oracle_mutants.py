"""The pins are strong enough: each planted slip in a copy of the oracle
fails at least one of them (CPU only; the mutants are built with gcc into a
temporary directory and never touch the real oracle library)."""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from paged_relative_bias_amd import inputs
from tests.bruteforce import dense_attention
from tests.test_oracle_pins import GOLDEN, _arr

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement): each is a mistake one could make
MUTANTS = [
    ("bias_by_key_not_distance",
     "const int di = d < R - 1 ? d : R - 1;",
     "const int di = j < R - 1 ? j : R - 1;"),
    ("bias_scaled_too",
     "s[j] = scale * dot + rd(rel_logits, dtype, roff + di);",
     "s[j] = scale * (dot + rd(rel_logits, dtype, roff + di));"),
    ("window_off_by_one",
     "(window <= 0 || d < window)", "(window <= 0 || d <= window)"),
    ("gqa_modulo_mapping", "const int g = h / G;", "const int g = h % Hkv;"),
    ("top_left_positions",
     "const int p = L - n_b + (int)(i - cu_q_lens[b]);",
     "const int p = (int)(i - cu_q_lens[b]);"),
    ("far_keys_dropped_not_clamped",
     "vis[j] = (d >= 0) &&", "vis[j] = (d >= 0) && d < R &&"),
    ("lse_without_log", "lse[r] = M + log(Z);", "lse[r] = M + Z;"),
    ("v_from_k_cache",
     "acc[k] += w * rd(v_cache, dtype, voff + k);",
     "acc[k] += w * rd(k_cache, dtype, voff + k);"),
    ("slot_from_wrong_key",
     "const int64_t voff = (((int64_t)blk * bs + j % bs) * Hkv + g) * D;",
     "const int64_t voff = (((int64_t)blk * bs + (bs - 1 - j % bs)) * Hkv + g) * D;"),
]


def _pins_pass():
    """A fast subset of the pins; False as soon as one fails."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        f32 = lambda k: torch.from_numpy(_arr(c[k]).astype(np.float32))
        out, lse = oracle.attention(
            dtype="fp32", q=f32("q"), k_cache=f32("k_cache"),
            v_cache=f32("v_cache"),
            block_table=np.array(c["block_table"], dtype=np.int32),
            seq_lens=np.array(c["seq_lens"], dtype=np.int32),
            cu_q_lens=np.array(c["cu_q_lens"], dtype=np.int32),
            rel_logits=f32("rel_logits"), window=c["window"], scale=c["scale"])
        if not (np.allclose(out, c["expected_out"], rtol=1e-6, atol=0) and
                np.allclose(lse, c["expected_lse"], rtol=1e-6, atol=0)):
            return False
    rng = np.random.default_rng(5)
    for (W, R) in [(7, 9), (0, 20)]:
        L = rng.integers(1, 60, size=3)
        n = np.array([rng.integers(1, l + 1) for l in L])
        b = inputs.make_batch(rng, L, n, num_q_heads=6, num_kv_heads=2,
                              head_dim=8, window=W, rel_len=R, dtype="fp32",
                              poison=False)
        out, lse = oracle.run_batch(b)
        ref, ref_lse = dense_attention(b)
        if not (np.allclose(out, ref, rtol=0, atol=1e-12) and
                np.allclose(lse, ref_lse, rtol=0, atol=1e-12)):
            return False
    return True


def test_real_oracle_passes_the_subset():
    assert _pins_pass()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC",
                           "-shared", "-o", str(lib), str(path), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(str(lib)))
    assert not _pins_pass(), name
