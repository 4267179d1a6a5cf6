"""fp64 CPU oracle for paged relative-bias attention (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the library.  It shares no code
with the HIP path; the two meet only in the input tensors.

The definition it evaluates, its page citations and the readings taken where
the pages are silent are documented at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "max_blocks_per_seq", "rel_len", "total_q")]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (fp64, IEEE, OpenMP)."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC",
                               "-shared", "-fno-fast-math", "-o", tmp, _SRC,
                               "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library and declare its entry points."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [
        ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_double,
        ctypes.POINTER(_Dims), P, P, P, ctypes.c_int64, P, P, ctypes.c_int32]
    lib.oracle_lse_combine.restype = None
    lib.oracle_lse_combine.argtypes = [ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_int32, P, P, P, P]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = load_library(_LIB)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _raw(t, dtype: str) -> np.ndarray:
    """Host array holding the exact stored bits (bf16 as uint16)."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if dtype == "bf16":
            assert t.dtype == torch.bfloat16
            return t.view(torch.int16).numpy()
        assert t.dtype == torch.float32
        return t.numpy()
    a = np.ascontiguousarray(t)
    if dtype == "bf16":
        assert a.dtype in (np.uint16, np.int16)
    else:
        assert a.dtype == np.float32
    return a


def _ptr(a) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def attention(*, dtype: str, q, k_cache, v_cache, block_table, seq_lens,
              cu_q_lens, rel_logits, window: int, scale: float,
              rows=None, key_lo=None, key_hi=None, threads: int = 0):
    """Evaluate the definition in fp64.

    q: [total_q, Hq, D]; k_cache / v_cache: [num_blocks, bs, Hkv, D];
    block_table: int32 [B, max_blocks]; seq_lens: int32 [B];
    cu_q_lens: int32 [B+1]; rel_logits: [total_q, Hq, R].
    rows: optional flat (i * Hq + h) indices.  key_lo/key_hi: optional
    per-sequence key range [lo, hi) intersected with the visible set.

    Returns (out, lse): out [total_q, Hq, D] (or [len(rows), D]) float64 and
    lse [total_q, Hq] (or [len(rows)]) float64.
    """
    lib = _load()
    qa, ka, va, ra = (_raw(x, dtype) for x in (q, k_cache, v_cache, rel_logits))
    total_q, Hq, D = qa.shape
    _, bs, Hkv, _ = ka.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cu = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
    dims = _Dims(num_seqs=sl.shape[0], num_q_heads=Hq, num_kv_heads=Hkv,
                 head_dim=D, block_size=bs, max_blocks_per_seq=bt.shape[1],
                 rel_len=ra.shape[-1], total_q=total_q)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.shape[0]
    else:
        n = total_q * Hq
    lo = None if key_lo is None else np.ascontiguousarray(key_lo, dtype=np.int32)
    hi = None if key_hi is None else np.ascontiguousarray(key_hi, dtype=np.int32)
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_attention(0 if dtype == "bf16" else 1, _ptr(qa), _ptr(ka),
                              _ptr(va), _ptr(bt), _ptr(sl), _ptr(cu), _ptr(ra),
                              int(window), float(scale), ctypes.byref(dims),
                              _ptr(lo), _ptr(hi), _ptr(rows), n, _ptr(out),
                              _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    if rows is None:
        return out.reshape(total_q, Hq, D), lse.reshape(total_q, Hq)
    return out, lse


def lse_combine(o_s: np.ndarray, lse_s: np.ndarray):
    """Merge partials o_s [S, n, D], lse_s [S, n] -> (out [n, D], lse [n])."""
    lib = _load()
    o_s = np.ascontiguousarray(o_s, dtype=np.float64)
    lse_s = np.ascontiguousarray(lse_s, dtype=np.float64)
    S, n, D = o_s.shape
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    lib.oracle_lse_combine(S, n, D, _ptr(o_s), _ptr(lse_s), _ptr(out), _ptr(lse))
    return out, lse


def run_batch(batch, rows=None, key_lo=None, key_hi=None, threads: int = 0):
    """Convenience: evaluate a batch object carrying the tensors above."""
    return attention(dtype=batch.dtype, q=batch.q, k_cache=batch.k_cache,
                     v_cache=batch.v_cache, block_table=batch.block_table,
                     seq_lens=batch.seq_lens, cu_q_lens=batch.cu_q_lens,
                     rel_logits=batch.rel_logits, window=batch.window,
                     scale=batch.scale, rows=rows, key_lo=key_lo,
                     key_hi=key_hi, threads=threads)
