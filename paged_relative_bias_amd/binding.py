"""Python binding of libinkling_rel_attn.so (ctypes; argument marshalling only).

Every step of the attention runs inside the library's HIP kernels; this
module only turns torch tensors into pointers and shapes, picks the current
torch stream, and raises on a non-OK status.  There is no fallback: if the
library is missing or the device is not gfx950, calls fail loudly.

Names mirror the C ABI in include/inkling_rel_attn.h:
    prefill, prefill_append, decode, decode_append, decode_noalloc,
    num_splits, decode_workspace_bytes, check_device, status_string.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinkling_rel_attn.so")

OK = 0
DTYPE_BF16, DTYPE_FP32 = 0, 1
SYMBOLS = (
    "inkling_rel_attn_prefill",
    "inkling_rel_attn_prefill_append",
    "inkling_rel_attn_decode",
    "inkling_rel_attn_decode_append",
    "inkling_rel_attn_decode_noalloc",
    "inkling_rel_attn_num_splits",
    "inkling_rel_attn_decode_workspace_bytes",
    "inkling_rel_attn_check_device",
    "inkling_rel_attn_status_string",
)


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "num_blocks", "max_blocks_per_seq", "rel_len", "total_q", "max_q_len",
        "max_seq_len", "dtype")]


class InklingError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Open the library (once) and declare its entry points."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing; build it with `python -m paged_relative_bias_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    DP = ctypes.POINTER(Dims)
    lib.inkling_rel_attn_prefill.restype = ctypes.c_int
    lib.inkling_rel_attn_prefill.argtypes = [P, P, P, P, P, P, P, I32, F32, P, DP, P]
    lib.inkling_rel_attn_prefill_append.restype = ctypes.c_int
    lib.inkling_rel_attn_prefill_append.argtypes = [P, P, P, P, P, P, P, P, P, I32, F32, P, DP, P]
    lib.inkling_rel_attn_decode.restype = ctypes.c_int
    lib.inkling_rel_attn_decode.argtypes = [P, P, P, P, P, P, I32, F32, I32, P,
                                            ctypes.c_size_t, P, DP, P]
    lib.inkling_rel_attn_decode_append.restype = ctypes.c_int
    lib.inkling_rel_attn_decode_append.argtypes = [P, P, P, P, P, P, P, P, I32, F32, I32, P,
                                                   ctypes.c_size_t, P, DP, P]
    lib.inkling_rel_attn_decode_noalloc.restype = ctypes.c_int
    lib.inkling_rel_attn_decode_noalloc.argtypes = [P, P, P, P, P, P, I32, F32, I32, P, DP, P]
    lib.inkling_rel_attn_num_splits.restype = I32
    lib.inkling_rel_attn_num_splits.argtypes = [DP, I32, I32]
    lib.inkling_rel_attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.inkling_rel_attn_decode_workspace_bytes.argtypes = [DP, I32, I32]
    lib.inkling_rel_attn_check_device.restype = ctypes.c_int
    lib.inkling_rel_attn_check_device.argtypes = [I32, ctypes.c_char_p, ctypes.c_size_t]
    lib.inkling_rel_attn_status_string.restype = ctypes.c_char_p
    lib.inkling_rel_attn_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().inkling_rel_attn_status_string(int(status)).decode()


def check_device(device: int = 0) -> tuple[int, str]:
    buf = ctypes.create_string_buffer(512)
    st = load().inkling_rel_attn_check_device(int(device), buf, len(buf))
    return st, buf.value.decode()


def make_dims(*, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
              max_blocks_per_seq, rel_len, total_q, max_q_len, max_seq_len,
              dtype, block_size=16) -> Dims:
    return Dims(num_seqs=num_seqs, num_q_heads=num_q_heads,
                num_kv_heads=num_kv_heads, head_dim=head_dim,
                block_size=block_size, num_blocks=num_blocks,
                max_blocks_per_seq=max_blocks_per_seq, rel_len=rel_len,
                total_q=total_q, max_q_len=max_q_len, max_seq_len=max_seq_len,
                dtype=dtype)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dims_for(q, k_cache, block_table, rel_logits, *, num_seqs, max_q_len,
             max_seq_len) -> Dims:
    total_q, hq, d = q.shape
    num_blocks, bs, hkv, _ = k_cache.shape
    return make_dims(num_seqs=num_seqs, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=d, block_size=bs, num_blocks=num_blocks,
                     max_blocks_per_seq=block_table.shape[1],
                     rel_len=rel_logits.shape[-1], total_q=total_q,
                     max_q_len=max_q_len, max_seq_len=max_seq_len,
                     dtype=_dtype_code(q))


def prefill(q, k_cache, v_cache, block_table, seq_lens, cu_q_lens, rel_logits,
            window: int, scale: float, out, *, max_q_len: int,
            max_seq_len: int, stream=None) -> None:
    """inkling_rel_attn_prefill on device tensors (see the C header)."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=max_q_len,
                    max_seq_len=max_seq_len)
    st = load().inkling_rel_attn_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(cu_q_lens), _ptr(rel_logits), int(window),
        float(scale), _ptr(out), ctypes.byref(dims), _stream(stream))
    if st != OK:
        raise InklingError(st, "inkling_rel_attn_prefill")


def prefill_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, cu_q_lens,
                   rel_logits, window: int, scale: float, out, *, max_q_len: int,
                   max_seq_len: int, stream=None) -> None:
    """inkling_rel_attn_prefill_append on device tensors: prefill that also
    stores the new tokens' k_new / v_new rows ([total_q, Hkv, D])."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=max_q_len,
                    max_seq_len=max_seq_len)
    st = load().inkling_rel_attn_prefill_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(cu_q_lens), _ptr(rel_logits),
        int(window), float(scale), _ptr(out), ctypes.byref(dims), _stream(stream))
    if st != OK:
        raise InklingError(st, "inkling_rel_attn_prefill_append")


def num_splits(dims: Dims, window: int, device: int = 0) -> int:
    return int(load().inkling_rel_attn_num_splits(ctypes.byref(dims), int(window),
                                                  int(device)))


def decode_workspace_bytes(dims: Dims, window: int, splits: int) -> int:
    return int(load().inkling_rel_attn_decode_workspace_bytes(
        ctypes.byref(dims), int(window), int(splits)))


def decode(q, k_cache, v_cache, block_table, seq_lens, rel_logits,
           window: int, scale: float, out, *, max_seq_len: int,
           num_splits: int = 0, workspace=None, stream=None) -> None:
    """inkling_rel_attn_decode on device tensors.  If `workspace` is None a
    torch buffer of the required size is allocated here (torch owns device
    memory; the library never allocates)."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=1,
                    max_seq_len=max_seq_len)
    need = decode_workspace_bytes(dims, window, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().inkling_rel_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(rel_logits), int(window), float(scale),
        int(num_splits), _ptr(workspace), ws_bytes, _ptr(out),
        ctypes.byref(dims), _stream(stream))
    if st != OK:
        raise InklingError(st, "inkling_rel_attn_decode")


def decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, rel_logits,
                   window: int, scale: float, out, *, max_seq_len: int,
                   num_splits: int = 0, stream=None) -> None:
    """inkling_rel_attn_decode_noalloc on device tensors: the same decode
    with the library's own per-GPU split buffer (no workspace argument)."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=1,
                    max_seq_len=max_seq_len)
    st = load().inkling_rel_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(rel_logits), int(window), float(scale),
        int(num_splits), _ptr(out), ctypes.byref(dims), _stream(stream))
    if st != OK:
        raise InklingError(st, "inkling_rel_attn_decode_noalloc")


def decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                  rel_logits, window: int, scale: float, out, *, max_seq_len: int,
                  num_splits: int = 0, workspace=None, stream=None) -> None:
    """inkling_rel_attn_decode_append on device tensors: decode that also
    stores k_new / v_new ([B, Hkv, D]) at key L_b - 1 of each sequence."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=1,
                    max_seq_len=max_seq_len)
    need = decode_workspace_bytes(dims, window, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().inkling_rel_attn_decode_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(rel_logits), int(window),
        float(scale), int(num_splits), _ptr(workspace), ws_bytes, _ptr(out),
        ctypes.byref(dims), _stream(stream))
    if st != OK:
        raise InklingError(st, "inkling_rel_attn_decode_append")


# --- pre-marshalled calls (for timing loops: no per-call Python work) -----

def prefill_args(q, k_cache, v_cache, block_table, seq_lens, cu_q_lens,
                 rel_logits, window, scale, out, *, max_q_len, max_seq_len,
                 stream=None):
    """Argument tuple for inkling_rel_attn_prefill; keeps `dims` alive."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=max_q_len,
                    max_seq_len=max_seq_len)
    return (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(cu_q_lens), _ptr(rel_logits), int(window),
            float(scale), _ptr(out), ctypes.byref(dims), _stream(stream)), dims


def decode_args(q, k_cache, v_cache, block_table, seq_lens, rel_logits,
                window, scale, out, *, max_seq_len, num_splits, workspace,
                stream=None):
    """Argument tuple for inkling_rel_attn_decode; keeps `dims` alive."""
    dims = dims_for(q, k_cache, block_table, rel_logits,
                    num_seqs=seq_lens.shape[0], max_q_len=1,
                    max_seq_len=max_seq_len)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(rel_logits), int(window), float(scale),
            int(num_splits), _ptr(workspace), ws_bytes, _ptr(out),
            ctypes.byref(dims), _stream(stream)), dims


def call(fn_name: str, args) -> None:
    st = getattr(load(), fn_name)(*args)
    if st != OK:
        raise InklingError(st, fn_name)
