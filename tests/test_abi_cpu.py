"""The C ABI loads, exports what its header declares, and validates host
arguments without touching a device (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

from paged_relative_bias_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "inkling_rel_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="library not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(inkling_rel_attn_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert set(_declared()) == set(B.SYMBOLS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def _dims(**kw):
    base = dict(num_seqs=2, num_q_heads=48, num_kv_heads=16, head_dim=128,
                num_blocks=100, max_blocks_per_seq=512, rel_len=512,
                total_q=2, max_q_len=1, max_seq_len=8192, dtype=B.DTYPE_BF16)
    base.update(kw)
    return B.make_dims(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _prefill(dims, window=512, scale=0.088, ptr=FAKE, out=FAKE):
    return B.load().inkling_rel_attn_prefill(ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                             window, scale, out,
                                             ctypes.byref(dims) if dims else None,
                                             None)


def _decode(dims, splits=1, ws=None, ws_bytes=0, scale=0.088, ptr=FAKE):
    return B.load().inkling_rel_attn_decode(ptr, ptr, ptr, ptr, ptr, ptr, 512,
                                            scale, splits, ws, ws_bytes, ptr,
                                            ctypes.byref(dims) if dims else None,
                                            None)


INVALID, UNSUP = 1, 2


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=48, num_kv_heads=7), INVALID),       # Hq % Hkv
    (dict(head_dim=96), UNSUP),
    (dict(block_size=8), UNSUP),
    (dict(dtype=7), UNSUP),
    (dict(rel_len=12), UNSUP),                              # 24 B rows
    (dict(num_q_heads=34, num_kv_heads=2), UNSUP),          # G = 17 > 16
    (dict(num_seqs=-1), INVALID),
    (dict(num_blocks=0), INVALID),
    (dict(max_blocks_per_seq=4), INVALID),                  # 64 keys < 8192
    (dict(max_q_len=9000), INVALID),                        # > max_seq_len
    (dict(num_seqs=70000, total_q=70000), UNSUP),           # grid limit
])
def test_bad_shapes_are_rejected_before_launch(kw, status):
    assert _prefill(_dims(**kw)) == status
    assert _decode(_dims(**kw)) == status


def test_null_and_nonfinite_arguments():
    assert _prefill(None) == INVALID
    assert _decode(None) == INVALID
    assert _prefill(_dims(), ptr=None) == INVALID
    assert _decode(_dims(), ptr=None) == INVALID
    assert _prefill(_dims(), scale=float("nan")) == INVALID
    assert _decode(_dims(), scale=float("inf")) == INVALID


def test_empty_batch_is_a_no_op():
    assert _prefill(_dims(num_seqs=0, total_q=0), ptr=None, out=None) == B.OK
    assert _decode(_dims(num_seqs=0, total_q=0), ptr=None) == B.OK


def test_decode_specific_checks():
    assert _decode(_dims(total_q=3)) == INVALID       # one row per sequence
    assert _decode(_dims(), splits=129) == INVALID
    assert _decode(_dims(), splits=-1) == INVALID
    assert _decode(_dims(), splits=8, ws=None) == 5   # workspace too small
    need = B.decode_workspace_bytes(_dims(), 512, 8)
    assert _decode(_dims(), splits=8, ws=ctypes.c_void_p(0x1000),
                   ws_bytes=need - 1) == 5
    assert _decode(_dims(), splits=8, ws=ctypes.c_void_p(0x1004),
                   ws_bytes=need) == INVALID          # misaligned


def test_workspace_size_formula():
    d = _dims(num_seqs=32, total_q=32, num_kv_heads=8)
    assert B.decode_workspace_bytes(d, 0, 1) == 0
    o = 8 * 32 * 48 * 128 * 4
    assert B.decode_workspace_bytes(d, 0, 8) == ((o + 255) // 256) * 256 + 8 * 32 * 48 * 4
    assert B.decode_workspace_bytes(d, 0, 129) == 0


def test_misaligned_tensor_is_rejected():
    d = _dims(num_seqs=2, total_q=2)
    odd = ctypes.c_void_p(0x1002)
    st = B.load().inkling_rel_attn_prefill(odd, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 512, 0.1,
                                           FAKE, ctypes.byref(d), None)
    assert st == 1   # INKLING_ERR_INVALID_ARGUMENT
    st = B.load().inkling_rel_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 512, 0.1, 1, None,
                                          0, odd, ctypes.byref(d), None)
    assert st == 1


def test_decode_append_needs_new_rows():
    # Rejected before any device work: null k_new / v_new.
    d = _dims(num_seqs=4, total_q=4)
    st = B.load().inkling_rel_attn_decode_append(
        None, None, None, None, None, None, None, None, 512, 1.0, 1, None, 0, None,
        ctypes.byref(d), None)
    assert st == 1   # INKLING_ERR_INVALID_ARGUMENT


def test_prefill_append_needs_new_rows():
    d = _dims(num_seqs=2, total_q=100, max_q_len=50)
    st = B.load().inkling_rel_attn_prefill_append(
        None, None, None, None, None, None, None, None, None, 512, 1.0, None,
        ctypes.byref(d), None)
    assert st == 1   # INKLING_ERR_INVALID_ARGUMENT


def test_split_heuristic_bounds():
    # 64 x 16 units already give four per compute unit on 256 CUs.
    assert B.num_splits(_dims(num_seqs=64, total_q=64), 512, -1) == 1
    # 32 x 8 global units: split to about two workgroups per CU.
    g = _dims(num_seqs=32, total_q=32, num_kv_heads=8)
    s = B.num_splits(g, 0, -1)
    assert 2 <= s <= 32
    one = _dims(num_seqs=1, total_q=1, num_kv_heads=1, num_q_heads=1)
    assert B.num_splits(one, 0, -1) == 32       # 8192 keys / 256 per split
    assert B.load().inkling_rel_attn_num_splits(None, 0, -1) == 1
    # A lone 512-key window (17 tiles) on an empty GPU: down to ~2 tiles
    # per split.
    assert B.num_splits(_dims(num_seqs=1, total_q=1), 512, -1) == 8
    assert B.num_splits(_dims(num_seqs=16, total_q=16), 512, -1) == 4


def test_status_strings_and_device_check_without_gpu():
    for s in range(7):
        assert isinstance(B.status_string(s), str) and B.status_string(s)
    st, msg = B.check_device(0)
    # In a container without a GPU the check reports it; on a gfx950 box it
    # passes.  Either way it returns a status and a message.
    assert st in (B.OK, 3, 4) and msg


def test_noalloc_rejects_oversized_split_workspace_without_a_device():
    """The no-allocation decode refuses, before touching any device, a call
    whose split partials would not fit the library's 32 MiB buffer."""
    d = _dims(num_seqs=64, total_q=64, num_kv_heads=8, rel_len=8192)
    st = B.load().inkling_rel_attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.088,
                                                  128, FAKE, ctypes.byref(d), None)
    assert st == 5   # INKLING_ERR_WORKSPACE_TOO_SMALL
    assert B.decode_workspace_bytes(d, 0, 128) > 32 << 20
    assert B.decode_workspace_bytes(d, 0, 8) <= 32 << 20
