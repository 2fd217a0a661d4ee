"""The C-ABI library builds, loads and exports every entry point of include/kvattn.h,
and rejects bad arguments on the host (no GPU needed: nothing here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from kv_cache_attention_amd import binding as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvattn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KVATTN_API\s+[\w\s\*]+?\b(kvattn_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(kb.EXPORTS)
    for n in ("kvattn_create", "kvattn_decode", "kvattn_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(dtype="f16", num_q_heads=32, num_kv_heads=8, head_dim=128, max_batch=4,
                max_q_len=5, cache_mode="contiguous", capacity=4096)
    base.update(kw)
    return kb.make_config(**base)


def test_config_validation_errors():
    lib = kb.load()
    h = ctypes.c_void_p()
    assert lib.kvattn_create(None, ctypes.byref(h)) == -1
    assert kb.kvattn_last_error()
    bad = [
        (_cfg(head_dim=96), -2),
        (_cfg(num_q_heads=30, num_kv_heads=8), -1),
        (_cfg(max_q_len=1025), -2),
        (_cfg(max_batch=0), -1),
        (_cfg(capacity=0), -1),
        (_cfg(cache_mode="paged", block_size=12, num_blocks=10, capacity=96), -1),
        (_cfg(cache_mode="paged", block_size=16, num_blocks=10, capacity=100), -1),
        (_cfg(cache_mode="paged", block_size=16, num_blocks=0, capacity=96), -1),
        (_cfg(scale=-1.0), -1),
    ]
    for cfg, code in bad:
        rc = lib.kvattn_create(ctypes.byref(cfg), ctypes.byref(h))
        assert rc == code, (rc, code, kb.kvattn_last_error())
        assert not h.value
    cfg = _cfg()
    cfg.dtype = 7
    assert lib.kvattn_create(ctypes.byref(cfg), ctypes.byref(h)) == -2


def test_null_handle_is_rejected():
    lib = kb.load()
    assert lib.kvattn_decode(None, None, None, None, None, None, 1, 0, 0, 0, None) == -1
    assert lib.kvattn_set_batch(None, 1) == -1
    assert lib.kvattn_set_stream(None, None) == -1
    assert lib.kvattn_set_split_len(None, 64) == -1
    assert lib.kvattn_plan(None, 1, 0, 0, 0, None, None, None) == -1
    assert lib.kvattn_check(None) == -1
    lib.kvattn_destroy(None)  # no-op


def test_flags_are_validated():
    lib = kb.load()
    h = ctypes.c_void_p()
    cfg = _cfg()
    cfg.flags = 4  # no such flag
    assert lib.kvattn_create(ctypes.byref(cfg), ctypes.byref(h)) == -1
    assert not h.value
    # the debug flag is known (creation itself needs a device, checked on the GPU)
    assert kb.kvattn_workspace_bytes(_cfg(debug=True, deterministic=True)) > 0


def test_workspace_bytes_is_host_only_and_bounded():
    n = kb.kvattn_workspace_bytes(_cfg())
    assert n > 0
    # the partials stay a small fraction of the cache they summarise
    cache = 4 * 4096 * 8 * 128 * 2 * 2
    assert n < cache
    with pytest.raises(kb.KVAttnError):
        kb.kvattn_workspace_bytes(_cfg(head_dim=80))
