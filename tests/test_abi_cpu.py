"""The C-ABI library loads and exports every entry point include/ds4moe.h
declares; argument validation returns errors without touching a GPU."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "ds4moe.h"


def declared_symbols():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(ds4moe_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import bit_quantized_moe_renorm_amd as m
    if not m.LIB_PATH.exists():
        from bit_quantized_moe_renorm_amd import build
        build.build()
    return m.load_library()


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("ds4moe_create", "ds4moe_route", "ds4moe_forward", "ds4moe_destroy", "ds4moe_last_error"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    import bit_quantized_moe_renorm_amd as m
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert sorted(m.SYMBOLS) == declared_symbols()


def test_validation_without_gpu(lib):
    import bit_quantized_moe_renorm_amd as m
    h = ctypes.c_void_p()
    # NULL description
    assert lib.ds4moe_create(None, None, ctypes.byref(h)) == m.EINVAL
    # bad sizes: n_embd not a supported power of two
    d = m.Desc(m.ABI_VERSION, 300, 256, 8, 2, 0, 4, m.BF16, 1, None, 1, 1, 1, 1, None, None, None, 0, None, 0, 0)
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    assert b"n_embd" in lib.ds4moe_last_error()
    # top_k > n_expert
    d = m.Desc(m.ABI_VERSION, 256, 256, 4, 6, 0, 4, m.BF16, 1, None, 1, 1, 1, 1, None, None, None, 0, None, 0, 0)
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    # wrong ABI version
    d = m.Desc(99, 256, 256, 8, 2, 0, 4, m.BF16, 1, None, 1, 1, 1, 1, None, None, None, 0, None, 0, 0)
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    # unknown expert format
    d = m.Desc(m.ABI_VERSION, 256, 256, 8, 2, 0, 4, m.BF16, 1, None, 1, 1, 1, 1, None, None, None, 7, None, 0, 0)
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    assert b"expert_format" in lib.ds4moe_last_error()
    # shared expert requested but missing
    d = m.Desc(m.ABI_VERSION, 256, 256, 8, 2, 1, 4, m.BF16, 1, None, 1, 1, 1, 1, None, None, None, 0, None, 0, 0)
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    # NULL handle on every per-handle entry point
    assert lib.ds4moe_forward(None, None, 1, None, None) == m.EINVAL
    assert lib.ds4moe_route(None, None, 1, None, None, None, None, None) == m.EINVAL
    assert lib.ds4moe_set_path(None, 0) == m.EINVAL
    assert lib.ds4moe_dequantize(None, 0, 0, None, None) == m.EINVAL
    assert lib.ds4moe_timing_enable(None, 1) == m.EINVAL
    assert lib.ds4moe_destroy(None) == m.OK
    # rmsnorm argument checks; n_tok == 0 is a no-op
    assert lib.ds4moe_rmsnorm(None, -1, 16, 1e-6, None, None) == m.EINVAL
    assert lib.ds4moe_rmsnorm(None, 1, 0, 1e-6, None, None) == m.EINVAL
    assert lib.ds4moe_rmsnorm(None, 0, 16, 1e-6, None, None) == m.OK
    # forward_stack: no layers, a NULL layer handle, bad eps
    assert lib.ds4moe_forward_stack(None, 1, None, 1, 1e-6, None, None) == m.EINVAL
    one_null = (ctypes.c_void_p * 1)(None)
    assert lib.ds4moe_forward_stack(one_null, 0, None, 1, 1e-6, None, None) == m.EINVAL
    assert lib.ds4moe_forward_stack(one_null, 1, 256, 1, 1e-6, 256, None) == m.EINVAL
    assert b"layer 0" in lib.ds4moe_last_error()
    assert lib.ds4moe_forward_stack(one_null, 1, 256, 1, -1.0, 256, None) == m.EINVAL
    # misaligned h or x (the kernels load 16 bytes at a time)
    assert lib.ds4moe_forward_stack(one_null, 1, 258, 1, 1e-6, 256, None) == m.EINVAL
    assert b"aligned" in lib.ds4moe_last_error()
    assert lib.ds4moe_forward_stack(one_null, 1, 256, 1, 1e-6, 264, None) == m.EINVAL
    assert b"aligned" in lib.ds4moe_last_error()
    # the newer per-handle entry points reject a NULL handle too
    assert lib.ds4moe_last_routing(None, 1, None, None, None, None, None) == m.EINVAL
    assert lib.ds4moe_status(None) == m.EINVAL
    assert lib.ds4moe_set_wait_limit(None, 4, 1) == m.EINVAL
    assert lib.ds4moe_forward_ids(None, None, None, 1, None, None) == m.EINVAL
    assert lib.ds4moe_route_ids(None, None, None, 1, None, None, None, None, None) == m.EINVAL
    assert lib.ds4moe_forward_stack_ids(None, 1, None, None, 1, 1e-6, None, None) == m.EINVAL
    assert lib.ds4moe_forward_stack_ids(one_null, 1, 256, 256, 1, 1e-6, 256, None) == m.EINVAL
    assert b"layer 0" in lib.ds4moe_last_error()
    # a hash table needs 1 <= n_vocab <= INT32_MAX / top_k and 4-byte alignment
    d = m.Desc(m.ABI_VERSION, 256, 256, 8, 2, 0, 4, m.BF16, 256, None, 256, 256, 256, 256, None, None, None, 0, 256, 0, 0)
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    assert b"n_vocab" in lib.ds4moe_last_error()
    d.n_vocab = 2 ** 31
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    d.n_vocab, d.hash_table = 1000, 258
    assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
    assert b"hash_table" in lib.ds4moe_last_error()
    # expert cache slots: 0, or top_k..n_expert
    d.hash_table, d.n_vocab = None, 0
    for slots in (-1, 1, 9):
        d.expert_cache_slots = slots
        assert lib.ds4moe_create(ctypes.byref(d), None, ctypes.byref(h)) == m.EINVAL
        assert b"expert_cache_slots" in lib.ds4moe_last_error()
    v = (ctypes.c_int64 * 4)()
    assert lib.ds4moe_cache_stats(None, v, None) == m.EINVAL
    assert lib.ds4moe_cache_slots(None, None, None) == m.EINVAL


def test_binding_has_no_fallback(tmp_path):
    """Without the built library the binding raises instead of computing anything."""
    import bit_quantized_moe_renorm_amd as m
    with pytest.raises(RuntimeError):
        m.load_library(tmp_path / "missing.so")
