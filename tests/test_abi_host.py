"""The C-ABI library loads and exports every entry point include/gqa_kv.h declares,
and its host-side validation behaves as documented.

Calls that fail validation enqueue nothing, so they run on the built library
itself. Calls that succeed enqueue kernels (creation zero-fills K and V), so
they run on the same host code (abi.cpp) linked against the CPU launch
simulator instead of the kernels (the ``hostcheck_lib`` fixture)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gqa_kv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from gqa_attention_preallocated_amd import _lib
    return _lib.load()


def test_header_declares_the_abi():
    names = _declared()
    for want in ["kv_cache_create", "kv_append", "gqa_attention", "kv_truncate"]:
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    from gqa_attention_preallocated_amd import _lib
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTED) == _declared()


@pytest.fixture(scope="module")
def host(hostcheck_lib):
    from gqa_attention_preallocated_amd import _lib
    return _lib.configure(hostcheck_lib)


def _fake_cache(lib, B=2, hk=2, max_len=64, d=16, dtype=0):
    h = ctypes.c_void_p()
    st = lib.kv_cache_create(B, hk, max_len, d, dtype, ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), None,
                             None, ctypes.byref(h))
    assert st == 0, lib.kv_last_error()
    return h


def _arr(vals):
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


def test_create_validation(lib):
    h = ctypes.c_void_p()
    bad = [
        (2, 2, 64, 24, 0, 3),       # head_dim not built
        (2, 2, 64, 16, 7, 3),       # unknown dtype
        (2, 0, 64, 16, 0, 1),       # no kv heads
        (-1, 2, 64, 16, 0, 1),
        (2, 2, 0, 16, 0, 1),
    ]
    for B, hk, S, d, dt, code in bad:
        assert lib.kv_cache_create(B, hk, S, d, dt, ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), None,
                                   None, ctypes.byref(h)) == code
    # misaligned buffer
    assert lib.kv_cache_create(2, 2, 64, 16, 0, ctypes.c_void_p((1 << 20) + 4), ctypes.c_void_p(2 << 20), None,
                               None, ctypes.byref(h)) == 1


def test_capacity_error_text_and_nothing_changes(host):
    lib = host
    h = _fake_cache(lib)
    st = lib.kv_append(h, ctypes.c_void_p(3 << 20), ctypes.c_void_p(4 << 20), 80, _arr([3, 70]), None)
    assert st == 2
    assert lib.kv_last_error().decode() == "row 1: 70 tokens > max_len 64"
    out = _arr([9, 9])
    assert lib.kv_get_lens(h, out) == 0 and list(out) == [0, 0]
    assert lib.kv_append(h, None, None, 5, _arr([6, 0]), None) == 1      # n_new > T
    assert lib.kv_append(h, None, None, 5, _arr([-1, 0]), None) == 1
    assert lib.kv_append(h, None, None, 5, _arr([0, 0]), None) == 0      # nothing to write
    lib.kv_cache_destroy(h)


def test_attention_argument_checks(host):
    lib = host
    h = _fake_cache(lib)
    size = ctypes.c_size_t()
    assert lib.gqa_attention_workspace_size(h, 3, 4, _arr([0, 0]), ctypes.byref(size)) == 1   # Hq % Hkv
    assert lib.gqa_attention_workspace_size(h, 4, 4, _arr([1, 0]), ctypes.byref(size)) == 1   # n_new > lens
    assert lib.gqa_attention_workspace_size(h, 4, 4, _arr([0, 0]), ctypes.byref(size)) == 0
    assert size.value == 0
    assert lib.gqa_attention_workspace_size(h, 2 * 129, 4, _arr([0, 0]), ctypes.byref(size)) == 3
    lib.kv_cache_destroy(h)


def test_truncate_rules_and_bytes(host):
    lib = host
    h = _fake_cache(lib, B=2, hk=2, max_len=64, d=16, dtype=1)
    assert lib.kv_cache_bytes(h) == 2 * 2 * 2 * 64 * 16 * 2
    assert lib.kv_live_bytes(h) == 0
    assert lib.kv_truncate(h, _arr([1, 0]), None) == 1
    assert lib.kv_last_error().decode() == "Invalid truncation length"
    assert lib.kv_truncate(h, _arr([0, 0]), None) == 0
    assert lib.kv_cache_set_policy(h, 3, 0) == 1
    assert lib.kv_cache_set_policy(h, 2, 64) == 0
    lib.kv_cache_destroy(h)


def test_paged_create_validation(lib, host):
    """kv_cache_create_paged refuses bad pool geometry and E4M3 storage before
    enqueueing anything; the block-table query refuses a linear cache."""
    h = ctypes.c_void_p()
    a, t = ctypes.c_void_p(1 << 20), ctypes.c_void_p(3 << 20)
    bad = [
        (64 - 16, 8, 4, 1, 1),      # page size not a power of two
        (32, 8, 4, 1, 1),           # below 64
        (1 << 17, 8, 4, 1, 1),      # above 65,536
        (64, 0, 4, 1, 1),           # no pages
        (64, 8, 0, 1, 1),           # no blocks
        (64, 8, 4, 2, 3),           # E4M3
    ]
    for P, pages, blocks, dt, code in bad:
        st = lib.kv_cache_create_paged(2, 2, pages, P, blocks, 64, dt, a, a, t, None, None, ctypes.byref(h))
        assert st == code, (P, pages, blocks, dt, lib.kv_last_error())
    st = lib.kv_cache_create_paged(2, 2, 8, 64, 4, 64, 1, a, a, ctypes.c_void_p((3 << 20) + 4), None, None,
                                   ctypes.byref(h))
    assert st == 1                  # misaligned block table
    lin = _fake_cache(host)
    assert host.kv_get_block_table(lin, _arr([0] * 8)) == 1
    assert host.kv_free_pages(lin) == 0
    assert host.kv_cache_destroy(lin) == 0
    assert host.kv_cache_destroy(None) == 0


def test_python_layer_refuses_without_gpu_buffers():
    import torch
    from gqa_attention_preallocated_amd import KVCache
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    with pytest.raises(Exception):
        KVCache(1, 1, 8, 16, device="cpu")
