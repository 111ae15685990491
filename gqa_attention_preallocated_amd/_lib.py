"""ctypes loader for libgqakv.so and the signatures of its C ABI (include/gqa_kv.h).

Only argument marshalling lives here. Loading fails loudly when the library
has not been built: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgqakv.so")

KV_OK = 0
KV_ERR_INVALID_ARG = 1
KV_ERR_CAPACITY = 2
KV_ERR_UNSUPPORTED = 3
KV_ERR_WORKSPACE = 4
KV_ERR_DEVICE = 5

KV_DTYPE_F32 = 0
KV_DTYPE_BF16 = 1

EXPORTED = (
    "kv_cache_create", "kv_cache_destroy", "kv_append", "gqa_attention_workspace_size",
    "gqa_attention", "kv_truncate", "kv_get_lens", "kv_cache_bytes", "kv_live_bytes",
    "kv_last_error", "kv_cache_set_policy", "kv_cache_create_ring", "kv_cache_create_fp8",
    "gqa_attention_tree", "kv_cache_create_paged", "kv_get_block_table", "kv_free_pages",
    "kv_append_attention", "kv_append_attention_workspace_size", "kv_append_attention_tree",
    "kv_append_attention_noalloc",
)

_lib = None


def load():
    """Load the built library once (after torch, so one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m gqa_attention_preallocated_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    import torch  # noqa: F401  (loads the HIP runtime torch was built with)
    _lib = configure(ctypes.CDLL(LIB_PATH))
    return _lib


def configure(lib):
    """Declare the C signatures of include/gqa_kv.h on a loaded library; returns it."""
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.kv_cache_create.argtypes = [I32, I32, I32, I32, ctypes.c_int, P, P, P, P, ctypes.POINTER(P)]
    lib.kv_cache_create.restype = ctypes.c_int
    lib.kv_cache_create_ring.argtypes = [I32, I32, I32, I32, ctypes.c_int, I32, P, P, P, P, ctypes.POINTER(P)]
    lib.kv_cache_create_ring.restype = ctypes.c_int
    FP = ctypes.POINTER(ctypes.c_float)
    lib.kv_cache_create_fp8.argtypes = [I32, I32, I32, I32, FP, FP, P, P, P, P, ctypes.POINTER(P)]
    lib.kv_cache_create_fp8.restype = ctypes.c_int
    lib.kv_cache_create_paged.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.c_int, P, P, P, P, P,
                                          ctypes.POINTER(P)]
    lib.kv_cache_create_paged.restype = ctypes.c_int
    lib.kv_get_block_table.argtypes = [P, I32P]
    lib.kv_get_block_table.restype = ctypes.c_int
    lib.kv_free_pages.argtypes = [P]
    lib.kv_free_pages.restype = I32
    lib.kv_cache_destroy.argtypes = [P]
    lib.kv_cache_destroy.restype = ctypes.c_int
    lib.kv_append.argtypes = [P, P, P, I32, I32P, P]
    lib.kv_append.restype = ctypes.c_int
    lib.gqa_attention_workspace_size.argtypes = [P, I32, I32, I32P, ctypes.POINTER(ctypes.c_size_t)]
    lib.gqa_attention_workspace_size.restype = ctypes.c_int
    lib.gqa_attention.argtypes = [P, P, I32, I32, I32P, P, P, ctypes.c_size_t, P]
    lib.gqa_attention.restype = ctypes.c_int
    lib.gqa_attention_tree.argtypes = [P, P, I32, I32, I32P, I32P, P, P, ctypes.c_size_t, P]
    lib.gqa_attention_tree.restype = ctypes.c_int
    lib.kv_append_attention.argtypes = [P, P, P, P, I32, I32, I32P, P, P, ctypes.c_size_t, P]
    lib.kv_append_attention.restype = ctypes.c_int
    lib.kv_append_attention_noalloc.argtypes = [P, P, P, P, I32, I32, I32P, P, P]
    lib.kv_append_attention_noalloc.restype = ctypes.c_int
    lib.kv_append_attention_tree.argtypes = [P, P, P, P, I32, I32, I32P, I32P, P, P, ctypes.c_size_t, P]
    lib.kv_append_attention_tree.restype = ctypes.c_int
    lib.kv_append_attention_workspace_size.argtypes = [P, I32, I32, I32P, ctypes.POINTER(ctypes.c_size_t)]
    lib.kv_append_attention_workspace_size.restype = ctypes.c_int
    lib.kv_truncate.argtypes = [P, I32P, P]
    lib.kv_truncate.restype = ctypes.c_int
    lib.kv_get_lens.argtypes = [P, I32P]
    lib.kv_get_lens.restype = ctypes.c_int
    lib.kv_cache_bytes.argtypes = [P]
    lib.kv_cache_bytes.restype = ctypes.c_uint64
    lib.kv_live_bytes.argtypes = [P]
    lib.kv_live_bytes.restype = ctypes.c_uint64
    lib.kv_last_error.argtypes = []
    lib.kv_last_error.restype = ctypes.c_char_p
    lib.kv_cache_set_policy.argtypes = [P, I32, I32]
    lib.kv_cache_set_policy.restype = ctypes.c_int
    return lib


def int32_array(values):
    """Host int32 array for an ABI call (values: any iterable of ints)."""
    vals = [int(x) for x in values]
    arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    return arr


def check(status, lib=None):
    """Map a kv_status to a Python exception."""
    if status == KV_OK:
        return
    lib = lib or load()
    msg = (lib.kv_last_error() or b"").decode()
    if status in (KV_ERR_INVALID_ARG, KV_ERR_CAPACITY, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE):
        raise ValueError(msg)
    raise RuntimeError(msg or f"kv_status {status}")
