"""Grouped-query attention over a contiguous, preallocated KV cache on MI355X.

Thin Python layer over the C ABI of ``libgqakv.so`` (include/gqa_kv.h): torch
provides device memory and the current stream; every step of the path runs in
the library's HIP kernels.

    cache = KVCache(batch, kv_heads, max_len, head_dim, dtype=torch.bfloat16)
    cache.append(k_new, v_new, n_new)          # in place at each row's length
    out = gqa_attention(q, cache, n_new)       # decode, verify or chunked prefill
    cache.truncate(new_lens)                   # rollback without copying

Follows "Implement grouped-query attention over a preallocated KV cache, with
no torch.cat, for both prefill chunks and decode" (inferenceinterviews.com,
"A strong answer") and the cache of "16. Prefill, decode and the KV cache"
(inference.shantanugoel.com, "Layout and validity").
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = ["KVCache", "gqa_attention", "append_attention", "append_attention_noalloc", "library_path"]

_DTYPES = {torch.float32: _lib.KV_DTYPE_F32, torch.bfloat16: _lib.KV_DTYPE_BF16}


def library_path():
    return _lib.LIB_PATH


def _stream_ptr(index=None):
    """The current HIP stream of device `index` (default: the current device)."""
    if index is None:
        index = torch.cuda.current_device()
    return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(index))


def _row_counts(n_new, batch):
    if isinstance(n_new, torch.Tensor):
        vals = n_new.detach().to("cpu").tolist()
    elif isinstance(n_new, int):
        vals = [n_new] * batch
    else:
        vals = [int(x) for x in n_new]
    if len(vals) != batch:
        raise ValueError(f"n_new has {len(vals)} entries for {batch} rows")
    return vals


class KVCache:
    """K and V [B, Hkv, max_len, d] allocated once on the GPU, plus per-row lengths.

    ``k`` and ``v`` are the preallocated buffers themselves (their data
    pointers never change); ``lens`` is the host copy of the per-row lengths and
    ``lens_dev`` the device copy the library keeps in stream order (None with
    ``device_lens=False``: then a rollback is host-only bookkeeping).

    With ``window=W`` the cache is a ring of ``max_len`` slots per row (a
    multiple of 64) that keeps only the latest tokens, and attention sees the
    last W positions ([MASK] "A strong answer", the reversal); lengths are then
    absolute positions and may exceed ``max_len``.

    With ``fp8_scales=(k_scale, v_scale)`` (one float per KV head each) K and
    V are stored as E4M3 codes (``k``/``v`` are uint8 tensors) and read back
    dequantized ([CH16] exercise 4); inputs and outputs stay bfloat16.

    With ``page_size=P, num_pages=N`` the cache is paged: ``k``/``v`` are one
    pool [N, Hkv, P, d] shared by all rows, ``block_table_dev`` the device
    block table [B, max_len // P] the library keeps, and a row takes pages only
    as it grows ([GQA] reversal: a block table and a paged kernel).
    """

    def __init__(self, batch, kv_heads, max_len, head_dim, dtype=torch.bfloat16, device="cuda",
                 device_lens=True, window=None, fp8_scales=None, page_size=None, num_pages=None):
        if dtype not in _DTYPES:
            raise ValueError(f"dtype {dtype} not supported (float32 or bfloat16)")
        self._lib = _lib.load()
        device = torch.device(device)
        if device.type != "cuda":
            raise ValueError("the cache lives in GPU memory (device='cuda')")
        shape = (batch, kv_heads, max_len, head_dim)
        if fp8_scales is not None and (dtype != torch.bfloat16 or window is not None):
            raise ValueError("an E4M3 cache takes bfloat16 inputs and has no window")
        self.paged = page_size is not None
        self.page_size = self.num_pages = None
        self.max_blocks = 0
        if self.paged:
            if num_pages is None or window is not None or fp8_scales is not None:
                raise ValueError("a paged cache needs num_pages and has no window or E4M3 storage")
            if max_len % page_size != 0:
                raise ValueError("max_len must be a multiple of page_size")
            pool = (int(num_pages), kv_heads, int(page_size), head_dim)
            self.page_size, self.num_pages, self.max_blocks = int(page_size), int(num_pages), max_len // page_size
            # kv_cache_create_paged sets the pool to zero on the current stream
            self.k = torch.empty(pool, dtype=dtype, device=device)
            self.v = torch.empty(pool, dtype=dtype, device=device)
            self.block_table_dev = torch.empty((max(batch, 1), self.max_blocks), dtype=torch.int32, device=device)
        else:
            store = torch.uint8 if fp8_scales is not None else dtype
            # kv_cache_create* sets K and V to zero on the current stream
            self.k = torch.empty(shape, dtype=store, device=device)
            self.v = torch.empty(shape, dtype=store, device=device)
        self.lens_dev = torch.zeros(max(batch, 1), dtype=torch.int32, device=device) if device_lens else None
        self.dtype = dtype
        self._device = self.k.device
        self.batch, self.kv_heads, self.max_len, self.head_dim = shape
        self.window = window
        self._ws = None
        h = ctypes.c_void_p()
        bufs = (ctypes.c_void_p(self.k.data_ptr()), ctypes.c_void_p(self.v.data_ptr()),
                ctypes.c_void_p(self.lens_dev.data_ptr() if device_lens else 0))
        with torch.cuda.device(device):
            if fp8_scales is not None:
                ks, vs = ([float(x) for x in sc] for sc in fp8_scales)
                if len(ks) != kv_heads or len(vs) != kv_heads:
                    raise ValueError("fp8_scales needs one K and one V scale per KV head")
                self.fp8_scales = (ks, vs)
                st = self._lib.kv_cache_create_fp8(batch, kv_heads, max_len, head_dim,
                                                   (ctypes.c_float * max(kv_heads, 1))(*ks),
                                                   (ctypes.c_float * max(kv_heads, 1))(*vs), *bufs,
                                                   _stream_ptr(), ctypes.byref(h))
            elif self.paged:
                st = self._lib.kv_cache_create_paged(batch, kv_heads, self.num_pages, self.page_size,
                                                     self.max_blocks, head_dim, _DTYPES[dtype], *bufs[:2],
                                                     ctypes.c_void_p(self.block_table_dev.data_ptr()), bufs[2],
                                                     _stream_ptr(), ctypes.byref(h))
            elif window is None:
                st = self._lib.kv_cache_create(batch, kv_heads, max_len, head_dim, _DTYPES[dtype], *bufs,
                                               _stream_ptr(), ctypes.byref(h))
            else:
                st = self._lib.kv_cache_create_ring(batch, kv_heads, max_len, head_dim, _DTYPES[dtype],
                                                    int(window), *bufs, _stream_ptr(), ctypes.byref(h))
        _lib.check(st, self._lib)
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.kv_cache_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def device(self):
        return self._device

    @property
    def lens(self):
        arr = (ctypes.c_int32 * max(1, self.batch))()
        _lib.check(self._lib.kv_get_lens(self._h, arr), self._lib)
        return list(arr)[: self.batch]

    @property
    def block_table(self):
        """Host copy of a paged cache's block table [B][max_blocks] (-1: no page)."""
        arr = (ctypes.c_int32 * max(1, self.batch * self.max_blocks))()
        _lib.check(self._lib.kv_get_block_table(self._h, arr), self._lib)
        flat = list(arr)
        return [flat[b * self.max_blocks:(b + 1) * self.max_blocks] for b in range(self.batch)]

    @property
    def free_pages(self):
        return int(self._lib.kv_free_pages(self._h))

    @property
    def bytes(self):
        """Bytes of the reservation (all of K and V)."""
        return int(self._lib.kv_cache_bytes(self._h))

    @property
    def live_bytes(self):
        """Bytes of the valid K and V prefixes."""
        return int(self._lib.kv_live_bytes(self._h))

    def _check_tensor(self, x, name, heads):
        if not isinstance(x, torch.Tensor) or x.device != self._device or x.dtype != self.dtype:
            raise ValueError(f"{name} must be a {self.dtype} tensor on {self.device}")
        if x.dim() != 4 or x.shape[0] != self.batch or x.shape[1] != heads or x.shape[3] != self.head_dim:
            raise ValueError(f"{name} must be [B={self.batch}, {heads}, T, d={self.head_dim}], got {tuple(x.shape)}")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def append(self, k_new, v_new, n_new):
        """Write n_new[b] tokens of row b in place at its current length."""
        self._check_tensor(k_new, "k_new", self.kv_heads)
        self._check_tensor(v_new, "v_new", self.kv_heads)
        if k_new.shape != v_new.shape:
            raise ValueError("k_new and v_new differ in shape")
        n = _row_counts(n_new, self.batch)
        st = self._lib.kv_append(self._h, ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
                                 k_new.shape[2], _lib.int32_array(n), _stream_ptr(self._device.index))
        _lib.check(st, self._lib)

    def truncate(self, new_lens):
        """Roll every row back to new_lens[b] tokens (a scalar applies to all rows)."""
        if isinstance(new_lens, int):
            new_lens = [new_lens] * self.batch
        n = _row_counts(new_lens, self.batch)
        _lib.check(self._lib.kv_truncate(self._h, _lib.int32_array(n), _stream_ptr(self._device.index)), self._lib)

    def reset(self):
        self.truncate(0)

    def set_policy(self, path=0, keys_per_split=0):
        """0/1/2 = automatic / split-K decode kernel / chunked-prefill kernel."""
        _lib.check(self._lib.kv_cache_set_policy(self._h, int(path), int(keys_per_split)), self._lib)

    def workspace_bytes(self, q_heads, T, n_new):
        n = _row_counts(n_new, self.batch)
        size = ctypes.c_size_t()
        _lib.check(self._lib.gqa_attention_workspace_size(self._h, q_heads, T, _lib.int32_array(n),
                                                          ctypes.byref(size)), self._lib)
        return int(size.value)

    def _workspace(self, nbytes):
        if nbytes == 0:
            return None
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws


def gqa_attention(q, cache: KVCache, n_new, out=None, workspace=None, parents=None):
    """Attention output [B, Hq, T, d] for the n_new[b] tokens each row just appended.

    q: [B, Hq, T, d] (Hq a multiple of the cache's Hkv); padded slots
    t >= n_new[b] come back as zeros. ``workspace`` (a uint8 CUDA tensor) may be
    given to avoid the cache's own grow-once scratch buffer. With ``parents``
    ([B, T] ints: -1 or an earlier node) the new tokens are a draft tree and
    each attends the committed keys plus its ancestors ([MASK] "What
    interviewers probe next").
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B, Hq, T, d]")
    cache._check_tensor(q, "q", q.shape[1])
    B, hq, T, d = q.shape
    n = _row_counts(n_new, B)
    arr = _lib.int32_array(n)
    if out is None:
        out = torch.empty_like(q)
    else:
        cache._check_tensor(out, "out", hq)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lib = cache._lib
    if workspace is None:
        size = ctypes.c_size_t()
        _lib.check(lib.gqa_attention_workspace_size(cache.handle, hq, T, arr, ctypes.byref(size)), lib)
        ws = cache._workspace(int(size.value))
    else:
        # a caller's workspace: the library checks its size (KV_ERR_WORKSPACE)
        if workspace.device != cache.device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the cache's device")
        ws = workspace
    ws_ptr = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
    ws_len = ws.numel() if ws is not None else 0
    if parents is None:
        st = lib.gqa_attention(cache.handle, ctypes.c_void_p(q.data_ptr()), hq, T, arr,
                               ctypes.c_void_p(out.data_ptr()), ws_ptr, ws_len, _stream_ptr(cache._device.index))
    else:
        flat = [int(x) for row in (parents.tolist() if hasattr(parents, "tolist") else parents) for x in row]
        if len(flat) != B * T:
            raise ValueError(f"parents must be [B={B}, T={T}]")
        st = lib.gqa_attention_tree(cache.handle, ctypes.c_void_p(q.data_ptr()), hq, T, arr,
                                    _lib.int32_array(flat), ctypes.c_void_p(out.data_ptr()), ws_ptr, ws_len,
                                    _stream_ptr(cache._device.index))
    _lib.check(st, lib)
    return out


def append_attention(cache: KVCache, k_new, v_new, q, n_new, out=None, workspace=None, parents=None):
    """``cache.append(k_new, v_new, n_new)`` then ``gqa_attention(q, cache, n_new,
    parents=parents)`` in one library call (kv_append_attention, or
    kv_append_attention_tree with ``parents``): rows on the decode kernel are
    appended by that kernel, so a decode or verify step is one launch. Same bits
    as the two calls."""
    cache._check_tensor(k_new, "k_new", cache.kv_heads)
    cache._check_tensor(v_new, "v_new", cache.kv_heads)
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B, Hq, T, d]")
    cache._check_tensor(q, "q", q.shape[1])
    B, hq, T, d = q.shape
    if k_new.shape[2] != T:
        raise ValueError("k_new and q differ in T")
    n = _row_counts(n_new, B)
    arr = _lib.int32_array(n)
    if out is None:
        out = torch.empty_like(q)
    else:
        cache._check_tensor(out, "out", hq)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lib = cache._lib
    if workspace is None:
        size = ctypes.c_size_t()
        _lib.check(lib.kv_append_attention_workspace_size(cache.handle, hq, T, arr, ctypes.byref(size)), lib)
        ws = cache._workspace(int(size.value))
    else:
        # a caller's workspace: the library checks its size (KV_ERR_WORKSPACE)
        if workspace.device != cache.device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the cache's device")
        ws = workspace
    ptrs = (ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(q.data_ptr()))
    ws_args = (ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), ws.numel() if ws is not None else 0,
               _stream_ptr(cache._device.index))
    if parents is None:
        st = lib.kv_append_attention(cache.handle, *ptrs, hq, T, arr, ctypes.c_void_p(out.data_ptr()), *ws_args)
    else:
        flat = [int(x) for row in (parents.tolist() if hasattr(parents, "tolist") else parents) for x in row]
        if len(flat) != B * T:
            raise ValueError(f"parents must be [B={B}, T={T}]")
        st = lib.kv_append_attention_tree(cache.handle, *ptrs, hq, T, arr, _lib.int32_array(flat),
                                          ctypes.c_void_p(out.data_ptr()), *ws_args)
    _lib.check(st, lib)
    return out


def append_attention_noalloc(cache: KVCache, k_new, v_new, q, n_new, out):
    """``append_attention`` through kv_append_attention_noalloc: no workspace,
    and nothing allocated by the library or here (``out`` is the caller's).
    The split partials live in the library's scratch on the cache's device,
    shared by every such call on that GPU: calls that may overlap there race.
    Raises ValueError when the call's partials need more than that scratch."""
    cache._check_tensor(k_new, "k_new", cache.kv_heads)
    cache._check_tensor(v_new, "v_new", cache.kv_heads)
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B, Hq, T, d]")
    cache._check_tensor(q, "q", q.shape[1])
    cache._check_tensor(out, "out", q.shape[1])
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    B, hq, T, _ = q.shape
    if k_new.shape[2] != T:
        raise ValueError("k_new and q differ in T")
    arr = _lib.int32_array(_row_counts(n_new, B))
    lib = cache._lib
    with torch.cuda.device(cache.device):     # the scratch of the cache's device
        st = lib.kv_append_attention_noalloc(cache.handle, ctypes.c_void_p(k_new.data_ptr()),
                                             ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                             hq, T, arr, ctypes.c_void_p(out.data_ptr()),
                                             _stream_ptr(cache._device.index))
    _lib.check(st, lib)
    return out
