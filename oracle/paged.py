"""Paged KV cache with a block table: the CPU reference.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/ and
``__graft_entry__.smoke()``.

Sources: [GQA] "Implement grouped-query attention over a preallocated KV cache,
with no torch.cat, for both prefill chunks and decode" (inferenceinterviews.com),
"A strong answer" (reserving max_len per row is the waste paged caches remove)
and its reversal paragraph (when row lengths differ by orders of magnitude, the
dense reservation mostly holds nothing, and a per-row table of pages read by
a page-aware kernel is the better layout); [CH16] "16. Prefill, decode and the KV cache", design choices
(a paged cache keeps the O(1) write without reserving the maximum up front).

Readings taken where the pages are silent (each listed in the design notes):
  * One pool of pages shared by all rows, laid out [num_pages, Hkv, P, d];
    logical block i of row b (tokens i*P .. i*P+P-1) lives in the page
    block_table[b][i].
  * A row gets pages as it grows; a call first checks that every row can get
    the pages it needs (else nothing changes), then hands them out row by row,
    each time the lowest-numbered free page. A rollback returns the pages that
    no longer hold a token; they are free for any row.
  * Attention is the plain definition over the row's logical sequence (keys
    0 .. len-1 gathered through the block table): paging changes where bytes
    live, never which keys a query sees.
"""

from __future__ import annotations

import heapq

import numpy as np

from .direct import _STORAGE, attention_row


class PagedCache:
    def __init__(self, batch, kv_heads, num_pages, page_size, max_blocks, head_dim, dtype="f32"):
        np_t, self.elem_bytes = _STORAGE[dtype]
        self.dtype = dtype
        self.k = np.zeros((num_pages, kv_heads, page_size, head_dim), np_t)
        self.v = np.zeros_like(self.k)
        self.page_size = page_size
        self.max_blocks = max_blocks
        self.table = np.full((batch, max_blocks), -1, np.int64)
        self.lens = np.zeros(batch, np.int64)
        self.free = list(range(num_pages))
        heapq.heapify(self.free)

    @property
    def batch(self):
        return self.table.shape[0]

    @property
    def kv_heads(self):
        return self.k.shape[1]

    @property
    def head_dim(self):
        return self.k.shape[3]

    def blocks(self, length):
        return -(-int(length) // self.page_size)

    def append(self, k_new, v_new, n_new):
        """Write n_new[b] tokens of row b at its length, taking pages as needed."""
        B = self.batch
        T = k_new.shape[2]
        n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
        need = 0
        for b in range(B):
            n = int(n_new[b])
            if n < 0 or n > T:
                raise ValueError(f"row {b}: n_new {n} outside 0..{T}")
            nb = self.blocks(self.lens[b] + n)
            if nb > self.max_blocks:
                raise ValueError(f"row {b}: {int(self.lens[b]) + n} tokens > {self.max_blocks} blocks "
                                 f"of {self.page_size}")
            need += nb - self.blocks(self.lens[b])
        if need > len(self.free):
            raise ValueError(f"{need} pages needed, {len(self.free)} free")
        for b in range(B):
            for i in range(self.blocks(self.lens[b]), self.blocks(self.lens[b] + n_new[b])):
                self.table[b, i] = heapq.heappop(self.free)
        for b in range(B):
            s = int(self.lens[b])
            for t in range(int(n_new[b])):
                p = s + t
                page, off = self.table[b, p // self.page_size], p % self.page_size
                self.k[page, :, off] = k_new[b, :, t]
                self.v[page, :, off] = v_new[b, :, t]
        self.lens += n_new

    def truncate(self, new_lens):
        new = np.broadcast_to(np.asarray(new_lens, dtype=np.int64), self.lens.shape)
        if np.any(new < 0) or np.any(new > self.lens):
            raise ValueError("Invalid truncation length")
        for b in range(self.batch):
            for i in range(self.blocks(new[b]), self.blocks(self.lens[b])):
                heapq.heappush(self.free, int(self.table[b, i]))
                self.table[b, i] = -1
        self.lens = new.copy()

    def gather(self, b):
        """Row b's logical K and V [Hkv, len, d] (stored values) through the block table."""
        L = int(self.lens[b])
        pages = [int(self.table[b, i]) for i in range(self.blocks(L))]
        if not pages:
            empty = np.zeros((self.kv_heads, 0, self.head_dim), self.k.dtype)
            return empty, empty
        k = np.concatenate([self.k[p] for p in pages], axis=1)[:, :L]
        v = np.concatenate([self.v[p] for p in pages], axis=1)[:, :L]
        return k, v


def attention(cache: PagedCache, q, n_new):
    """Output [B, Hq, T, d] (float64): the plain definition over each row's
    gathered keys ([GQA] "A strong answer")."""
    q = np.asarray(q)
    B, hq, T, d = q.shape
    n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
    out = np.zeros((B, hq, T, d), np.float64)
    for b in range(B):
        L, n = int(cache.lens[b]), int(n_new[b])
        if n < 0 or n > T or n > L:
            raise ValueError(f"row {b}: bad n_new {n}")
        if n == 0:
            continue
        k, v = cache.gather(b)
        out[b] = attention_row(k, v, L, n, q[b], cache.dtype, [(h, t) for h in range(hq) for t in range(T)])
    return out
