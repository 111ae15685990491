"""Sliding-window attention over a ring-buffer KV cache: the CPU reference.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/ and
``__graft_entry__.smoke()``.

Sources (titles of the pages; sections named in each docstring):
  [MASK]  "Write the causal mask for a decode step with a KV cache, where the
          query is shorter than the keys" (inferenceinterviews.com), "A strong
          answer" (the reversal paragraph) and "Common mistakes".
  [CH16]  "16. Prefill, decode and the KV cache" (inference.shantanugoel.com),
          the exercise on a cache that keeps only the last w positions in a
          ring buffer.

What the pages fix: with a window W the causal rule gains a lower bound, so a
query at absolute position p sees key j exactly when p - W < j <= p; the cache
may be a ring buffer whose slot index is not the token's position, so the
comparison must use the positions stored with the tokens, never slot indices.

Readings taken where the pages are silent (each listed in the design notes):
  * Token p of a row lives in slot p mod C of a C-slot ring; the row's length
    counts every token ever appended (its next absolute position).
  * Each slot stores the absolute position of the token it holds (-1 while
    empty), and visibility is decided on that stored position.
  * An append may not overwrite a key that one of its own new queries still
    needs: after the write the oldest position kept must not exceed the
    lowest key the first new query sees.
  * A rollback to n' is valid when 0 <= n' <= length and the keys the next
    query at position n' would need (from n' - W + 1 on) are still held.

Arithmetic is float64; stored values are widened exactly (``direct.to_float64``).
"""

from __future__ import annotations

import numpy as np

from .direct import _STORAGE, attend_one, kv_head_of, query_position, to_float64


def window_visible(j, pos, length, window):
    """Key at absolute position j is visible to a query at absolute position pos.

    [MASK] "A strong answer": causality j <= pos plus the window's lower bound
    j > pos - W; j < length keeps stale slots (rolled-back tokens) out; j >= 0
    excludes slots that were never written. Works on scalars and numpy arrays.
    """
    return (j >= 0) & (j <= pos) & (j > pos - window) & (j < length)


class RingCache:
    """K and V as [B, Hkv, C, d] rings plus the stored position of every slot.

    [CH16] exercise 3: the cache keeps only the last positions in a ring
    buffer. ``lens[b]`` is row b's absolute length (its next position);
    ``pos[b, s]`` is the position held by slot s (-1 if never written).
    """

    def __init__(self, batch, kv_heads, capacity, head_dim, window, dtype="f32"):
        if dtype not in _STORAGE:
            raise ValueError(f"unknown storage dtype {dtype!r}")
        if not 1 <= window <= capacity:
            raise ValueError(f"window {window} must be in 1..capacity {capacity}")
        self.dtype = dtype
        np_t, self.elem_bytes = _STORAGE[dtype]
        shape = (batch, kv_heads, capacity, head_dim)
        self.k = np.zeros(shape, np_t)
        self.v = np.zeros(shape, np_t)
        self.pos = np.full((batch, capacity), -1, np.int64)
        self.lens = np.zeros(batch, np.int64)
        self.window = int(window)

    @property
    def batch(self):
        return self.k.shape[0]

    @property
    def kv_heads(self):
        return self.k.shape[1]

    @property
    def capacity(self):
        return self.k.shape[2]

    @property
    def head_dim(self):
        return self.k.shape[3]

    def oldest_kept(self, length):
        """Lowest absolute position a row of this length still holds."""
        return max(0, int(length) - self.capacity)

    def lowest_needed(self, pos):
        """Lowest key a query at absolute position pos may see ([MASK] lower bound)."""
        return max(0, int(pos) - self.window + 1)

    def append(self, k_new, v_new, n_new):
        """Write n_new[b] tokens of row b at positions lens[b] .. lens[b]+n_new[b]-1.

        Token p goes to slot p mod C and the slot records p. Every row is checked
        before anything is written (the same validate-then-write reading as the
        linear cache); a row whose write would evict a key its first new query
        still needs raises ValueError and nothing changes.
        """
        B, hk, C, d = self.k.shape
        k_new = np.asarray(k_new)
        v_new = np.asarray(v_new)
        if k_new.shape != v_new.shape or k_new.ndim != 4:
            raise ValueError("k_new and v_new must both be [B, Hkv, T, d]")
        if k_new.shape[0] != B or k_new.shape[1] != hk or k_new.shape[3] != d:
            raise ValueError("Cache batch/head/width shapes differ")
        T = k_new.shape[2]
        n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
        if n_new.shape[0] != B:
            raise ValueError("n_new must have one entry per row")
        for b in range(B):
            n, s = int(n_new[b]), int(self.lens[b])
            if n < 0 or n > T:
                raise ValueError(f"row {b}: n_new {n} outside 0..{T}")
            if n > 0 and self.oldest_kept(s + n) > self.lowest_needed(s):
                raise ValueError(f"row {b}: {n} new tokens would evict keys the window still needs "
                                 f"(capacity {C}, window {self.window})")
        for b in range(B):
            s, n = int(self.lens[b]), int(n_new[b])
            for t in range(n):
                slot = (s + t) % C
                self.k[b, :, slot] = k_new[b, :, t]
                self.v[b, :, slot] = v_new[b, :, t]
                self.pos[b, slot] = s + t
        self.lens += n_new

    def truncate(self, new_lens):
        """Roll rows back to new_lens[b]; nothing is copied.

        Valid when 0 <= n' <= length and the ring still holds every key the next
        query (at position n') would need: lowest_needed(n') >= oldest_kept(length).
        Else ValueError("Invalid truncation length") and nothing changes.
        """
        new = np.broadcast_to(np.asarray(new_lens, dtype=np.int64), self.lens.shape)
        for b in range(self.batch):
            n2, L = int(new[b]), int(self.lens[b])
            if n2 < 0 or n2 > L or self.lowest_needed(n2) < self.oldest_kept(L):
                raise ValueError("Invalid truncation length")
        self.lens = new.copy()


def attention(cache: RingCache, q, n_new):
    """Windowed GQA output [B, Hq, T, d] (float64) for the tokens just appended.

    Query t of row b sits at lens[b] - n_new[b] + t ([MASK] TL;DR); it reads
    KV head h // G ([GQA] decision 1) and every slot whose STORED position is
    visible under the window ([MASK] "A strong answer", reversal; "Common
    mistakes": never the slot index). Padded slots and rows with no new tokens
    give zeros.
    """
    q = np.asarray(q)
    B, hq, T, d = q.shape
    hk = cache.kv_heads
    if B != cache.batch or d != cache.head_dim or hq % hk != 0 or hq == 0:
        raise ValueError("q must be [B, Hq, T, d] with the cache's B and d and Hq a multiple of Hkv")
    n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
    out = np.zeros((B, hq, T, d), np.float64)
    for b in range(B):
        L, n = int(cache.lens[b]), int(n_new[b])
        if n < 0 or n > T or n > L:
            raise ValueError(f"row {b}: bad n_new {n}")
        out[b] = attention_row(cache.k[b], cache.v[b], cache.pos[b], L, n, q[b], cache.dtype, cache.window,
                               [(h, t) for h in range(hq) for t in range(n)])
    return out


def attention_row(k_slots, v_slots, stored, length, n_new_b, q_row, dtype, window, pairs):
    """Outputs of one row for the listed (head, t) pairs; zeros elsewhere.

    k_slots, v_slots: [Hkv, C, d] stored values of the row's ring; stored: [C]
    absolute position held by each slot (-1: empty); q_row: [Hq, T, d]. Used by
    ``attention`` and by the full-size tests to check sampled outputs.
    """
    hk, _, d = k_slots.shape
    hq, T, _ = q_row.shape
    G = hq // hk
    out = np.zeros((hq, T, d), np.float64)
    for h, t in pairs:
        if t >= n_new_b:
            continue
        kvh = kv_head_of(h, G)
        p = query_position(length, n_new_b, t)
        vis = window_visible(np.asarray(stored), p, length, window)
        out[h, t] = attend_one(to_float64(k_slots[kvh][vis], dtype), to_float64(v_slots[kvh][vis], dtype),
                               to_float64(q_row[h, t], dtype), d)
    return out
