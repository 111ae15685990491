"""The direct CPU reference: preallocated cache plus loop-over-queries attention.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg.

Sources (titles of the pages; sections named in each docstring):
  [GQA]   "Implement grouped-query attention over a preallocated KV cache, with
          no torch.cat, for both prefill chunks and decode" (inferenceinterviews.com)
  [MASK]  "Write the causal mask for a decode step with a KV cache, where the
          query is shorter than the keys" (inferenceinterviews.com)
  [CH16]  "16. Prefill, decode and the KV cache" (inference.shantanugoel.com)

Arithmetic is float64 throughout. Stored values (float32, or bfloat16 kept as
uint16 bit patterns) are widened exactly before any arithmetic.
"""

from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# storage
# --------------------------------------------------------------------------

_STORAGE = {"f32": (np.float32, 4), "bf16": (np.uint16, 2)}


def to_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (float32, or bf16 bit patterns).

    A bfloat16 is the upper half of a float32, so its value is the float32
    whose high 16 bits are the stored bits and whose low 16 bits are zero.
    """
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def kv_cache_bytes(layers, batch, tokens, kv_heads, head_dim, bytes_per_value=2):
    """KV bytes = 2 (K and V) x layers x batch x tokens x kv_heads x head_dim x bytes.

    [CH16] section "How big is the cache?": the formula counts KV heads, not
    query heads, which is why grouped-query attention shrinks the cache.
    """
    return 2 * layers * batch * tokens * kv_heads * head_dim * bytes_per_value


# --------------------------------------------------------------------------
# the cache: allocate once, write in place, roll back without copying
# --------------------------------------------------------------------------

class Cache:
    """K and V as [B, Hkv, max_len, d], allocated once, plus a length per row.

    [GQA] "A strong answer": the buffers are zero-filled at construction and
    never reallocated; ``lens[b]`` counts the tokens row b holds. Rows have
    their own lengths (the reading taken where [CH16] "Layout and validity"
    advances all rows together: the ragged form is the one attention needs).
    """

    def __init__(self, batch, kv_heads, max_len, head_dim, dtype="f32"):
        if dtype not in _STORAGE:
            raise ValueError(f"unknown storage dtype {dtype!r}")
        self.dtype = dtype
        np_t, self.elem_bytes = _STORAGE[dtype]
        shape = (batch, kv_heads, max_len, head_dim)
        self.k = np.zeros(shape, np_t)
        self.v = np.zeros(shape, np_t)
        self.lens = np.zeros(batch, np.int64)

    @property
    def batch(self):
        return self.k.shape[0]

    @property
    def kv_heads(self):
        return self.k.shape[1]

    @property
    def max_len(self):
        return self.k.shape[2]

    @property
    def head_dim(self):
        return self.k.shape[3]

    def append(self, k_new, v_new, n_new):
        """Write n_new[b] new tokens of row b at positions lens[b] .. lens[b]+n_new[b]-1.

        ``k_new``/``v_new`` are [B, Hkv, T, d]; slots t >= n_new[b] are padding
        and are never read. [GQA] "A strong answer": the write goes in place at
        the row's current length, history is untouched, and a row that would
        pass max_len raises ``ValueError("row {b}: {s+n} tokens > max_len {S}")``.

        Reading taken on atomicity: every row is checked before any byte is
        written ([CH16] "Layout and validity" checks capacity before copying),
        so a failed call changes neither the buffers nor the lengths, and the
        length only moves after the write ([GQA] "Common mistakes").
        """
        B, hk, S, d = self.k.shape
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
            n = int(n_new[b])
            if n < 0 or n > T:
                raise ValueError(f"row {b}: n_new {n} outside 0..{T}")
            s = int(self.lens[b])
            if s + n > S:
                raise ValueError(f"row {b}: {s + n} tokens > max_len {S}")
        for b in range(B):
            s, n = int(self.lens[b]), int(n_new[b])
            self.k[b, :, s:s + n] = k_new[b, :, :n]
            self.v[b, :, s:s + n] = v_new[b, :, :n]
        self.lens += n_new

    def truncate(self, new_lens):
        """Forget tokens past new_lens[b]; nothing is copied or cleared.

        [CH16] "Layout and validity": the valid range is 0 <= n <= current
        length, else ``ValueError("Invalid truncation length")``; slots past the
        length keep stale data that attention never reads. A scalar applies to
        every row; an array gives each row its own rollback point (speculative
        rollback differs per row).
        """
        new = np.broadcast_to(np.asarray(new_lens, dtype=np.int64), self.lens.shape)
        if np.any(new < 0) or np.any(new > self.lens):
            raise ValueError("Invalid truncation length")
        self.lens = new.copy()

    def reset(self):
        self.truncate(0)

    @property
    def bytes(self):
        """Bytes of the reservation: every element of K and V ([CH16] ``bytes``)."""
        return (self.k.size + self.v.size) * self.elem_bytes

    @property
    def live_bytes(self):
        """Bytes of valid K and V: the formula of [CH16] with tokens = lens."""
        return int(kv_cache_bytes(1, 1, int(self.lens.sum()), self.kv_heads,
                                  self.head_dim, self.elem_bytes))


# --------------------------------------------------------------------------
# the three rules: head map, absolute positions, visibility
# --------------------------------------------------------------------------

def kv_head_of(h, group):
    """Query head h reads KV head h // G ([GQA] "How to approach it").

    Consecutive query heads share a KV head; h % Hkv would interleave the groups
    ([GQA] "Common mistakes").
    """
    return h // group


def query_position(length, n_new, t):
    """Absolute position of chunk query t: the chunk is the LAST n_new tokens.

    [GQA] TL;DR: query t sits at len - n_new + t, with len counted after the
    append. [MASK] TL;DR: for T queries over S keys, row i sits at S - T + i.
    """
    return length - n_new + t


def key_visible(j, pos, length):
    """Key j is visible to a query at absolute position pos (bottom-right rule).

    [MASK] TL;DR: j <= i + (S - T), i.e. j <= pos; and j < length keeps stale
    slots past the row's length out ([CH16] "Layout and validity"). Works on
    scalars and on numpy index arrays.
    """
    return (j <= pos) & (j < length)


def decode_causal_mask(T, S):
    """Bool [T, S]: entry (i, j) is True when key j may be attended by query i.

    The T queries are the last T of S positions ([MASK] "A strong answer").
    Built element by element from ``query_position`` and ``key_visible``.
    """
    m = np.zeros((T, S), dtype=bool)
    for i in range(T):
        pos = query_position(S, T, i)
        for j in range(S):
            m[i, j] = key_visible(j, pos, S)
    return m


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attend_one(keys, values, q, head_dim):
    """Plain softmax attention of one query over the given keys (float64).

    keys, values: [n, d] -- exactly the keys the query may see; q: [d].
    Scores are q.k / sqrt(d) ([GQA] "A strong answer"); the max is subtracted
    before exp, which changes nothing mathematically. No visible key gives a
    zero vector, never NaN.
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], np.float64)
    s = keys @ q / math.sqrt(head_dim)
    m = s.max()
    p = np.exp(s - m)
    return (p @ values) / p.sum()


def _check_call(cache_batch, kv_heads, head_dim, lens, q_shape, n_new):
    B, hq, T, d = q_shape
    if B != cache_batch or d != head_dim:
        raise ValueError("q must be [B, Hq, T, d] with the cache's B and d")
    if hq % kv_heads != 0 or hq == 0:
        raise ValueError(f"q_heads {hq} is not a multiple of kv_heads {kv_heads}")
    n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
    if n_new.shape[0] != B:
        raise ValueError("n_new must have one entry per row")
    for b in range(B):
        if n_new[b] < 0 or n_new[b] > T:
            raise ValueError(f"row {b}: n_new {int(n_new[b])} outside 0..{T}")
        if n_new[b] > lens[b]:
            raise ValueError(f"row {b}: n_new {int(n_new[b])} > length {int(lens[b])}")
    return n_new


def attention(cache: Cache, q, n_new):
    """GQA output [B, Hq, T, d] (float64) for the n_new[b] tokens just appended.

    The "direct reference" of [GQA] "A strong answer": per row, repeat the KV
    heads so query head h has its own copy of KV head h // G, then loop over
    every head and every real query and take a plain softmax over keys 0..pos.
    Padded slots t >= n_new[b], rows with no new tokens, an empty batch and an
    all-empty cache give zeros ([GQA] "A strong answer"; fully masked rows must
    not produce NaN).
    """
    q = np.asarray(q)
    B, hq, T, d = q.shape
    hk = cache.kv_heads
    n_new = _check_call(cache.batch, hk, cache.head_dim, cache.lens, q.shape, n_new)
    G = hq // hk
    out = np.zeros((B, hq, T, d), np.float64)
    for b in range(B):
        L = int(cache.lens[b])
        n = int(n_new[b])
        if n == 0:
            continue
        out[b] = attention_row(cache.k[b], cache.v[b], L, n, q[b], cache.dtype,
                               [(h, t) for h in range(hq) for t in range(T)])
    return out


def attention_row(k_row, v_row, length, n_new_b, q_row, dtype, pairs):
    """Outputs of one batch row for the listed (head, t) pairs.

    k_row, v_row: [Hkv, >= length, d] stored values of that row; q_row:
    [Hq, T, d] stored values. Returns [Hq, T, d] float64 with zeros everywhere
    except the listed pairs with t < n_new_b. Used by ``attention`` for whole
    rows and by the full-size tests to check sampled outputs one by one.
    """
    hk, _, d = k_row.shape
    hq, T, _ = q_row.shape
    G = hq // hk
    k64 = to_float64(k_row[:, :length], dtype)
    v64 = to_float64(v_row[:, :length], dtype)
    # repeat the KV heads: entry h is the copy query head h reads (views, so
    # the repetition costs no memory; the values are those of np.repeat)
    kr = [k64[kv_head_of(h, G)] for h in range(hq)]
    vr = [v64[kv_head_of(h, G)] for h in range(hq)]
    j = np.arange(length)
    out = np.zeros((hq, T, d), np.float64)
    for h, t in pairs:
        if t >= n_new_b:
            continue
        pos = query_position(length, n_new_b, t)
        vis = key_visible(j, pos, length)
        qv = to_float64(q_row[h, t], dtype)
        out[h, t] = attend_one(kr[h][vis], vr[h][vis], qv, d)
    return out
