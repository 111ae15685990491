"""Tree-based speculative verify over the linear cache: the CPU reference.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/ and
``__graft_entry__.smoke()``.

Source: [MASK] "Write the causal mask for a decode step with a KV cache, where
the query is shorter than the keys" (inferenceinterviews.com), "What
interviewers probe next". When the draft is a tree rather than a chain, the
new tokens' block of the mask is no longer triangular: a draft token sees
every committed key, and among the new tokens only those on its own path to
the root, which parent pointers describe.

Readings taken where the page is silent (each listed in the design notes):
  * The n_new[b] tree nodes of row b are the tokens just appended, in node
    order: node u is the key at absolute position len - n_new + u.
  * parents[b][u] is -1 for a node hanging off the last committed token, or the
    index of an earlier node (0 <= parents[b][u] < u), so a tree is given in
    topological order.
  * Node t (query t) sees every committed key (positions below len - n_new)
    and the nodes on its path to the root, itself included.
"""

from __future__ import annotations

import numpy as np

from .direct import Cache, attend_one, kv_head_of, to_float64


def ancestors(parents, t):
    """Nodes on the path from node t to the root, t included (parent pointers)."""
    out = []
    u = t
    while u >= 0:
        out.append(u)
        u = int(parents[u])
    return out


def check_parents(parents, n):
    """A valid tree in topological order: every parent is -1 or an earlier node."""
    for u in range(n):
        if not (-1 <= int(parents[u]) < u):
            raise ValueError(f"node {u}: parent {int(parents[u])} is not -1 or an earlier node")


def tree_visible(length, n_new, parents, t):
    """Bool [length]: the keys node t may attend ([MASK] "What interviewers probe next")."""
    base = length - n_new
    vis = np.zeros(length, dtype=bool)
    vis[:base] = True
    for u in ancestors(parents, t):
        vis[base + u] = True
    return vis


def attention(cache: Cache, q, n_new, parents):
    """Output [B, Hq, T, d] (float64): query t of row b attends the committed keys
    and its ancestors; query head h reads KV head h // G; padded slots are zero."""
    q = np.asarray(q)
    B, hq, T, d = q.shape
    hk = cache.kv_heads
    G = hq // hk
    n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
    parents = np.asarray(parents).reshape(B, -1)
    out = np.zeros((B, hq, T, d), np.float64)
    for b in range(B):
        L, n = int(cache.lens[b]), int(n_new[b])
        if n < 0 or n > T or n > L:
            raise ValueError(f"row {b}: bad n_new {n}")
        check_parents(parents[b], n)
        k64 = to_float64(cache.k[b, :, :L], cache.dtype)
        v64 = to_float64(cache.v[b, :, :L], cache.dtype)
        for t in range(n):
            vis = tree_visible(L, n, parents[b], t)
            for h in range(hq):
                kvh = kv_head_of(h, G)
                out[b, h, t] = attend_one(k64[kvh][vis], v64[kvh][vis], to_float64(q[b, h, t], cache.dtype), d)
    return out
