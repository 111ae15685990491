"""A second CPU formulation of the same attention, used to cross-check ``direct``.

TEST INFRASTRUCTURE (see the package docstring).

``direct`` walks every (head, query) pair, gathers exactly the keys that query
may see and normalises with a subtracted maximum. This module takes a
different route through the same definition:

  * it works one (row, KV head) block at a time, over that row's own live
    prefix only (no batch-wide padding to the longest row);
  * the G query heads of the block and its real queries form one matrix of
    G * n_new rows, multiplied against the prefix keys in one product;
  * visibility is the bottom-right-aligned lower triangle of an
    (n_new x S) rectangle, ``tril(k = S - n_new)``, the closed form stated in
    "Write the causal mask for a decode step with a KV cache, where the query
    is shorter than the keys" (TL;DR, j <= i + (S - T));
  * the softmax is normalised in log space: each probability is
    exp(score - logsumexp(visible scores)), with the log-sum-exp taken by a
    reduction of numpy's ``logaddexp``.

Padded query slots and rows with no new tokens are never computed, so they
stay at the zeros the output starts from. Every real query sees at least key
0 (its position is >= 0 because n_new <= S), so no guard is needed. The module
shares only the storage decoder with ``direct``; the tests require the two to
agree to 1e-10 in float64.
"""

from __future__ import annotations

import numpy as np

from .direct import to_float64


def _block(keys, values, queries, n, S):
    """Attention of one (row, KV head) block.

    keys, values: [S, d] float64, the row's live prefix; queries: [G, n, d]
    float64, the block's real queries (the last n of the S positions).
    Returns [G, n, d].
    """
    G, _, d = queries.shape
    flat = queries.reshape(G * n, d)
    logits = (flat @ keys.T).reshape(G, n, S) / np.sqrt(d)
    seen = np.tril(np.ones((n, S), dtype=bool), k=S - n)       # query i: keys 0 .. S - n + i
    logits = np.where(seen[None], logits, -np.inf)
    lse = np.logaddexp.reduce(logits, axis=-1, keepdims=True)  # [G, n, 1]
    weights = np.exp(logits - lse)                             # masked keys: exp(-inf) = 0
    return weights @ values


def attention(k, v, lens, q, n_new, dtype):
    """k, v: stored [B, Hkv, >=max(lens), d]; q: stored [B, Hq, T, d].

    Returns float64 [B, Hq, T, d]: for each row b, query t < n_new[b] of head
    h attends keys 0 .. lens[b] - n_new[b] + t of KV head h // G.
    """
    q64 = to_float64(q, dtype)
    B, hq, T, d = q64.shape
    hk = k.shape[1]
    G = hq // hk
    out = np.zeros((B, hq, T, d), np.float64)
    for b in range(B):
        S, n = int(lens[b]), int(n_new[b])
        if n == 0:
            continue
        for kvh in range(hk):
            heads = slice(kvh * G, (kvh + 1) * G)     # the query heads that read KV head kvh
            keys = to_float64(k[b, kvh, :S], dtype)
            values = to_float64(v[b, kvh, :S], dtype)
            out[b, heads, :n] = _block(keys, values, q64[b, heads, :n], n, S)
    return out
