"""A second CPU formulation of the same attention, written independently.

TEST INFRASTRUCTURE (see the package docstring).

Where ``direct`` repeats KV heads and loops over queries, this one keeps the
group on its own axis ([B, Hkv, G, T, d], the query reshape described in the
TL;DR of "Implement grouped-query attention over a preallocated KV cache")
and builds the whole visibility tensor at once from index arithmetic:
  * key j < lens[b]                              (ragged rows),
  * key j <= lens[b] - n_new[b] + t              (offset causal rule),
  * t < n_new[b]                                 (padded query slots),
then takes a softmax whose max and denominator are guarded so a fully masked
row yields zeros. It shares nothing with ``direct`` but the storage decoder,
and the tests require the two to agree to 1e-10 in float64.
"""

from __future__ import annotations

import numpy as np

from .direct import to_float64


def attention(k, v, lens, q, n_new, dtype):
    """k, v: stored [B, Hkv, >=max(lens), d]; q: stored [B, Hq, T, d].

    Returns float64 [B, Hq, T, d].
    """
    q64 = to_float64(q, dtype)
    B, hq, T, d = q64.shape
    hk = k.shape[1]
    grp = hq // hk
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    n_new = np.asarray(n_new, dtype=np.int64).reshape(B)
    L = int(lens.max()) if B else 0
    out = np.zeros((B, hq, T, d), np.float64)
    if L == 0 or T == 0:
        return out
    k64 = to_float64(k[:, :, :L], dtype)                 # [B, Hkv, L, d]
    v64 = to_float64(v[:, :, :L], dtype)
    qg = q64.reshape(B, hk, grp, T, d)                   # group on its own axis
    scores = np.matmul(qg, k64[:, :, None].swapaxes(-1, -2)) * (1.0 / np.sqrt(d))  # [B,Hkv,G,T,L]

    key = np.arange(L)[None, None, :]                    # [1, 1, L]
    tq = np.arange(T)[None, :, None]                     # [1, T, 1]
    first = (lens - n_new)[:, None, None]                # absolute position of t = 0
    ok = (key < lens[:, None, None]) & (key <= first + tq) & (tq < n_new[:, None, None])
    ok = ok[:, None, None]                               # [B, 1, 1, T, L]

    scores = np.where(ok, scores, -np.inf)
    row_max = scores.max(axis=-1, keepdims=True)
    row_max = np.where(np.isfinite(row_max), row_max, 0.0)
    w = np.where(ok, np.exp(scores - row_max), 0.0)
    den = w.sum(axis=-1, keepdims=True)
    w = w / np.where(den > 0.0, den, 1.0)
    res = np.matmul(w, v64[:, :, None])                  # [B, Hkv, G, T, d]
    return res.reshape(B, hq, T, d)
