"""Pins of the sliding-window ring-buffer oracle (oracle/window.py).

Each pin ties the windowed reference to something other than itself: the
pinned linear-cache oracle (oracle/direct.py) on the window's suffix, closed
forms (W = 1, q = 0), visible-key counts, and planted mistakes that must fail.
Pages: [MASK] "Write the causal mask for a decode step with a KV cache, where
the query is shorter than the keys", "A strong answer" (the reversal) and
"Common mistakes"; [CH16] "16. Prefill, decode and the KV cache", exercise 3.
"""

import numpy as np
import pytest

from oracle import direct, window


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _stream(B, hk, d, total, chunk_sizes, seed):
    """Seeded K/V history [B, Hkv, total, d] and a list of per-call n_new."""
    rng = np.random.default_rng(seed)
    return _rand(rng, B, hk, total, d), _rand(rng, B, hk, total, d)


def _feed(cache, k_all, v_all, calls):
    """Append calls (list of per-row n_new) in order; yields after each call."""
    B = k_all.shape[0]
    done = np.zeros(B, np.int64)
    for n in calls:
        T = max(max(n), 1)
        kn = np.zeros((B, k_all.shape[1], T, k_all.shape[3]), np.float32)
        vn = np.zeros_like(kn)
        for b in range(B):
            kn[b, :, :n[b]] = k_all[b, :, done[b]:done[b] + n[b]]
            vn[b, :, :n[b]] = v_all[b, :, done[b]:done[b] + n[b]]
        cache.append(kn, vn, n)
        done += np.asarray(n)
        yield T, n


def test_window_covering_everything_is_plain_causal_attention():
    """W = C >= every length and no wrap: exactly the linear-cache oracle."""
    B, hk, G, d, C = 2, 2, 3, 16, 64
    k_all, v_all = _stream(B, hk, d, 60, None, 1)
    ring = window.RingCache(B, hk, C, d, window=C)
    lin = direct.Cache(B, hk, C, d)
    rng = np.random.default_rng(2)
    calls = [[5, 3], [1, 1], [7, 0], [4, 6], [1, 1]]
    for (T, n), _ in zip(_feed(ring, k_all, v_all, calls), _feed(lin, k_all, v_all, calls)):
        q = _rand(rng, B, hk * G, T, d)
        assert np.array_equal(window.attention(ring, q, n), direct.attention(lin, q, n))


def test_decode_equals_attention_over_the_last_w_tokens():
    """A decode query sees exactly the last W positions: plain attention over a
    fresh linear cache holding only those tokens agrees, across many wraps of a
    small ring (C = 16, W = 12, 90 tokens)."""
    B, hk, G, d, C, W = 2, 1, 4, 8, 16, 12
    total = 90
    k_all, v_all = _stream(B, hk, d, total, None, 3)
    ring = window.RingCache(B, hk, C, d, window=W)
    rng = np.random.default_rng(4)
    calls = [[1, 1]] * total
    for step, (T, n) in enumerate(_feed(ring, k_all, v_all, calls)):
        q = _rand(rng, B, hk * G, 1, d)
        got = window.attention(ring, q, n)
        p = step                                   # the query's absolute position
        lo = max(0, p - W + 1)
        lin = direct.Cache(B, hk, W, d)
        lin.append(k_all[:, :, lo:p + 1], v_all[:, :, lo:p + 1], [p + 1 - lo] * B)
        want = direct.attention(lin, q, [1] * B)
        assert np.abs(got - want).max() <= 1e-12, step


def test_chunks_match_per_query_windows_over_the_full_history():
    """T > 1 chunks through a wrapping ring: query at p equals softmax attention
    over the linear history restricted to positions max(0, p-W+1) .. p."""
    B, hk, G, d, C, W = 2, 2, 2, 16, 32, 20
    total = 160
    k_all, v_all = _stream(B, hk, d, total, None, 5)
    ring = window.RingCache(B, hk, C, d, window=W)
    rng = np.random.default_rng(6)
    calls = [[13, 9], [1, 4], [8, 13], [13, 13], [2, 0], [12, 11], [13, 13], [5, 1], [13, 13],
             [13, 13], [13, 13], [13, 13], [13, 13], [13, 13]]
    done = np.zeros(B, np.int64)
    for T, n in _feed(ring, k_all, v_all, calls):
        done += np.asarray(n)
        q = _rand(rng, B, hk * G, T, d)
        got = window.attention(ring, q, n)
        for b in range(B):
            L = int(done[b])
            for h in range(hk * G):
                for t in range(T):
                    if t >= n[b]:
                        assert not got[b, h, t].any()
                        continue
                    p = L - n[b] + t
                    lo = max(0, p - W + 1)
                    keys = k_all[b, h // G, lo:p + 1].astype(np.float64)
                    vals = v_all[b, h // G, lo:p + 1].astype(np.float64)
                    s = keys @ q[b, h, t].astype(np.float64) / np.sqrt(d)
                    w = np.exp(s - s.max())
                    assert np.abs(got[b, h, t] - (w @ vals) / w.sum()).max() <= 1e-12


def test_window_of_one_returns_the_own_value():
    """W = 1: each query sees only itself, so the output is its own V row."""
    B, hk, G, d, C = 1, 2, 2, 8, 8
    k_all, v_all = _stream(B, hk, d, 30, None, 7)
    ring = window.RingCache(B, hk, C, d, window=1)
    rng = np.random.default_rng(8)
    done = 0
    for T, n in _feed(ring, k_all, v_all, [[3]] * 10):
        q = _rand(rng, B, hk * G, T, d)
        out = window.attention(ring, q, n)
        for h in range(hk * G):
            for t in range(3):
                assert np.array_equal(out[0, h, t], v_all[0, h // G, done + t].astype(np.float64))
        done += 3


def test_zero_query_gives_the_mean_of_the_band():
    """q = 0: uniform weights over the visible keys, i.e. the mean of V over
    positions max(0, p-W+1) .. p (pins both band edges)."""
    B, hk, G, d, C, W = 1, 1, 2, 4, 24, 7
    k_all, v_all = _stream(B, hk, d, 60, None, 9)
    ring = window.RingCache(B, hk, C, d, window=W)
    done = 0
    for T, n in _feed(ring, k_all, v_all, [[5]] * 12):
        out = window.attention(ring, np.zeros((B, hk * G, T, d), np.float32), n)
        for t in range(5):
            p = done + t
            want = v_all[0, 0, max(0, p - W + 1):p + 1].astype(np.float64).mean(axis=0)
            assert np.abs(out[0, 0, t] - want).max() <= 1e-12
        done += 5


def test_visible_counts_follow_the_window():
    """Per query: min(W, p + 1) visible keys; T = 4 over S = 4,096 with W = 1,024
    gives 1,024 each ([MASK] verify example with the window's lower bound)."""
    S, T, W = 4096, 4, 1024
    j = np.arange(S)
    for i in range(T):
        p = S - T + i
        assert int(window.window_visible(j, p, S, W).sum()) == min(W, p + 1) == 1024
    for p in range(0, 40):
        assert int(window.window_visible(np.arange(p + 1), p, p + 1, 16).sum()) == min(16, p + 1)


def _slot_index_attention(cache, q, n_new):
    """Planted mistake of [MASK] "Common mistakes": the mask built from slot
    indices instead of the stored positions."""
    B, hq, T, d = q.shape
    G = hq // cache.kv_heads
    out = np.zeros((B, hq, T, d))
    for b in range(B):
        L, n = int(cache.lens[b]), int(n_new[b])
        slots = np.arange(cache.capacity)
        for h in range(hq):
            for t in range(n):
                p = L - n + t
                vis = window.window_visible(slots, p, L, cache.window)
                out[b, h, t] = direct.attend_one(cache.k[b, h // G][vis].astype(np.float64),
                                                 cache.v[b, h // G][vis].astype(np.float64),
                                                 q[b, h, t].astype(np.float64), d)
    return out


def test_planted_slot_index_mask_fails_after_a_wrap():
    B, hk, G, d, C, W = 1, 1, 2, 8, 16, 12
    k_all, v_all = _stream(B, hk, d, 40, None, 10)
    ring = window.RingCache(B, hk, C, d, window=W)
    rng = np.random.default_rng(11)
    worst = 0.0
    for step, (T, n) in enumerate(_feed(ring, k_all, v_all, [[1]] * 40)):
        q = _rand(rng, B, hk * G, 1, d)
        worst = max(worst, np.abs(_slot_index_attention(ring, q, n) - window.attention(ring, q, n)).max())
    assert worst > 1e-2            # the slot-index mask is wrong once the ring wraps


def test_planted_off_by_one_window_fails_the_own_value_pin():
    vis_right = window.window_visible(np.arange(10), 9, 10, 1)
    vis_wrong = (np.arange(10) <= 9) & (np.arange(10) >= 9 - 1)      # j >= p - W
    assert vis_right.sum() == 1 and vis_wrong.sum() == 2


def test_ring_slots_hold_the_tokens_bit_exactly():
    B, hk, d, C = 2, 2, 8, 16
    k_all, v_all = _stream(B, hk, d, 50, None, 12)
    ring = window.RingCache(B, hk, C, d, window=8)
    done = np.zeros(B, np.int64)
    for T, n in _feed(ring, k_all, v_all, [[5, 3], [6, 8], [9, 9], [9, 0], [7, 9]]):
        done += np.asarray(n)
        for b in range(B):
            L = int(done[b])
            for p in range(max(0, L - C), L):
                s = p % C
                assert ring.pos[b, s] == p
                assert np.array_equal(ring.k[b, :, s], k_all[b, :, p])
                assert np.array_equal(ring.v[b, :, s], v_all[b, :, p])
    assert ring.lens.tolist() == done.tolist()


def test_append_that_would_evict_needed_keys_changes_nothing():
    """C = 16, W = 8: at most C - W + 1 = 9 tokens per call once the ring is full."""
    B, hk, d, C, W = 2, 1, 4, 16, 8
    k_all, v_all = _stream(B, hk, d, 60, None, 13)
    ring = window.RingCache(B, hk, C, d, window=W)
    list(_feed(ring, k_all, v_all, [[16, 16]]))
    before = (ring.k.copy(), ring.v.copy(), ring.pos.copy(), ring.lens.copy())
    with pytest.raises(ValueError, match="evict"):
        list(_feed(ring, k_all[:, :, 16:], v_all[:, :, 16:], [[9, 10]]))   # row 1 asks for 10
    assert all(np.array_equal(a, b) for a, b in zip(before, (ring.k, ring.v, ring.pos, ring.lens)))
    list(_feed(ring, k_all[:, :, 16:], v_all[:, :, 16:], [[9, 9]]))        # 9 is the limit
    assert ring.lens.tolist() == [25, 25]


def test_truncate_validity_in_a_ring():
    """Rollback keeps working while the ring still holds the next query's window."""
    B, hk, d, C, W = 1, 1, 4, 16, 8
    k_all, v_all = _stream(B, hk, d, 40, None, 14)
    ring = window.RingCache(B, hk, C, d, window=W)
    list(_feed(ring, k_all, v_all, [[9], [9], [9]]))            # length 27, ring holds 11..26
    with pytest.raises(ValueError, match="Invalid truncation length"):
        ring.truncate([28])
    with pytest.raises(ValueError, match="Invalid truncation length"):
        ring.truncate([17])                                     # would need key 10, evicted
    ring.truncate([18])                                         # needs 11..17: held
    assert ring.lens.tolist() == [18]
