"""Pins of the paged-cache oracle (oracle/paged.py).

[GQA] "Implement grouped-query attention over a preallocated KV cache, with no
torch.cat, for both prefill chunks and decode", the reversal paragraph (rows
whose lengths differ by orders of magnitude call for per-row page tables) and [CH16]
"16. Prefill, decode and the KV cache", design choices (a paged cache keeps the
O(1) write without reserving max_len per row). Pins: paging changes where the
bytes live, never the result, so outputs equal the linear oracle bit for bit
for any interleaving of rows; the pages a row holds are exactly
ceil(len / page_size); a rollback frees whole pages for any row; a call that
cannot get its pages changes nothing; and a planted mistake in the gather
(pages taken in the wrong order) fails the equality.
"""

import numpy as np
import pytest

from oracle import direct, paged


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _drive(rng, B, hk, G, d, P, pages, blocks, calls):
    """The same appends into a paged and a linear oracle; attention after each call."""
    pc = paged.PagedCache(B, hk, pages, P, blocks, d)
    lc = direct.Cache(B, hk, P * blocks, d, "f32")
    outs = []
    for T, n in calls:
        k, v = _rand(rng, B, hk, T, d), _rand(rng, B, hk, T, d)
        q = _rand(rng, B, hk * G, T, d)
        pc.append(k, v, n)
        lc.append(k, v, n)
        a, b = paged.attention(pc, q, n), direct.attention(lc, q, n)
        outs.append((a, b))
    return pc, lc, outs


def test_equals_the_linear_cache_bit_for_bit():
    rng = np.random.default_rng(0)
    calls = [(70, [70, 3, 0]), (1, [1, 1, 1]), (5, [5, 0, 2]), (64, [64, 64, 64]), (1, [0, 1, 1])]
    pc, lc, outs = _drive(rng, 3, 2, 3, 16, 64, 12, 4, calls)
    for a, b in outs:
        assert np.array_equal(a, b)
    for b in range(3):
        k, v = pc.gather(b)
        L = int(lc.lens[b])
        assert np.array_equal(k, lc.k[b, :, :L]) and np.array_equal(v, lc.v[b, :, :L])


def test_rows_interleave_in_the_pool():
    """Rows that grow in turn get pages that alternate in the pool, and the
    result is still the linear cache's."""
    rng = np.random.default_rng(1)
    calls = [(64, [64, 64])] * 3 + [(1, [1, 1])]
    pc, _, outs = _drive(rng, 2, 1, 2, 8, 64, 8, 4, calls)
    assert pc.table[0, :4].tolist() == [0, 2, 4, 6] and pc.table[1, :4].tolist() == [1, 3, 5, 7]
    for a, b in outs:
        assert np.array_equal(a, b)


def test_pages_held_follow_the_lengths():
    rng = np.random.default_rng(2)
    P = 64
    pc = paged.PagedCache(4, 2, 40, P, 16, 8)
    lens = np.zeros(4, np.int64)
    for step in range(6):
        n = rng.integers(0, 150, 4)
        T = int(n.max())
        pc.append(_rand(rng, 4, 2, T, 8), _rand(rng, 4, 2, T, 8), n)
        lens += n
        held = (pc.table >= 0).sum(axis=1)
        assert held.tolist() == [-(-int(L) // P) for L in lens]
        used = pc.table[pc.table >= 0]
        assert len(set(used.tolist())) == len(used)               # no page is given twice
        assert len(pc.free) + len(used) == 40


def test_rollback_frees_whole_pages_for_any_row():
    rng = np.random.default_rng(3)
    pc = paged.PagedCache(2, 1, 6, 64, 6, 8)
    pc.append(_rand(rng, 2, 1, 200, 8), _rand(rng, 2, 1, 200, 8), [200, 64])   # 4 + 1 pages
    assert sorted(pc.free) == [5]
    pc.truncate([65, 64])                                                       # row 0 keeps 2 pages
    assert pc.table[0].tolist() == [0, 1, -1, -1, -1, -1]
    assert sorted(pc.free) == [2, 3, 5]
    pc.append(_rand(rng, 2, 1, 64, 8), _rand(rng, 2, 1, 64, 8), [0, 64])       # row 1 grows into page 2
    assert pc.table[1, :2].tolist() == [4, 2]
    with pytest.raises(ValueError):
        pc.truncate([66, 0])


def test_a_call_that_cannot_get_its_pages_changes_nothing():
    rng = np.random.default_rng(4)
    pc = paged.PagedCache(2, 1, 3, 64, 4, 8)
    pc.append(_rand(rng, 2, 1, 64, 8), _rand(rng, 2, 1, 64, 8), [64, 64])
    before = (pc.k.copy(), pc.table.copy(), pc.lens.copy(), sorted(pc.free))
    with pytest.raises(ValueError, match="pages needed"):
        pc.append(_rand(rng, 2, 1, 65, 8), _rand(rng, 2, 1, 65, 8), [65, 1])    # 2 + 1 > 1 free
    with pytest.raises(ValueError, match="blocks"):
        pc.append(_rand(rng, 2, 1, 200, 8), _rand(rng, 2, 1, 200, 8), [200, 0])  # 5 blocks > 4
    assert np.array_equal(pc.k, before[0]) and np.array_equal(pc.table, before[1])
    assert np.array_equal(pc.lens, before[2]) and sorted(pc.free) == before[3]


def test_ragged_rows_need_a_fraction_of_the_dense_reservation():
    """[GQA] reversal: one long row and many short ones. The pool holds exactly
    the pages the lengths need; a dense cache reserves max_len for every row."""
    P, lens = 64, [8000, 40, 300, 12, 900, 5, 64, 65]
    max_len = 8192
    pages = sum(-(-L // P) for L in lens)
    pc = paged.PagedCache(len(lens), 1, pages, P, max_len // P, 4)
    T = max(lens)
    pc.append(np.zeros((len(lens), 1, T, 4), np.float32), np.zeros((len(lens), 1, T, 4), np.float32), lens)
    assert len(pc.free) == 0
    assert pages * P < len(lens) * max_len / 5


def test_planted_mistake_page_order_fails():
    rng = np.random.default_rng(5)
    calls = [(64, [64, 64]), (64, [64, 64]), (3, [3, 3])]
    pc, lc, _ = _drive(rng, 2, 1, 2, 8, 64, 8, 4, calls)
    q = _rand(rng, 2, 2, 3, 8)
    good = paged.attention(pc, q, [3, 3])
    assert np.array_equal(good, direct.attention(lc, q, [3, 3]))
    # the mistake: blocks of a row gathered in reverse order
    pc.table[:, :3] = pc.table[:, 2::-1].copy()
    assert np.abs(paged.attention(pc, q, [3, 3]) - good).max() > 1e-3
