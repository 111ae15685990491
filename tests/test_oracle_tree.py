"""Pins of the tree-verify oracle (oracle/tree.py).

[MASK] "Write the causal mask for a decode step with a KV cache, where the
query is shorter than the keys", "What interviewers probe next": a draft
node sees the committed keys and its own path to the root. Pins: a chain is the ordinary
causal verify of the linear oracle, a tree of roots is T independent decode
steps, other branches never reach a node, visible counts follow depth, and the
plain causal triangle fails on a branching tree.
"""

import numpy as np
import pytest

from oracle import direct, tree


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _cache(rng, B, hk, d, S, prefix, n):
    c = direct.Cache(B, hk, S, d, "f32")
    k, v = _rand(rng, B, hk, prefix + n, d), _rand(rng, B, hk, prefix + n, d)
    c.append(k, v, [prefix + n] * B)
    return c, k, v


def test_chain_is_the_causal_verify():
    rng = np.random.default_rng(0)
    B, hk, G, d, n = 2, 2, 2, 16, 6
    c, _, _ = _cache(rng, B, hk, d, 64, 30, n)
    q = _rand(rng, B, hk * G, n, d)
    chain = np.tile(np.arange(-1, n - 1), (B, 1))
    assert np.array_equal(tree.attention(c, q, [n] * B, chain), direct.attention(c, q, [n] * B))


def test_roots_are_independent_decode_steps():
    """Every node hangs off the committed prefix: node t equals a T=1 decode over
    the prefix followed by node t alone."""
    rng = np.random.default_rng(1)
    B, hk, G, d, n, P = 1, 2, 3, 8, 5, 20
    c, k, v = _cache(rng, B, hk, d, 64, P, n)
    q = _rand(rng, B, hk * G, n, d)
    out = tree.attention(c, q, [n], np.full((B, n), -1))
    for t in range(n):
        one = direct.Cache(B, hk, 64, d, "f32")
        one.append(np.concatenate([k[:, :, :P], k[:, :, P + t:P + t + 1]], 2),
                   np.concatenate([v[:, :, :P], v[:, :, P + t:P + t + 1]], 2), [P + 1])
        want = direct.attention(one, q[:, :, t:t + 1], [1])
        assert np.array_equal(out[:, :, t:t + 1], want)


# eight candidates in two branches: 0 -> 1 -> 2 -> 3 and 0 -> 4 -> 5, 6 -> 7 off the prefix
PARENTS8 = [-1, 0, 1, 2, 0, 4, -1, 6]


def test_other_branches_never_reach_a_node():
    rng = np.random.default_rng(2)
    B, hk, G, d, n, P = 1, 1, 4, 16, 8, 40
    c, _, _ = _cache(rng, B, hk, d, 64, P, n)
    q = _rand(rng, B, hk * G, n, d)
    before = tree.attention(c, q, [n], [PARENTS8])
    c.k[0, 0, P + 4:P + 6] += 5.0          # perturb the branch 4 -> 5
    c.v[0, 0, P + 4:P + 6] -= 3.0
    after = tree.attention(c, q, [n], [PARENTS8])
    for t in range(n):
        touched = t in (4, 5)
        assert np.array_equal(before[0, :, t], after[0, :, t]) != touched, t


def test_visible_counts_follow_depth():
    L, n, P = 48, 8, 40
    depth = [1, 2, 3, 4, 2, 3, 1, 2]       # nodes on the path to the root, the node included
    for t in range(n):
        assert int(tree.tree_visible(L, n, PARENTS8, t).sum()) == P + depth[t]
        assert tree.ancestors(PARENTS8, t)[0] == t


def test_planted_causal_triangle_fails_on_a_branching_tree():
    rng = np.random.default_rng(3)
    B, hk, G, d, n, P = 1, 1, 2, 16, 8, 10
    c, _, _ = _cache(rng, B, hk, d, 32, P, n)
    q = _rand(rng, B, hk * G, n, d)
    assert np.abs(tree.attention(c, q, [n], [PARENTS8]) - direct.attention(c, q, [n])).max() > 1e-2


def test_parents_must_be_topological():
    for bad in ([0], [-1, 1], [-1, 0, 5], [-2]):
        with pytest.raises(ValueError):
            tree.check_parents(bad, len(bad))
    tree.check_parents(PARENTS8, 8)
