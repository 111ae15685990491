"""GPU parity of tree-based speculative verify (gqa_attention_tree).

The HIP path against oracle/tree.py on the same seeded bits. [MASK] "Write the
causal mask for a decode step with a KV cache, where the query is shorter than
the keys", "What interviewers probe next": each draft token attends the full
cache plus its own ancestors, built from parent pointers.
"""

import numpy as np
import pytest
import torch

from oracle import direct, tree
import workloads as W
from gpu_util import TORCH_DTYPE, assert_close, from_dev, out_f64, to_dev

pytestmark = pytest.mark.gpu

TREES = {
    "eight": [-1, 0, 1, 2, 0, 4, -1, 6],               # two branches and a second root
    "star": [-1, 0, 0, 0, 0, 0],                        # one root, five children
    "roots": [-1, -1, -1, -1],
    "deep": [-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14],   # a 16-node chain
    "mixed": [-1, 0, -1, 2, 1, 4, 2, 6, 3, 0, 9, 9],
}


def _lib():
    from gqa_attention_preallocated_amd import KVCache, gqa_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return KVCache, gqa_attention


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("name", sorted(TREES))
def test_tree_verify(dt, d, name):
    KVCache, gqa_attention = _lib()
    par = TREES[name]
    T = len(par)
    B, hk = 3, 2
    G = 4 if T <= 16 else 2
    shape = W.Shape("tree", dt, B, hk * G, hk, d, 512)
    n = [T, T - 1, 0]
    parents = np.array([par, par, par], np.int64)
    for policy in [(0, 0), (1, 32)]:
        cache = KVCache(B, hk, 512, d, dtype=TORCH_DTYPE[dt])
        cache.set_policy(*policy)
        ref = direct.Cache(B, hk, 512, d, dt)
        _, k, v = W.step_inputs(shape, 41, 0, 300, [300, 77, 10], pad="nan")
        cache.append(to_dev(k, dt), to_dev(v, dt), [300, 77, 10])
        ref.append(k, v, [300, 77, 10])
        q, k, v = W.step_inputs(shape, 41, 1, T, n, pad="nan")
        cache.append(to_dev(k, dt), to_dev(v, dt), n)
        ref.append(k, v, n)
        out = gqa_attention(to_dev(q, dt), cache, n, parents=parents)
        assert_close(out_f64(out, dt), tree.attention(ref, q, n, parents), dt, f"tree {name} policy {policy}")
        raw = from_dev(out, dt)
        for b in range(B):
            assert not raw[b, :, n[b]:].view(np.uint8).any()


def test_chain_gives_the_bits_of_plain_attention():
    """A chain (each node's parent the node before it) is the causal rule, so
    the tree call gives the bits of plain attention on the same kernel. Tree
    verify always runs on the split-K decode kernel; the plain call here has
    48 columns a row, which the automatic plan would give to the prefill
    kernel, so the cache is set to the decode kernel for both calls."""
    KVCache, gqa_attention = _lib()
    B, hk, G, d, T = 4, 8, 4, 128, 12
    shape = W.Shape("chain", "bf16", B, hk * G, hk, d, 2048)
    cache = KVCache(B, hk, 2048, d)
    cache.set_policy(1, 0)
    _, k, v = W.step_inputs(shape, 5, 0, 1500, [1500, 900, 1200, 64], pad="normal")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [1500, 900, 1200, 64])
    q, k, v = W.step_inputs(shape, 5, 1, T, [T] * B, pad="normal")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [T] * B)
    chain = np.tile(np.arange(-1, T - 1), (B, 1))
    a = from_dev(gqa_attention(to_dev(q, "bf16"), cache, [T] * B, parents=chain), "bf16")
    b = from_dev(gqa_attention(to_dev(q, "bf16"), cache, [T] * B), "bf16")
    assert np.array_equal(a, b)


def test_tree_refusals():
    KVCache, gqa_attention = _lib()
    cache = KVCache(1, 1, 64, 16, dtype=torch.float32)
    k = torch.randn(1, 1, 8, 16, device="cuda")
    cache.append(k, k, [8])
    q = torch.randn(1, 4, 4, 16, device="cuda")
    with pytest.raises(ValueError, match="parent"):
        gqa_attention(q, cache, [4], parents=[[-1, 0, 2, 1]])
    cache.set_policy(2, 0)
    with pytest.raises(ValueError):
        gqa_attention(q, cache, [4], parents=[[-1, 0, 1, 2]])


def test_llama_tree_verify():
    """Llama-3.1-8B-shaped verify (B=16, 4,092 cached, Hq=32, Hkv=8, d=128, bf16)
    with the pages' eight candidate tokens as a tree: sampled rows against the oracle."""
    KVCache, gqa_attention = _lib()
    sh, seed = W.LLAMA8B_VERIFY, 2
    B = sh.batch
    cache = KVCache(B, sh.kv_heads, sh.max_len, sh.head_dim)
    for start in range(0, 4092, 2048):
        m = min(2048, 4092 - start)
        rows = [W.prefix_kv(sh, seed, b, start, m) for b in range(B)]
        cache.append(to_dev(np.stack([r[0] for r in rows]), "bf16"), to_dev(np.stack([r[1] for r in rows]), "bf16"),
                     [m] * B)
    par = TREES["eight"]
    T, n = 8, [8] * B
    q, k, v = W.step_inputs(sh, seed, 10_000, T, n, pad="nan")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
    out = out_f64(gqa_attention(to_dev(q, "bf16"), cache, n, parents=[par] * B), "bf16")
    for b in [0, 7, 15]:
        ref = direct.Cache(1, sh.kv_heads, 4100, sh.head_dim, "bf16")
        kh, vh = W.prefix_kv(sh, seed, b, 0, 4092)
        ref.append(np.concatenate([kh, k[b, :, :T]], axis=1)[None], np.concatenate([vh, v[b, :, :T]], axis=1)[None],
                   [4100])
        want = tree.attention(ref, q[b:b + 1], [T], [par])
        assert_close(out[b:b + 1], want, "bf16", f"tree verify row {b}")
