"""GPU parity of sliding-window attention over a ring-buffer cache.

The HIP path (KVCache(window=W) -> kv_cache_create_ring, kv_append,
gqa_attention, kv_truncate through the C ABI) against the windowed CPU oracle
(oracle/window.py), on the same seeded bits: ring contents and lengths bit for
bit after every call, outputs within the contract tolerances. Pages: [MASK]
"Write the causal mask for a decode step with a KV cache, where the query is
shorter than the keys", "A strong answer" (the reversal) and "Common
mistakes"; [CH16] "16. Prefill, decode and the KV cache", exercise 3.
"""

import numpy as np
import pytest
import torch

from oracle import window
import workloads as W
from gpu_util import TORCH_DTYPE, assert_close, from_dev, out_f64, same_bytes, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    from gqa_attention_preallocated_amd import KVCache, gqa_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return KVCache, gqa_attention


def _run_ring(dt, d, C, win, policy, calls, seed, rollback_every=0):
    KVCache, gqa_attention = _lib()
    B, hk, G = 3, 2, 4
    shape = W.Shape("ring", dt, B, hk * G, hk, d, C)
    cache = KVCache(B, hk, C, d, dtype=TORCH_DTYPE[dt], window=win)
    cache.set_policy(*policy)
    ref = window.RingCache(B, hk, C, d, win, dt)
    for i, call in enumerate(calls):
        T, n = call["T"], call["n_new"]
        q, k, v = W.step_inputs(shape, seed, i, T, n, pad="nan")
        cache.append(to_dev(k, dt), to_dev(v, dt), n)
        ref.append(k, v, n)
        assert cache.lens == ref.lens.tolist()
        if max(n) > 0:
            out = gqa_attention(to_dev(q, dt), cache, n)
            assert_close(out_f64(out, dt), window.attention(ref, q, n), dt, f"ring call {i} policy {policy}")
            raw = from_dev(out, dt)
            for b in range(B):
                assert not raw[b, :, n[b]:].view(np.uint8).any(), "padded slot not +0.0"
        assert same_bytes(from_dev(cache.k, dt), ref.k), f"K ring differs after call {i}"
        assert same_bytes(from_dev(cache.v, dt), ref.v), f"V ring differs after call {i}"
        if rollback_every and i % rollback_every == rollback_every - 1:
            # roll every row back by up to 3 tokens where the ring allows it
            new = []
            for b in range(B):
                L = int(ref.lens[b])
                cand = max(0, L - 3)
                new.append(cand if ref.lowest_needed(cand) >= ref.oldest_kept(L) else L)
            cache.truncate(new)
            ref.truncate(new)
    assert cache.lens_dev.cpu().tolist()[:B] == ref.lens.tolist()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d,C,win", [(16, 64, 1), (64, 128, 50), (128, 128, 128), (128, 192, 64), (32, 256, 200)])
def test_ring_schedule(dt, d, C, win):
    """Decode steps and chunks through a ring that wraps, under the automatic
    kernel choice, the split-K decode kernel with tiny splits and the chunked-
    prefill kernel with tiny splits (windows 1 .. capacity, not multiples of 64)."""
    calls, lens = W.ring_schedule(d + C + win, 3, C, win, 60, min(16, C - win + 1))
    for policy in [(0, 0), (1, 32), (2, 64)]:
        _run_ring(dt, d, C, win, policy, calls, 21, rollback_every=7)


def test_ring_refusals_change_nothing():
    """An append that would evict a key its first new query needs, and a rollback
    below what the ring holds, raise ValueError and leave cache and lengths as
    they were ([MASK] "Common mistakes": the window must never silently lose keys)."""
    KVCache, gqa_attention = _lib()
    C, win, d = 128, 64, 64
    cache = KVCache(1, 1, C, d, dtype=torch.float32, window=win)
    k = torch.randn(1, 1, 128, d, device="cuda")
    cache.append(k, k, [128])
    before = (cache.k.clone(), cache.lens)
    with pytest.raises(ValueError, match="evict"):
        cache.append(k, k, [66])
    cache.append(k[:, :, :65].contiguous(), k[:, :, :65].contiguous(), [65])   # holds 65 .. 192
    with pytest.raises(ValueError, match="Invalid truncation length"):
        cache.truncate([127])
    assert cache.lens == [193]
    cache.truncate([128])
    assert cache.lens == [128]
    assert before[1] == [128] and before[0].shape == cache.k.shape


def test_window_covering_the_cache_matches_the_linear_cache():
    """W = capacity and no wrap: the ring gives the same bits as a linear cache."""
    KVCache, gqa_attention = _lib()
    B, hk, G, d, C = 2, 2, 4, 128, 256
    shape = W.Shape("cover", "bf16", B, hk * G, hk, d, C)
    ring = KVCache(B, hk, C, d, window=C)
    lin = KVCache(B, hk, C, d)
    for i, (T, n) in enumerate([(100, [100, 37]), (1, [1, 1]), (64, [64, 0]), (4, [4, 4])]):
        q, k, v = W.step_inputs(shape, 3, i, T, n, pad="normal")
        for c in (ring, lin):
            c.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
        a = from_dev(gqa_attention(to_dev(q, "bf16"), ring, n), "bf16")
        b = from_dev(gqa_attention(to_dev(q, "bf16"), lin, n), "bf16")
        assert np.array_equal(a, b), i


def test_llama_window_decode():
    """Llama-3.1-8B-shaped decode (B=32, Hq=32, Hkv=8, d=128, bf16) with a
    4,096-key window over an 8,192-slot ring after 20,000 tokens: sampled rows
    against the oracle, and the wrapped ring contents bit for bit."""
    KVCache, gqa_attention = _lib()
    sh, seed = W.LLAMA8B_WINDOW_DECODE, 2
    B, hk, d, C, win = sh.batch, sh.kv_heads, sh.head_dim, sh.max_len, sh.notes["window"]
    L = sh.notes["cached"]
    cache = KVCache(B, hk, C, d, window=win)
    # positions 0 .. L-C-1 are overwritten before the step: device noise
    g = torch.Generator(device="cuda").manual_seed(5)
    done = 0
    while done < L - C:
        n = min(4096, L - C - done)
        noise = torch.randn(B, hk, n, d, device="cuda", generator=g).to(torch.bfloat16)
        cache.append(noise, noise, [n] * B)
        done += n
    # the last C positions from the seeded generator (the second chunk wraps)
    hist = []
    while done < L:
        n = min(4096, L - done)
        rows = [W.prefix_kv(sh, seed, b, done, n) for b in range(B)]
        kh = np.stack([r[0] for r in rows])
        vh = np.stack([r[1] for r in rows])
        cache.append(to_dev(kh, "bf16"), to_dev(vh, "bf16"), [n] * B)
        hist.append((done, kh, vh))
        done += n
    nn = [1] * B
    q, k, v = W.step_inputs(sh, seed, 10_000, 1, nn, pad="nan")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), nn)
    out = out_f64(gqa_attention(to_dev(q, "bf16"), cache, nn), "bf16")
    assert np.isfinite(out).all()
    for b in [0, 17, 31]:
        ks = np.zeros((hk, C, d), np.uint16)
        vs = np.zeros_like(ks)
        stored = np.full(C, -1, np.int64)
        for start, kh, vh in hist:
            pos = np.arange(start, start + kh.shape[2])
            ks[:, pos % C], vs[:, pos % C], stored[pos % C] = kh[b], vh[b], pos
        ks[:, L % C], vs[:, L % C], stored[L % C] = k[b, :, 0], v[b, :, 0], L
        assert same_bytes(from_dev(cache.k[b], "bf16"), ks), f"row {b}: ring K differs"
        ref = window.attention_row(ks, vs, stored, L + 1, 1, q[b], "bf16", win, [(h, 0) for h in range(sh.q_heads)])
        assert_close(out[b], ref, "bf16", f"window decode row {b}")


def test_windowed_chunked_prefill():
    """512-token chunks with a 1,000-key window through a 2,048-slot ring (the
    chunked-prefill kernel, window start not on a tile): sampled (head, query)
    pairs of every chunk against the oracle."""
    KVCache, gqa_attention = _lib()
    B, hk, G, d, C, win = 2, 8, 4, 128, 2048, 1000
    shape = W.Shape("wchunks", "bf16", B, hk * G, hk, d, C)
    cache = KVCache(B, hk, C, d, window=win)
    ref = window.RingCache(B, hk, C, d, win, "bf16")
    rng = np.random.default_rng(9)
    for i in range(10):
        n = [512, 512] if i % 3 else [512, 300]
        q, k, v = W.step_inputs(shape, 4, i, 512, n, pad="nan")
        cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
        ref.append(k, v, n)
        out = out_f64(gqa_attention(to_dev(q, "bf16"), cache, n), "bf16")
        for b in range(B):
            pairs = [(int(h), int(t)) for h, t in zip(rng.integers(0, hk * G, 24), rng.integers(0, n[b], 24))]
            pairs += [(0, 0), (hk * G - 1, n[b] - 1)]
            want = window.attention_row(ref.k[b], ref.v[b], ref.pos[b], int(ref.lens[b]), n[b], q[b], "bf16", win,
                                        pairs)
            sel = tuple(np.array(pairs).T)
            assert_close(out[b][sel], want[sel], "bf16", f"chunk {i} row {b}")
            assert not out[b, :, n[b]:].any()
    assert ref.lens.tolist()[0] > 2 * C
