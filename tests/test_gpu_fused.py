"""GPU parity of kv_append_attention (append and attention in one call).

The fused call must leave exactly what kv_append followed by gqa_attention
leaves: the same output bits, the same cache bytes, the same host and device
lengths, after every call of a schedule with prefill chunks, decode and verify
steps, empty rows and a rollback, on every cache kind (float32, bfloat16,
sliding-window ring, paged, E4M3: the decode kernel stores the codes and
quantizes the new keys it reads exactly as the append kernel does) and under
each kernel selection. The
unfused pair is itself checked against the oracle elsewhere; the outputs here
are also checked against the oracle directly for the linear caches.
[GQA] "A strong answer" (each step appends at the row's length, then attends).
"""

import numpy as np
import pytest
import torch

from oracle import direct
import workloads as W
from gpu_util import TORCH_DTYPE, assert_close, fill_rows, from_dev, out_f64, to_dev

pytestmark = pytest.mark.gpu

POLICIES = [(0, 0), (1, 0), (2, 0), (1, 32), (2, 64)]


def _lib():
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return KVCache, append_attention, gqa_attention


def _make(KVCache, kind, B, hk, S, d):
    if kind == "f32":
        return KVCache(B, hk, S, d, dtype=torch.float32)
    if kind == "bf16":
        return KVCache(B, hk, S, d)
    if kind == "ring":
        return KVCache(B, hk, 256, d, window=64)
    if kind == "paged":
        return KVCache(B, hk, S, d, page_size=64, num_pages=B * S // 64)
    if kind == "fp8":
        return KVCache(B, hk, S, d, fp8_scales=([0.02 + 0.01 * h for h in range(hk)], [0.03] * hk))
    raise ValueError(kind)


def _same_state(a, b, what):
    torch.cuda.synchronize()
    assert a.lens == b.lens, f"{what}: lengths"
    assert torch.equal(a.lens_dev, b.lens_dev), f"{what}: device lengths"
    assert torch.equal(a.lens_dev[: a.batch].cpu(), torch.tensor(a.lens, dtype=torch.int32)), f"{what}: lens_dev"
    assert torch.equal(a.k.view(torch.uint8), b.k.view(torch.uint8)), f"{what}: K bytes"
    assert torch.equal(a.v.view(torch.uint8), b.v.view(torch.uint8)), f"{what}: V bytes"
    if a.page_size is not None:
        assert a.block_table == b.block_table, f"{what}: block table"


CALLS = [(70, [70, 33, 0]), (1, [1, 1, 1]), (5, [5, 2, 5]), (130, [3, 130, 64]), (1, [1, 0, 1]),
         "rollback", (64, [64, 64, 64]), (4, [4, 4, 1]), (190, [190, 7, 189]), (1, [1, 1, 1]),
         (16, [16, 3, 9])]


@pytest.mark.parametrize("kind", ["f32", "bf16", "ring", "paged", "fp8"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_fused_matches_append_then_attention(kind, d):
    KVCache, append_attention, gqa_attention = _lib()
    B, hk, G, S = 3, 2, 4, 768
    dt = "f32" if kind == "f32" else "bf16"
    shape = W.Shape("fused", dt, B, hk * G, hk, d, S)
    for policy in POLICIES:
        ref, fus = _make(KVCache, kind, B, hk, S, d), _make(KVCache, kind, B, hk, S, d)
        oracle = direct.Cache(B, hk, S, d, dt) if kind in ("f32", "bf16") else None
        for c in (ref, fus):
            c.set_policy(*policy)
        for i, call in enumerate(CALLS):
            what = f"{kind} d={d} policy {policy} call {i}"
            if call == "rollback":
                new = [L - L // 3 for L in ref.lens]
                ref.truncate(new)
                fus.truncate(new)
                if oracle is not None:
                    oracle.truncate(new)
                _same_state(ref, fus, what)
                continue
            T, n = call
            q, k, v = W.step_inputs(shape, 61, i, T, n, pad="nan")
            qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
            ref.append(kd, vd, n)
            want = gqa_attention(qd, ref, n)
            got = append_attention(fus, kd, vd, qd, n)
            _same_state(ref, fus, what)
            assert torch.equal(want.view(torch.uint8), got.view(torch.uint8)), f"{what}: output bits"
            raw = from_dev(got, dt)
            for b in range(B):
                assert not raw[b, :, n[b]:].view(np.uint8).any(), f"{what}: padded slot not +0.0"
            if oracle is not None:
                oracle.append(k, v, n)
                assert_close(out_f64(got, dt), direct.attention(oracle, q, n), dt, what)


@pytest.mark.parametrize("paged", [False, True])
def test_fused_llama_decode_verify_and_mixed(paged):
    """Llama-3.1-8B heads (8 KV heads, group 4, d = 128), bfloat16, rows of a
    few thousand keys: a decode step, a verify step and a mixed batch (decode,
    verify, prefill and idle rows) give the bits of the unfused pair."""
    KVCache, append_attention, gqa_attention = _lib()
    B, hk, G, d, S = 8, 8, 4, 128, 4608
    shape = W.Shape("fused_llama", "bf16", B, hk * G, hk, d, S)
    kw = dict(page_size=256, num_pages=B * S // 256) if paged else {}
    ref, fus = KVCache(B, hk, S, d, **kw), KVCache(B, hk, S, d, **kw)
    lens = [4000, 3001, 2500, 17, 4095, 1, 2048, 3333]
    fill_rows([ref, fus], shape, 71, lens)
    for step, (T, n) in enumerate([(1, [1] * B), (4, [4] * B), (300, [1, 4, 300, 0, 1, 64, 0, 4]), (1, [1] * B)]):
        q, k, v = W.step_inputs(shape, 71, 10 + step, T, n, pad="nan")
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        ref.append(kd, vd, n)
        want = gqa_attention(qd, ref, n)
        got = append_attention(fus, kd, vd, qd, n)
        _same_state(ref, fus, f"step {step}")
        assert torch.equal(want.view(torch.uint8), got.view(torch.uint8)), f"step {step}: output bits"


def test_fused_refusals_change_nothing():
    """A call refused for either half (capacity, head count, workspace) leaves
    the lengths, the device lengths and the cache bytes as they were."""
    KVCache, append_attention, gqa_attention = _lib()
    cache = KVCache(2, 2, 128, 64)
    k = torch.randn(2, 2, 100, 64, device="cuda").to(torch.bfloat16)
    cache.append(k, k, [100, 50])
    torch.cuda.synchronize()
    before = (cache.lens, cache.lens_dev.clone(), cache.k.clone(), cache.v.clone())
    q = torch.randn(2, 8, 40, 64, device="cuda").to(torch.bfloat16)
    kn = torch.randn(2, 2, 40, 64, device="cuda").to(torch.bfloat16)
    with pytest.raises(ValueError):                                    # row 0 would pass max_len
        append_attention(cache, kn, kn, q, [40, 1])
    with pytest.raises(ValueError):                                    # 5 query heads over 2 KV heads
        append_attention(cache, kn, kn, q[:, :5].contiguous(), [1, 1])
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):                                    # split rows need a workspace
        cache.set_policy(1, 32)
        append_attention(cache, kn, kn, q, [1, 1], workspace=ws)
    torch.cuda.synchronize()
    assert cache.lens == before[0]
    assert torch.equal(cache.lens_dev, before[1])
    assert torch.equal(cache.k, before[2]) and torch.equal(cache.v, before[3])


def test_fused_empty_inputs():
    """No new tokens, T = 0 and B = 0 give zeros of the right shape and change
    nothing; a row with no new tokens beside rows with some is zero-filled."""
    KVCache, append_attention, gqa_attention = _lib()
    cache = KVCache(2, 2, 16, 32, dtype=torch.float32)
    q = torch.full((2, 4, 3, 32), float("nan"), device="cuda")
    kn = torch.full((2, 2, 3, 32), float("nan"), device="cuda")
    out = append_attention(cache, kn, kn, q, [0, 0])       # empty cache, nothing appended
    assert torch.equal(out, torch.zeros_like(out))
    assert cache.lens == [0, 0]
    q0 = torch.zeros((2, 4, 0, 32), device="cuda")
    k0 = torch.zeros((2, 2, 0, 32), device="cuda")
    assert append_attention(cache, k0, k0, q0, [0, 0]).shape == (2, 4, 0, 32)
    c0 = KVCache(0, 2, 16, 32, dtype=torch.float32)
    z = torch.zeros((0, 4, 3, 32), device="cuda")
    assert append_attention(c0, torch.zeros((0, 2, 3, 32), device="cuda"),
                            torch.zeros((0, 2, 3, 32), device="cuda"), z, []).shape == (0, 4, 3, 32)
    kv = torch.randn(2, 2, 3, 32, device="cuda")
    qq = torch.randn(2, 4, 3, 32, device="cuda")
    out = append_attention(cache, kv, kv, qq, [2, 0])
    torch.cuda.synchronize()
    assert cache.lens == [2, 0]
    assert torch.equal(out[1], torch.zeros_like(out[1]))
    assert torch.equal(out[0, :, 2:], torch.zeros_like(out[0, :, 2:]))
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("seed", range(12))
def test_fused_random_trials(seed):
    """Seeded random shapes and schedules (1, 2 or 4 KV heads, G 1..8, 1..3 rows,
    chunks of 1..8 tokens, d in 16..128), each call made as one
    kv_append_attention and as kv_append + gqa_attention on a twin cache: the
    same output, cache and length bits, under each kernel selection."""
    KVCache, append_attention, gqa_attention = _lib()
    shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
    kind = ["f32", "bf16", "paged", "fp8"][seed % 4]
    dt = "f32" if kind == "f32" else "bf16"
    shape = W.Shape(shape.name, dt, shape.batch, shape.q_heads, shape.kv_heads, shape.head_dim, 64)
    B, hk, d = shape.batch, shape.kv_heads, shape.head_dim

    def make():
        if kind == "paged":
            return KVCache(B, hk, 64, d, page_size=64, num_pages=B)
        if kind == "fp8":
            return KVCache(B, hk, 64, d, fp8_scales=([0.05] * hk, [0.05] * hk))
        return KVCache(B, hk, 64, d, dtype=TORCH_DTYPE[dt])

    for policy in [(0, 0), (1, 32), (2, 64)]:
        ref, fus = make(), make()
        for c in (ref, fus):
            c.set_policy(*policy)
        for i, call in enumerate(calls):
            T, n = call["T"], call["n_new"]
            q, k, v = W.step_inputs(shape, 91 + seed, i, T, n, pad="nan")
            qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
            ref.append(kd, vd, n)
            want = gqa_attention(qd, ref, n)
            got = append_attention(fus, kd, vd, qd, n)
            what = f"seed {seed} {kind} policy {policy} call {i}"
            _same_state(ref, fus, what)
            assert torch.equal(want.view(torch.uint8), got.view(torch.uint8)), f"{what}: output bits"


@pytest.mark.parametrize("paged", [False, True])
def test_fused_tree_matches_append_then_tree_attention(paged):
    """kv_append_attention_tree: the draft tree's tokens appended and verified in
    one launch, with the bits of kv_append + gqa_attention_tree ([MASK] "What
    interviewers probe next"), rolled back after every step as a verifier does;
    refusals (a ring, a bad parent) change nothing."""
    KVCache, append_attention, gqa_attention = _lib()
    B, hk, G, d, S = 3, 2, 4, 128, 512
    shape = W.Shape("tree_fused", "bf16", B, hk * G, hk, d, S)
    kw = dict(page_size=64, num_pages=B * S // 64) if paged else {}
    ref, fus = KVCache(B, hk, S, d, **kw), KVCache(B, hk, S, d, **kw)
    base = [300, 17, 64]
    fill_rows([ref, fus], shape, 5, base)
    par = [[-1, 0, 1, 2, 0, 4, -1, 6], [-1, -1, 1, 1, 3, 0, 5, 2], [-1, 0, 0, 0, 1, 2, 3, 4]]
    for step, n in enumerate([[8, 8, 8], [5, 8, 0], [1, 2, 3]]):
        q, k, v = W.step_inputs(shape, 5, step, 8, n, pad="nan")
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        ref.append(kd, vd, n)
        want = gqa_attention(qd, ref, n, parents=par)
        got = append_attention(fus, kd, vd, qd, n, parents=par)
        _same_state(ref, fus, f"tree step {step}")
        assert torch.equal(want.view(torch.uint8), got.view(torch.uint8)), f"tree step {step}: output bits"
        ref.truncate(base)
        fus.truncate(base)
    torch.cuda.synchronize()
    before = (fus.lens, fus.k.clone(), fus.v.clone())
    q, k, v = W.step_inputs(shape, 5, 9, 8, [8, 8, 8], pad="nan")
    with pytest.raises(ValueError):                    # node 3's parent is not an earlier node
        append_attention(fus, to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(q, "bf16"), [8, 8, 8],
                         parents=[[-1, 0, 1, 3, 0, 4, -1, 6]] * 3)
    torch.cuda.synchronize()
    assert fus.lens == before[0] and torch.equal(fus.k, before[1]) and torch.equal(fus.v, before[2])
    ring = KVCache(B, hk, 256, d, window=64)
    with pytest.raises(ValueError):                    # tree verify runs on linear caches
        append_attention(ring, to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(q, "bf16"), [1, 1, 1],
                         parents=[[-1] * 8] * 3)
    assert ring.lens == [0, 0, 0]
