"""GPU parity at small sizes: the HIP path through the C ABI against the CPU oracle.

Cache contents and lengths must match the oracle bit for bit after every call;
attention outputs within 1e-5 (float32) or 2e-2 plus the relative gate
(bfloat16). Each schedule also runs with the split-K decode kernel and the
chunked-prefill kernel forced, and with tiny key splits, so both kernels and the
split combine see every row class in float32.
"""

import numpy as np
import pytest
import torch

from oracle import direct
import workloads as W
from gpu_util import assert_close, from_dev, out_f64, same_bytes, to_dev, TORCH_DTYPE

pytestmark = pytest.mark.gpu

POLICIES = [(0, 0), (1, 0), (2, 0), (1, 32), (2, 64)]


def _lib():
    from gqa_attention_preallocated_amd import KVCache, gqa_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return KVCache, gqa_attention


def _run_schedule(shape, calls, seed, policy, check_bytes=True):
    KVCache, gqa_attention = _lib()
    dt = shape.dtype
    cache = KVCache(shape.batch, shape.kv_heads, shape.max_len, shape.head_dim, dtype=TORCH_DTYPE[dt])
    cache.set_policy(*policy)
    ref = direct.Cache(shape.batch, shape.kv_heads, shape.max_len, shape.head_dim, dt)
    k_ptr = cache.k.data_ptr()
    worst = 0.0
    for i, call in enumerate(calls):
        T, n = call["T"], call["n_new"]
        q, k, v = W.step_inputs(shape, seed, i, T, n, pad="nan")
        cache.append(to_dev(k, dt), to_dev(v, dt), n)
        ref.append(k, v, n)
        out = gqa_attention(to_dev(q, dt), cache, n)
        want = direct.attention(ref, q, n)
        got = out_f64(out, dt)
        err = assert_close(got, want, dt, f"{shape.name} call {i} policy {policy}")
        worst = max(worst, err or 0.0)
        # padded slots and empty rows are exactly +0.0
        raw = from_dev(out, dt)
        for b in range(shape.batch):
            pad = raw[b, :, n[b]:]
            assert not pad.view(np.uint8).any(), "padded slot not +0.0"
        assert cache.lens == ref.lens.tolist()
        assert cache.lens_dev.cpu().tolist()[: shape.batch] == ref.lens.tolist()
        if check_bytes:
            assert same_bytes(from_dev(cache.k, dt), ref.k), f"K differs after call {i}"
            assert same_bytes(from_dev(cache.v, dt), ref.v), f"V differs after call {i}"
    assert cache.k.data_ptr() == k_ptr          # allocated once, written in place
    return worst


@pytest.mark.parametrize("policy", POLICIES)
def test_tiny_fp32_schedule(policy):
    _run_schedule(W.TINY_FP32, W.tiny_schedule(0), 0, policy)


@pytest.mark.parametrize("seed", range(16))
def test_random_trials_fp32(seed):
    shape, calls = W.trial_spec(seed, head_dims=(16, 128))
    for policy in [(0, 0), (1, 32), (2, 64)]:
        _run_schedule(shape, calls, seed, policy, check_bytes=(policy == (0, 0)))


@pytest.mark.parametrize("seed", range(100, 112))
def test_random_trials_bf16(seed):
    shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
    shape = W.Shape(shape.name, "bf16", shape.batch, shape.q_heads, shape.kv_heads, shape.head_dim,
                    shape.max_len)
    for policy in [(0, 0), (1, 32), (2, 64)]:
        _run_schedule(shape, calls, seed, policy, check_bytes=(policy == (0, 0)))


def test_random_trials_wide():
    """200 more seeded schedules (shapes, group sizes, head dims 16..128, row
    mixes), each in float32 and bfloat16 under every kernel selection and the
    tiny key splits: 2,000 schedules against the oracle in one test (about 20 s)."""
    for seed in range(16, 216):
        shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
        for dt in ("f32", "bf16"):
            sh = W.Shape(shape.name, dt, shape.batch, shape.q_heads, shape.kv_heads, shape.head_dim,
                         shape.max_len)
            for policy in POLICIES:
                _run_schedule(sh, calls, seed, policy, check_bytes=(policy == (0, 0)))


@pytest.mark.parametrize("hk,G", [(1, 8), (1, 32), (4, 1), (2, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mqa_mha_and_odd_groups(hk, G, dtype):
    """MQA (one KV head) and MHA (G = 1) are the same code path."""
    shape = W.Shape(f"g{G}", dtype, 2, hk * G, hk, 64, 160)
    calls = [{"T": 70, "n_new": [70, 33]}, {"T": 1, "n_new": [1, 1]}, {"T": 5, "n_new": [5, 2]},
             {"T": 40, "n_new": [3, 40]}]
    for policy in [(0, 0), (1, 0), (2, 0)]:
        _run_schedule(shape, calls, 7, policy, check_bytes=False)


@pytest.mark.parametrize("hk,G,d", [(1, 128, 64), (2, 64, 128), (1, 65, 32)])
def test_largest_groups(hk, G, d):
    """The largest group sizes: G = 64 still fits a decode work item (64
    columns); above it every row runs on the prefill kernel (256 columns), up
    to the ABI's limit of G = 128."""
    shape = W.Shape(f"g{G}", "bf16", 2, hk * G, hk, d, 160)
    calls = [{"T": 70, "n_new": [70, 33]}, {"T": 1, "n_new": [1, 1]}, {"T": 5, "n_new": [5, 2]},
             {"T": 40, "n_new": [3, 40]}]
    for policy in [(0, 0), (1, 0), (2, 0), (1, 32)]:
        _run_schedule(shape, calls, 9, policy, check_bytes=False)


def test_split_count_invariance():
    """Many small key splits vs one split agree within float32 rounding."""
    KVCache, gqa_attention = _lib()
    shape = W.Shape("splits", "f32", 2, 8, 2, 128, 1024)
    cache = KVCache(2, 2, 1024, 128, dtype=torch.float32)
    _, k, v = W.step_inputs(shape, 3, 0, 900, [900, 611], pad="normal")
    cache.append(to_dev(k, "f32"), to_dev(v, "f32"), [900, 611])
    q, _, _ = W.step_inputs(shape, 3, 1, 4, [4, 4], pad="normal")
    outs = []
    for policy in [(1, 32), (1, 96), (1, 1024), (2, 64), (2, 1024)]:
        cache.set_policy(*policy)
        outs.append(out_f64(gqa_attention(to_dev(q, "f32"), cache, [4, 4]), "f32"))
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_prefill_many_key_tiles(dt, d):
    """The chunked-prefill kernel over items of many 64-key tiles (its staging
    ring and the split of work between waves), at every head dim: a long
    row fed 96 queries at a time beside two short rows that stop growing,
    with the kernel forced and with one split per row (final lengths 1,968, 131, 71)."""
    shape = W.Shape("tiles", dt, 3, 16, 2, d, 2048)
    calls = [{"T": 96, "n_new": [96, 96, 70]}, {"T": 64, "n_new": [64, 34, 0]},
             {"T": 96, "n_new": [96, 0, 0]}] + [{"T": 96, "n_new": [96, 0, 0]}] * 17 + \
            [{"T": 96, "n_new": [80, 1, 1]}]
    _run_schedule(shape, calls, 11, (2, 4096), check_bytes=False)


@pytest.mark.parametrize("policy", [(0, 0), (1, 32), (2, 64)])
def test_more_rows_than_one_launch(policy):
    """150 rows: every kernel (append, decode, prefill, combine, zero fill)
    is split over several launches of at most 64 rows, with decode, verify,
    prefill and idle rows mixed in each call and a rollback between calls."""
    B = 150
    shape = W.Shape("rows150", "bf16", B, 8, 2, 32, 512)
    rng = np.random.default_rng(12)
    first = rng.integers(1, 300, B)
    calls = [{"T": int(first.max()), "n_new": first.tolist()}]
    for _ in range(2):
        n = rng.choice([0, 1, 3, 40], B)
        calls.append({"T": 40, "n_new": n.tolist()})
    KVCache, gqa_attention = _lib()
    cache = KVCache(B, 2, 512, 32)
    cache.set_policy(*policy)
    ref = direct.Cache(B, 2, 512, 32, "bf16")
    for i, call in enumerate(calls):
        T, n = call["T"], call["n_new"]
        q, k, v = W.step_inputs(shape, 13, i, T, n, pad="nan")
        cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
        ref.append(k, v, n)
        out = gqa_attention(to_dev(q, "bf16"), cache, n)
        assert_close(out_f64(out, "bf16"), direct.attention(ref, q, n), "bf16", f"call {i} policy {policy}")
        raw = from_dev(out, "bf16")
        for b in range(B):
            assert not raw[b, :, n[b]:].view(np.uint8).any(), "padded slot not +0.0"
        assert same_bytes(from_dev(cache.k, "bf16"), ref.k) and same_bytes(from_dev(cache.v, "bf16"), ref.v)
        if i == 1:
            back = [max(0, L - 2) for L in cache.lens]
            cache.truncate(back)
            ref.truncate(back)
        assert cache.lens_dev.cpu().tolist()[:B] == ref.lens.tolist()


def test_nan_in_padding_and_stale_tail_never_leaks():
    """NaN in padded q/k/v slots and in the cache past each row's length must not
    reach the output (stale slots are never read)."""
    KVCache, gqa_attention = _lib()
    for dt in ["f32", "bf16"]:
        shape = W.Shape("nan", dt, 3, 8, 2, 128, 256)
        for policy in [(0, 0), (1, 32), (2, 64)]:
            cache = KVCache(3, 2, 256, 128, dtype=TORCH_DTYPE[dt])
            cache.set_policy(*policy)
            ref = direct.Cache(3, 2, 256, 128, dt)
            _, k, v = W.step_inputs(shape, 5, 0, 100, [100, 37, 0], pad="nan")
            cache.append(to_dev(k, dt), to_dev(v, dt), [100, 37, 0])
            ref.append(k, v, [100, 37, 0])
            cache.truncate([60, 37, 0])
            ref.truncate([60, 37, 0])
            for b, L in enumerate([60, 37, 0]):
                cache.k[b, :, L:] = float("nan")
                cache.v[b, :, L:] = float("nan")
            q2, k2, v2 = W.step_inputs(shape, 5, 1, 8, [3, 8, 0], pad="nan")
            cache.append(to_dev(k2, dt), to_dev(v2, dt), [3, 8, 0])
            ref.append(k2, v2, [3, 8, 0])
            got = out_f64(gqa_attention(to_dev(q2, dt), cache, [3, 8, 0]), dt)
            assert_close(got, direct.attention(ref, q2, [3, 8, 0]), dt, f"nan tail {dt} {policy}")


def test_deterministic_run_to_run():
    KVCache, gqa_attention = _lib()
    shape = W.Shape("det", "bf16", 4, 32, 8, 128, 2048)
    cache = KVCache(4, 8, 2048, 128)
    _, k, v = W.step_inputs(shape, 9, 0, 1500, [1500, 700, 1200, 64], pad="normal")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [1500, 700, 1200, 64])
    q, _, _ = W.step_inputs(shape, 9, 1, 64, [64, 4, 1, 64], pad="normal")
    qd = to_dev(q, "bf16")
    a = gqa_attention(qd, cache, [64, 4, 1, 64]).clone()
    b = gqa_attention(qd, cache, [64, 4, 1, 64]).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_no_device_allocation_on_the_hot_path():
    KVCache, gqa_attention = _lib()
    shape = W.Shape("alloc", "bf16", 4, 32, 8, 128, 4096)
    cache = KVCache(4, 8, 4096, 128)
    _, k, v = W.step_inputs(shape, 2, 0, 1024, [1024] * 4, pad="normal")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [1024] * 4)
    q, k1, v1 = W.step_inputs(shape, 2, 1, 1, [1] * 4, pad="normal")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k1, "bf16"), to_dev(v1, "bf16")
    out = torch.empty_like(qd)
    cache.append(kd, vd, [1] * 4)                   # size the workspace at the lengths attention sees
    ws = torch.empty(cache.workspace_bytes(32, 1, [1] * 4) + 1024, dtype=torch.uint8, device="cuda")
    cache.truncate([1024] * 4)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(5):
        cache.append(kd, vd, [1] * 4)
        gqa_attention(qd, cache, [1] * 4, out=out, workspace=ws)
        cache.truncate([1024] * 4)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before


def test_overflow_changes_nothing_on_device():
    KVCache, _ = _lib()
    shape = W.Shape("ovf", "bf16", 2, 8, 2, 64, 32)
    cache = KVCache(2, 2, 32, 64)
    _, k, v = W.step_inputs(shape, 1, 0, 30, [30, 20], pad="normal")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [30, 20])
    torch.cuda.synchronize()
    snap_k, snap_v = cache.k.clone(), cache.v.clone()
    with pytest.raises(ValueError, match=r"row 0: 33 tokens > max_len 32"):
        cache.append(to_dev(k[:, :, :3].copy(), "bf16"), to_dev(v[:, :, :3].copy(), "bf16"), [3, 3])
    torch.cuda.synchronize()
    assert torch.equal(cache.k.view(torch.int16), snap_k.view(torch.int16))
    assert torch.equal(cache.v.view(torch.int16), snap_v.view(torch.int16))
    assert cache.lens == [30, 20]
    assert cache.lens_dev.cpu().tolist() == [30, 20]
    with pytest.raises(ValueError, match="Invalid truncation length"):
        cache.truncate([31, 0])


def test_empty_inputs_give_zero_shapes():
    KVCache, gqa_attention = _lib()
    cache = KVCache(2, 2, 16, 32, dtype=torch.float32)
    q = torch.full((2, 4, 3, 32), float("nan"), device="cuda")
    out = gqa_attention(q, cache, [0, 0])          # empty cache, no new tokens
    assert torch.equal(out, torch.zeros_like(out))
    q0 = torch.zeros((2, 4, 0, 32), device="cuda")
    assert gqa_attention(q0, cache, [0, 0]).shape == (2, 4, 0, 32)
    c0 = KVCache(0, 2, 16, 32, dtype=torch.float32)
    assert gqa_attention(torch.zeros((0, 4, 3, 32), device="cuda"), c0, []).shape == (0, 4, 3, 32)


def test_bytes_accounting():
    KVCache, _ = _lib()
    cache = KVCache(32, 8, 8192, 128)
    assert cache.bytes == direct.kv_cache_bytes(1, 32, 8192, 8, 128, 2) == 2 ** 30
    assert cache.live_bytes == 0
    shape = W.Shape("b", "bf16", 32, 32, 8, 128, 8192)
    _, k, v = W.step_inputs(shape, 0, 0, 16, [16] * 32, pad="normal")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [16] * 32)
    assert cache.live_bytes == direct.kv_cache_bytes(1, 32, 16, 8, 128, 2)


def test_create_zero_fills_every_cache_kind():
    """kv_cache_create* set K, V (a paged cache: the pool) and the device lengths
    to zero on the stream ([GQA] "A strong answer" and [CH16] "Layout and
    validity" build the cache from zeros): buffers holding 0xFF bytes before
    the call read back as zeros, through the C ABI on caller-owned memory."""
    import ctypes
    from gqa_attention_preallocated_amd import _lib as L
    lib = L.load()
    _lib()
    B, hk, S, d = 3, 2, 128, 64
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream().cuda_stream)
    for kind in ["f32", "bf16", "ring", "fp8", "paged"]:
        elem = {"f32": 4, "bf16": 2, "ring": 2, "fp8": 1, "paged": 2}[kind]
        rows = 5 * 64 if kind == "paged" else B * S          # the paged pool: 5 pages of 64 tokens
        k = torch.full((rows * hk * d * elem,), 0xFF, dtype=torch.uint8, device="cuda")
        v = torch.full_like(k, 0xFF)
        lens = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        table = torch.full((B * 2,), 7, dtype=torch.int32, device="cuda")
        h = P()
        args = (P(k.data_ptr()), P(v.data_ptr()), P(lens.data_ptr()))
        if kind == "ring":
            st = lib.kv_cache_create_ring(B, hk, S, d, 1, 64, *args, stream, ctypes.byref(h))
        elif kind == "fp8":
            sc = (ctypes.c_float * hk)(*([0.1] * hk))
            st = lib.kv_cache_create_fp8(B, hk, S, d, sc, sc, *args, stream, ctypes.byref(h))
        elif kind == "paged":
            st = lib.kv_cache_create_paged(B, hk, 5, 64, 2, d, 1, *args[:2], P(table.data_ptr()), args[2], stream,
                                           ctypes.byref(h))
        else:
            st = lib.kv_cache_create(B, hk, S, d, 0 if kind == "f32" else 1, *args, stream, ctypes.byref(h))
        assert st == 0, lib.kv_last_error()
        torch.cuda.synchronize()
        assert not k.any() and not v.any(), kind
        assert lens.tolist() == [0] * B
        if kind == "paged":
            assert table.tolist() == [-1] * (B * 2)
        assert lib.kv_cache_destroy(h) == 0
