"""Byte offsets past 2^32: caches of 8 GiB per tensor.

B=2 rows, 8 KV heads, d=128: a linear bfloat16 cache with max_len 2^21, a
paged bfloat16 pool of the same size (pages of 256 tokens, the two rows'
pages interleaved), and an E4M3 cache with max_len 2^22 (one byte per
element). K and V are 2^33 bytes each, so the second row's keys sit past
4 GiB and the last (row, KV head)'s past 7.5 GiB (in the pool, the last
pages). Every key is zero except two marked ones per (row, KV
head): one near the start of the row and one near its end, with distinct V
rows per (row, KV head). With q along the first axis, a query's output has a
closed form (the definition of softmax attention, [GQA] "A strong answer":
zero-score keys with zero V add weight 1 each and nothing to the sum):

    out = (e^{s1} v1 + e^{s2} v2) / (e^{s1} + e^{s2} + N - 2)

with N the keys the query sees. A key read from a wrapped 32-bit offset (a
zero row instead of a marked one, or another head's) moves the output by
far more than the tolerance. The append path is checked byte for byte at the
marked rows, and the decode (split-K rows merged across work groups) and
prefill kernels are checked at every head and query.
"""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

B, HKV, G, D = 2, 8, 4, 128
HQ = HKV * G
CH = 1 << 16                     # tokens per append call
PAGE = 256
K1, K2 = 2.0, 3.0                # their keys: K1 or K2 at d = 0, zero elsewhere
QA = 11.3125                     # q = (QA, 0, ...): bfloat16 nearest to sqrt(128)


def _v_rows():
    """Distinct V rows per (row, KV head), exact in bfloat16."""
    v1 = np.zeros((B, HKV, D))
    v2 = np.zeros((B, HKV, D))
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    half = np.where(np.arange(D) < D // 2, 1.0, -0.5)
    for b in range(B):
        for h in range(HKV):
            i = b * HKV + h
            v1[b, h] = (i % 5 + 1) * 0.25 * sign
            v2[b, h] = (i % 3 + 1) * 0.5 * half
    return v1, v2


def _expected(v1, v2, n_keys):
    """out[b, hq, :] for a query that sees n_keys keys (both marked ones among them)."""
    s1, s2 = QA * K1 / math.sqrt(D), QA * K2 / math.sqrt(D)
    w1, w2 = math.exp(s1), math.exp(s2)
    o = (w1 * v1 + w2 * v2) / (w1 + w2 + (n_keys - 2))        # [B, HKV, D]
    return np.repeat(o, G, axis=1)                              # query head hq uses KV head hq // G


def _check(got, want, what):
    scale = np.abs(want).max(axis=-1, keepdims=True)
    err = np.abs(got - want) / scale
    assert err.max() < 2e-2, f"{what}: worst error {err.max():.3g} of the row's largest output"


def _row_view(cache, kind, x, j):
    """[B, HKV, D] stored rows of position j (codes for E4M3, as floats)."""
    if kind == "paged":
        tbl = cache.block_table
        rows = [x[tbl[b][j // PAGE], :, j % PAGE, :] for b in range(B)]
        return torch.stack(rows).float().cpu().numpy()
    return x[:, :, j, :].float().cpu().numpy()


@pytest.mark.parametrize("kind", ["linear", "paged", "fp8"])
def test_offsets_past_4GiB(kind):
    from gqa_attention_preallocated_amd import KVCache, append_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v1, v2 = _v_rows()
    L = 1 << (22 if kind == "fp8" else 21)       # max_len
    F = L - 128                                  # keys appended before the attention calls
    J1, J2 = 1000, F - 300                       # the two marked positions of every (row, KV head)
    if kind == "paged":
        cache = KVCache(B, HKV, L, D, page_size=PAGE, num_pages=B * L // PAGE)
    elif kind == "fp8":
        # unit scales: the marked values are exact E4M3 codes
        cache = KVCache(B, HKV, L, D, fp8_scales=([1.0] * HKV, [1.0] * HKV))
    else:
        cache = KVCache(B, HKV, L, D)
    assert cache.k.numel() * cache.k.element_size() == 1 << 33
    kz = torch.zeros((B, HKV, CH, D), dtype=torch.bfloat16, device="cuda")
    vz = torch.zeros_like(kz)
    print(f"filling {B} rows to {F} keys", flush=True)
    for start in range(0, F, CH):
        n = min(CH, F - start)
        k, v = kz, vz
        marks = [(j, kk, vv) for j, kk, vv in ((J1, K1, v1), (J2, K2, v2)) if start <= j < start + n]
        if marks:
            k, v = kz.clone(), vz.clone()
            for j, kk, vv in marks:
                k[:, :, j - start, 0] = kk
                v[:, :, j - start, :] = torch.tensor(vv, dtype=torch.bfloat16, device="cuda")
        cache.append(k, v, [n] * B)
    torch.cuda.synchronize()
    assert cache.lens == [F] * B

    # the append wrote the marked rows where they belong, past 4 GiB too (an
    # E4M3 row: nonzero codes exactly where the values are nonzero)
    for j, kk, vv in ((J1, K1, v1), (J2, K2, v2)):
        want_k = np.zeros((B, HKV, D))
        want_k[:, :, 0] = kk
        krow, vrow = _row_view(cache, kind, cache.k, j), _row_view(cache, kind, cache.v, j)
        if kind == "fp8":
            assert np.array_equal(krow != 0, want_k != 0) and np.array_equal(vrow != 0, vv != 0), f"codes at {j}"
        else:
            assert np.array_equal(krow, want_k), f"K rows at position {j}"
            assert np.array_equal(vrow, vv), f"V rows at position {j}"
    assert not _row_view(cache, kind, cache.k, F - 1).any() and not _row_view(cache, kind, cache.v, F - 1).any()
    if kind == "paged":
        last = max(max(row) for row in cache.block_table)
        assert last == B * L // PAGE - 1, "the pool's last page holds keys"

    # decode step: one new (zero) token per row, attention over F + 1 keys
    kn = torch.zeros((B, HKV, 1, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, HQ, 1, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = QA
    print("decode step", flush=True)
    out = append_attention(cache, kn, kn.clone(), q, [1] * B)
    torch.cuda.synchronize()
    _check(out[:, :, 0].float().cpu().numpy(), _expected(v1, v2, F + 1), "decode")

    # a 64-token chunk per row (prefill kernel): query t sees F + 2 + t keys
    T = 64
    kn = torch.zeros((B, HKV, T, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, HQ, T, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = QA
    print("prefill chunk", flush=True)
    out = append_attention(cache, kn, kn.clone(), q, [T] * B)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for t in range(T):
        _check(got[:, :, t], _expected(v1, v2, F + 2 + t), f"prefill query {t}")
    assert cache.lens == [F + 1 + T] * B
