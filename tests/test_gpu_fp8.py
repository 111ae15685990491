"""GPU parity of the E4M3 (FP8) KV cache with one scale per KV head.

The HIP path (KVCache(fp8_scales=...) -> kv_cache_create_fp8, kv_append,
gqa_attention through the C ABI) against oracle/fp8.py on the same seeded
bits: the stored codes bit for bit after every append (the quantization is an
integer decision taken in float32 on both sides), outputs within the bfloat16
contract. [CH16] "16. Prefill, decode and the KV cache", exercise 4.
"""

import numpy as np
import pytest
import torch

from oracle import fp8
import workloads as W
from gpu_util import assert_close, from_dev, out_f64, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    from gqa_attention_preallocated_amd import KVCache, gqa_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return KVCache, gqa_attention


def _codes(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_fp8_schedule(d):
    """Chunks and decode steps at every head dim under each kernel selection; one
    KV head's scale is small enough that its values saturate at +-448."""
    KVCache, gqa_attention = _lib()
    B, hk, G, S = 3, 2, 4, 256
    shape = W.Shape("fp8", "bf16", B, hk * G, hk, d, S)
    ks, vs = [0.05, 0.004], [0.02, 0.004]
    calls = [{"T": 70, "n_new": [70, 33, 0]}, {"T": 1, "n_new": [1, 1, 1]}, {"T": 5, "n_new": [5, 2, 5]},
             {"T": 40, "n_new": [3, 40, 17]}, {"T": 1, "n_new": [1, 0, 1]}, {"T": 64, "n_new": [64, 64, 64]}]
    for policy in [(0, 0), (1, 0), (2, 0), (1, 32), (2, 64)]:
        cache = KVCache(B, hk, S, d, fp8_scales=(ks, vs))
        cache.set_policy(*policy)
        ref = fp8.Fp8Cache(B, hk, S, d, ks, vs)
        for i, call in enumerate(calls):
            T, n = call["T"], call["n_new"]
            q, k, v = W.step_inputs(shape, 31, i, T, n, pad="nan")
            cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
            ref.append(k, v, n)
            assert np.array_equal(_codes(cache.k), ref.k), f"K codes differ after call {i} policy {policy}"
            assert np.array_equal(_codes(cache.v), ref.v), f"V codes differ after call {i} policy {policy}"
            out = gqa_attention(to_dev(q, "bf16"), cache, n)
            assert_close(out_f64(out, "bf16"), fp8.attention(ref, q, n), "bf16", f"call {i} policy {policy}")
            raw = from_dev(out, "bf16")
            for b in range(B):
                assert not raw[b, :, n[b]:].view(np.uint8).any(), "padded slot not +0.0"
    assert (ref.k[:, 1] == 0x7E).any() or (ref.k[:, 1] == 0xFE).any()      # saturation happened


def test_fp8_bytes_and_rejections():
    KVCache, gqa_attention = _lib()
    c = KVCache(2, 8, 1024, 128, fp8_scales=([0.01] * 8, [0.01] * 8))
    assert c.bytes == 2 * 2 * 8 * 1024 * 128          # one byte per element
    with pytest.raises(ValueError):
        KVCache(2, 2, 64, 64, fp8_scales=([0.01, 0.0], [0.01, 0.01]))
    with pytest.raises(ValueError):
        KVCache(2, 2, 64, 64, fp8_scales=([0.01], [0.01]))


def test_llama_fp8_decode():
    """Llama-3.1-8B-shaped decode (B=32, 4,096 cached + 1, Hq=32, Hkv=8, d=128)
    over an E4M3 cache: sampled rows against the oracle, codes of those rows
    bit for bit."""
    KVCache, gqa_attention = _lib()
    sh, seed = W.LLAMA8B_DECODE, 1
    B, hk, d = sh.batch, sh.kv_heads, sh.head_dim
    ks = [2.0 ** -9 + 1e-5 * h for h in range(hk)]
    vs = [2.0 ** -9 - 1e-5 * h for h in range(hk)]
    cache = KVCache(B, hk, sh.max_len, d, fp8_scales=(ks, vs))
    for start in range(0, 4096, 2048):
        rows = [W.prefix_kv(sh, seed, b, start, 2048) for b in range(B)]
        cache.append(to_dev(np.stack([r[0] for r in rows]), "bf16"), to_dev(np.stack([r[1] for r in rows]), "bf16"),
                     [2048] * B)
    n = [1] * B
    q, k, v = W.step_inputs(sh, seed, 10_000, 1, n, pad="nan")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
    out = out_f64(gqa_attention(to_dev(q, "bf16"), cache, n), "bf16")
    assert np.isfinite(out).all()
    for b in [0, 9, 31]:
        ref = fp8.Fp8Cache(1, hk, 4097, d, ks, vs)
        kh, vh = W.prefix_kv(sh, seed, b, 0, 4096)
        ref.append(np.concatenate([kh, k[b, :, :1]], axis=1)[None], np.concatenate([vh, v[b, :, :1]], axis=1)[None],
                   [4097])
        assert np.array_equal(_codes(cache.k[b, :, :4097]), ref.k[0]), f"row {b}: K codes differ"
        assert np.array_equal(_codes(cache.v[b, :, :4097]), ref.v[0]), f"row {b}: V codes differ"
        k64, v64 = ref.dequantized(0)
        want = fp8.attention_row(k64, v64, 4097, 1, q[b], "bf16", [(h, 0) for h in range(sh.q_heads)])
        assert_close(out[b], want, "bf16", f"fp8 decode row {b}")


def test_fp8_error_against_a_bf16_cache():
    """[CH16] exercise 4 measures the error of the FP8 cache against a bfloat16
    one over 1,000 decode steps. Here: 1,000 decode steps of a Llama-shaped
    row set (B=4, from 512 to 1,512 cached tokens), the attention outputs of
    the two caches compared at every step. With no model there are no logits:
    the error is taken on the attention output, relative to its largest
    value. E4M3 keeps 3 mantissa bits (a code is within 2^-4 of its value),
    but each output averages thousands of keys, so the measured worst is
    about 3%; the gate is about twice that."""
    KVCache, gqa_attention = _lib()
    B, hk, G, d, S = 4, 8, 4, 128, 2048
    shape = W.Shape("fp8err", "bf16", B, hk * G, hk, d, S, value_scale=1.0 / np.sqrt(128.0))
    sc = [2.0 ** -9] * hk
    c8 = KVCache(B, hk, S, d, fp8_scales=(sc, sc))
    c16 = KVCache(B, hk, S, d)
    q, k, v = W.step_inputs(shape, 6, 0, 512, [512] * B, pad="normal")
    for c in (c8, c16):
        c.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [512] * B)
    worst, total = 0.0, 0.0
    steps = 1000
    for step in range(1, steps + 1):
        q, k, v = W.step_inputs(shape, 6, step, 1, [1] * B, pad="normal")
        outs = []
        for c in (c8, c16):
            c.append(to_dev(k, "bf16"), to_dev(v, "bf16"), [1] * B)
            outs.append(out_f64(gqa_attention(to_dev(q, "bf16"), c, [1] * B), "bf16"))
        rel = float(np.abs(outs[0] - outs[1]).max() / np.abs(outs[1]).max())
        worst = max(worst, rel)
        total += rel
    print(f"fp8 vs bf16 cache, {steps} decode steps: worst relative error {worst:.4f}, "
          f"mean {total / steps:.4f}")
    assert worst < 0.065, worst
