"""Pins for the CPU oracle: facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (fixtures under tests/golden/, each citing its page and section),
closed forms, library routines for special cases (torch's scaled dot-product
attention, numpy's tril/repeat/mean) and brute-force invariants. The planted
mistake tests at the end patch one plausible error into the oracle at a time and
require that some pin here fails.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden, read_golden_rows
from oracle import direct, vectorised
import workloads as W


def _fill(c, k, v):
    """Append whole rows [B, Hkv, n, d] to an empty oracle cache."""
    n = np.full(c.batch, k.shape[2])
    c.append(k, v, n)


# --------------------------------------------------------------------------
# the mask: printed examples and closed forms
# --------------------------------------------------------------------------

def test_rectangle_mask_matches_printed_example():
    rows = read_golden_rows("rectangle_mask_prefix3_chunk2.txt")
    m = direct.decode_causal_mask(2, 5)
    for i, r in enumerate(rows):
        assert direct.query_position(5, 2, i) == r[0]
        assert m[i].astype(int).tolist() == r[1:]


@pytest.mark.parametrize("S", [1, 2, 37, 4096])
def test_single_decode_row_is_all_ones(S):
    assert direct.decode_causal_mask(1, S).all()


@pytest.mark.parametrize("S", [1, 5, 37])
def test_prefill_from_empty_is_tril(S):
    assert np.array_equal(direct.decode_causal_mask(S, S), np.tril(np.ones((S, S), bool)))


def test_verify_mask_counts():
    g = read_golden("mask_page_numbers.txt")
    T, S = g["verify_T"], g["verify_S"]
    m = direct.decode_causal_mask(T, S)
    assert m.size == g["verify_total"]
    assert (~m).sum() == g["verify_masked"]
    assert (~m).sum() == T * (T - 1) // 2           # closed form of the corner triangle
    for i in range(T):
        assert m[i].sum() == g["verify_offset"] + i + 1


@pytest.mark.parametrize("T,S", [(1, 1), (3, 7), (5, 37), (8, 8), (2, 40)])
def test_mask_is_lower_right_tril(T, S):
    # numpy's tril with diagonal offset S - T is the bottom-right triangle
    ref = np.tril(np.ones((T, S), bool), k=S - T)
    assert np.array_equal(direct.decode_causal_mask(T, S), ref)


# --------------------------------------------------------------------------
# chunked feeding equals whole-sequence attention
# --------------------------------------------------------------------------

def _chunk_vs_full(S, T, d=16, hk=2, G=2, seed=7, dtype="f32"):
    rng = np.random.default_rng(seed)
    k = W.draw(rng, (1, hk, S, d), dtype)
    v = W.draw(rng, (1, hk, S, d), dtype)
    q = W.draw(rng, (1, hk * G, S, d), dtype)
    full = direct.Cache(1, hk, 64, d, dtype)
    _fill(full, k, v)
    out_full = direct.attention(full, q, [S])
    inc = direct.Cache(1, hk, 64, d, dtype)
    _fill(inc, k[:, :, :S - T], v[:, :, :S - T])
    inc.append(k[:, :, S - T:], v[:, :, S - T:], [T])
    out_inc = direct.attention(inc, q[:, :, S - T:], [T])
    return out_full[:, :, S - T:], out_inc


def test_incremental_chunk_equals_full_exactly():
    g = read_golden("mask_page_numbers.txt")
    a, b = _chunk_vs_full(g["chunk_S"], g["chunk_T"])
    assert np.abs(a - b).max() == g["chunk_max_abs_diff"]


def test_three_way_feed_agrees():
    """Whole sequence vs prefix + chunk + single tokens through one cache.

    "16. Prefill, decode and the KV cache", section "Prove equivalence".
    """
    S, d, hk, G = 23, 16, 2, 3
    rng = np.random.default_rng(11)
    k = W.draw(rng, (1, hk, S, d), "f32")
    v = W.draw(rng, (1, hk, S, d), "f32")
    q = W.draw(rng, (1, hk * G, S, d), "f32")
    whole = direct.Cache(1, hk, 32, d)
    _fill(whole, k, v)
    ref = direct.attention(whole, q, [S])
    c = direct.Cache(1, hk, 32, d)
    pieces = [(0, 9), (9, 16)] + [(i, i + 1) for i in range(16, S)]
    got = np.zeros_like(ref)
    for lo, hi in pieces:
        c.append(k[:, :, lo:hi], v[:, :, lo:hi], [hi - lo])
        got[:, :, lo:hi] = direct.attention(c, q[:, :, lo:hi], [hi - lo])
    assert np.abs(got - ref).max() <= 1e-12


# --------------------------------------------------------------------------
# special cases that reduce to a library routine
# --------------------------------------------------------------------------

def _sdpa(q64, k64, v64, T, S, gqa):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q64, k64, v64))
    mask = torch.ones(T, S, dtype=torch.bool).tril(diagonal=S - T)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, enable_gqa=gqa).numpy()


@pytest.mark.parametrize("G", [1, 4])
def test_prefill_from_empty_matches_torch_causal(G):
    S, d, hk = 19, 16, 2
    rng = np.random.default_rng(3)
    k = W.draw(rng, (2, hk, S, d), "f32")
    v = W.draw(rng, (2, hk, S, d), "f32")
    q = W.draw(rng, (2, hk * G, S, d), "f32")
    c = direct.Cache(2, hk, 32, d)
    _fill(c, k, v)
    ours = direct.attention(c, q, [S, S])
    qt, kt, vt = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           enable_gqa=(G > 1)).numpy()
    assert np.abs(ours - ref).max() <= 1e-12


@pytest.mark.parametrize("G,T,S", [(1, 5, 37), (4, 5, 37), (8, 1, 30), (2, 8, 9)])
def test_chunk_matches_torch_lower_right(G, T, S):
    d, hk = 16, 2
    rng = np.random.default_rng(5)
    k = W.draw(rng, (1, hk, S, d), "f32")
    v = W.draw(rng, (1, hk, S, d), "f32")
    q = W.draw(rng, (1, hk * G, T, d), "f32")
    c = direct.Cache(1, hk, 40, d)
    _fill(c, k[:, :, :S - T], v[:, :, :S - T])
    c.append(k[:, :, S - T:], v[:, :, S - T:], [T])
    ours = direct.attention(c, q, [T])
    ref = _sdpa(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), T, S, G > 1)
    assert np.abs(ours - ref).max() <= 1e-12


def test_chunk_matches_torch_causal_lower_right_bias():
    from torch.nn.attention.bias import causal_lower_right
    T, S, d, G, hk = 4, 11, 16, 2, 1
    rng = np.random.default_rng(9)
    k = W.draw(rng, (1, hk, S, d), "f32")
    v = W.draw(rng, (1, hk, S, d), "f32")
    q = W.draw(rng, (1, hk * G, T, d), "f32")
    c = direct.Cache(1, hk, 16, d)
    _fill(c, k, v)
    ours = direct.attention(c, q, [T])
    kt = torch.from_numpy(np.repeat(k, G, axis=1).astype(np.float64))
    vt = torch.from_numpy(np.repeat(v, G, axis=1).astype(np.float64))
    qt = torch.from_numpy(q.astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=causal_lower_right(T, S)).numpy()
    assert np.abs(ours - ref).max() <= 1e-12


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_zero_query_gives_prefix_mean():
    """q = 0 makes every visible score equal, so out = mean of V over keys 0..pos."""
    hk, G, d = 2, 3, 16
    rng = np.random.default_rng(1)
    c = direct.Cache(2, hk, 40, d)
    k = W.draw(rng, (2, hk, 20, d), "f32")
    v = W.draw(rng, (2, hk, 20, d), "f32")
    c.append(k, v, [20, 13])
    # chunk: row 0 gets 6 new tokens (positions 14..19), row 1 gets 2 (11..12)
    c.truncate([14, 11])
    c.append(k[:, :, 14:20], v[:, :, 14:20], [6, 2])
    T = 6
    q = np.zeros((2, hk * G, T, d), np.float32)
    out = direct.attention(c, q, [6, 2])
    for b, (L, n) in enumerate([(20, 6), (13, 2)]):
        for h in range(hk * G):
            for t in range(T):
                if t >= n:
                    assert not out[b, h, t].any()
                    continue
                pos = L - n + t
                want = c.v[b, h // G, :pos + 1].astype(np.float64).mean(axis=0)
                assert np.abs(out[b, h, t] - want).max() <= 1e-12


def test_constant_values_give_that_constant():
    hk, G, d = 2, 2, 16
    rng = np.random.default_rng(2)
    c = direct.Cache(1, hk, 32, d)
    k = W.draw(rng, (1, hk, 17, d), "f32")
    v = np.full((1, hk, 17, d), 0.625, np.float32)
    c.append(k, v, [17])
    q = W.draw(rng, (1, hk * G, 17, d), "f32")
    out = direct.attention(c, q, [17])
    assert np.abs(out - 0.625).max() <= 1e-12


def test_head_labelled_values_pin_the_head_map():
    """V of KV head k holds k+1 everywhere, so query head h must output h//G + 1.

    Distinguishes h // G from h % Hkv ("Implement grouped-query attention ...",
    section "Common mistakes").
    """
    hk, G, d = 4, 3, 16
    rng = np.random.default_rng(4)
    c = direct.Cache(1, hk, 16, d)
    k = W.draw(rng, (1, hk, 9, d), "f32")
    v = np.broadcast_to((np.arange(hk, dtype=np.float32) + 1)[None, :, None, None], (1, hk, 9, d)).copy()
    c.append(k, v, [9])
    q = W.draw(rng, (1, hk * G, 9, d), "f32")
    out = direct.attention(c, q, [9])
    for h in range(hk * G):
        assert np.abs(out[0, h] - (h // G + 1)).max() <= 1e-12


def test_dominant_key_selects_its_value_row():
    """Make one visible key's score dominate: the output is that key's V row."""
    hk, G, d, S = 1, 2, 16, 12
    rng = np.random.default_rng(8)
    k = W.draw(rng, (1, hk, S, d), "f32") * np.float32(1e-3)
    v = W.draw(rng, (1, hk, S, d), "f32")
    q = np.zeros((1, hk * G, 1, d), np.float32)
    q[..., 0] = 1.0
    hot = 5
    k[0, 0, hot, 0] = 2000.0        # score 2000 / 4 = 500 above the rest
    c = direct.Cache(1, hk, 16, d)
    _fill(c, k, v)
    c.truncate(S - 1)
    c.append(k[:, :, S - 1:], v[:, :, S - 1:], [1])
    out = direct.attention(c, q, [1])
    assert np.abs(out[0, :, 0] - v[0, 0, hot].astype(np.float64)).max() <= 1e-12


def test_repeat_of_kv_heads_matches_numpy_repeat():
    hk, G = 3, 4
    heads = [direct.kv_head_of(h, G) for h in range(hk * G)]
    assert heads == np.repeat(np.arange(hk), G).tolist()
    assert heads != np.tile(np.arange(hk), G).tolist()


# --------------------------------------------------------------------------
# zeros, never NaN
# --------------------------------------------------------------------------

def test_empty_batch_and_empty_cache_give_zeros():
    c0 = direct.Cache(0, 2, 8, 16)
    assert direct.attention(c0, np.zeros((0, 4, 3, 16), np.float32), []).shape == (0, 4, 3, 16)
    c = direct.Cache(2, 2, 8, 16)
    q = np.full((2, 4, 3, 16), np.nan, np.float32)
    out = direct.attention(c, q, [0, 0])
    assert out.shape == (2, 4, 3, 16) and not out.any()
    assert not np.isnan(vectorised.attention(c.k, c.v, c.lens, q, [0, 0], "f32")).any()


def test_padded_slots_are_zero_and_nan_never_leaks():
    shape = W.Shape("pad", "f32", 2, 4, 2, 16, 32)
    c = direct.Cache(2, 2, 32, 16)
    q, k, v = W.step_inputs(shape, 3, 0, 6, [6, 2], pad="nan")
    c.append(k, v, [6, 2])
    q, _, _ = W.step_inputs(shape, 3, 1, 6, [6, 2], pad="nan")
    out = direct.attention(c, q, [6, 2])
    assert np.isfinite(out).all()
    assert not out[1, :, 2:].any()
    out2 = vectorised.attention(c.k, c.v, c.lens, q, [6, 2], "f32")
    assert np.isfinite(out2).all()


# --------------------------------------------------------------------------
# the cache: append, overflow, truncate, bytes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_writes_exact_bits_in_place(dtype):
    shape = W.Shape("app", dtype, 3, 4, 2, 16, 24)
    c = direct.Cache(3, 2, 24, 16, dtype)
    k_id = id(c.k)
    before_k = c.k.copy()
    q, k, v = W.step_inputs(shape, 1, 0, 5, [5, 0, 3], pad="nan")
    c.append(k, v, [5, 0, 3])
    assert id(c.k) == k_id                      # allocated once, written in place
    expect = before_k.copy()
    expect[0, :, 0:5] = k[0, :, :5]
    expect[2, :, 0:3] = k[2, :, :3]
    assert np.array_equal(c.k.view(np.uint8), expect.view(np.uint8))
    assert c.lens.tolist() == [5, 0, 3]
    c.append(k, v, [1, 2, 0])
    assert np.array_equal(c.v[0, :, 5].view(np.uint8), v[0, :, 0].view(np.uint8))
    assert np.array_equal(c.v[1, :, 0:2].view(np.uint8), v[1, :, 0:2].view(np.uint8))
    assert c.lens.tolist() == [6, 2, 3]


def test_overflow_on_last_row_raises_and_changes_nothing():
    shape = W.Shape("ovf", "f32", 2, 2, 1, 16, 8)
    c = direct.Cache(2, 1, 8, 16)
    _, k, v = W.step_inputs(shape, 2, 0, 6, [6, 6], pad="normal")
    c.append(k, v, [6, 6])
    snap_k, snap_v, snap_l = c.k.copy(), c.v.copy(), c.lens.copy()
    _, k2, v2 = W.step_inputs(shape, 2, 1, 3, [3, 3], pad="normal")
    with pytest.raises(ValueError, match=r"row 1: 9 tokens > max_len 8"):
        c.append(k2, v2, [2, 3])
    assert np.array_equal(c.k.view(np.uint8), snap_k.view(np.uint8))
    assert np.array_equal(c.v.view(np.uint8), snap_v.view(np.uint8))
    assert c.lens.tolist() == snap_l.tolist()
    c.append(k2, v2, [2, 0])                 # exactly full is allowed
    c.append(k2, v2, [0, 2])
    assert c.lens.tolist() == [8, 8]
    c.append(k2, v2, [0, 0])                 # zero tokens at max_len is not an overflow


def test_bad_n_new_rejected():
    c = direct.Cache(1, 1, 8, 16)
    k = np.zeros((1, 1, 2, 16), np.float32)
    with pytest.raises(ValueError):
        c.append(k, k, [3])
    with pytest.raises(ValueError):
        c.append(k, k, [-1])


def test_truncate_rolls_back_without_copy():
    shape = W.Shape("tr", "f32", 2, 2, 1, 16, 16)
    c = direct.Cache(2, 1, 16, 16)
    _, k, v = W.step_inputs(shape, 4, 0, 8, [8, 5], pad="normal")
    c.append(k, v, [8, 5])
    snap = c.k.copy()
    c.truncate([3, 5])
    assert c.lens.tolist() == [3, 5]
    assert np.array_equal(c.k, snap)                 # stale data stays
    with pytest.raises(ValueError, match="Invalid truncation length"):
        c.truncate([4, 5])
    with pytest.raises(ValueError, match="Invalid truncation length"):
        c.truncate(-1)
    c.reset()
    assert c.lens.tolist() == [0, 0]


def test_stale_tail_after_truncate_is_never_read():
    """After a rollback the old tokens stay in the buffer but attention must not see them."""
    hk, G, d = 1, 2, 16
    rng = np.random.default_rng(12)
    k = W.draw(rng, (1, hk, 10, d), "f32")
    v = W.draw(rng, (1, hk, 10, d), "f32")
    c = direct.Cache(1, hk, 16, d)
    _fill(c, k, v)
    c.truncate(6)
    c.k[0, :, 6:] = np.nan
    c.v[0, :, 6:] = np.nan
    q = W.draw(rng, (1, hk * G, 2, d), "f32")
    out = direct.attention(c, q, [2])
    assert np.isfinite(out).all()
    fresh = direct.Cache(1, hk, 16, d)
    _fill(fresh, k[:, :, :6], v[:, :, :6])
    assert np.array_equal(out, direct.attention(fresh, q, [2]))


def test_kv_bytes_closed_forms():
    g = read_golden("kv_bytes.txt")
    per_tok = direct.kv_cache_bytes(32, 1, 1, 8, 128, 2)
    assert per_tok == g["llama31_8b_bytes_per_token"]
    assert direct.kv_cache_bytes(32, 1, 4096, 8, 128) == g["llama31_8b_final_cache_4096"]
    assert direct.kv_cache_bytes(32, 32, 8192, 8, 128) == g["llama31_8b_reserve_32x8192"]
    assert sum(range(4096)) == g["concat_tokens_copied_4096"]
    qwen = direct.kv_cache_bytes(28, 1, 1, 8, 128, 2)
    assert qwen == g["qwen3_06b_bytes_per_token_kib"] * 1024
    assert direct.kv_cache_bytes(28, 1, 2048, 8, 128) == g["qwen3_06b_2048_tokens_mib"] * 2**20
    assert direct.kv_cache_bytes(28, 1, 32768, 8, 128) == g["qwen3_06b_32k_tokens_gib"] * 2**30
    assert direct.kv_cache_bytes(32, 1, 8192, 8, 128) == g["eightb_8k_gqa8_gib"] * 2**30
    assert direct.kv_cache_bytes(32, 1, 8192, 32, 128) == g["eightb_8k_mha32_gib"] * 2**30


def test_cache_bytes_is_the_reservation():
    c = direct.Cache(32, 8, 8192, 128, "bf16")
    # one layer of the 32 x 8,192 reservation: 1/32 of 32 GiB
    assert c.bytes == direct.kv_cache_bytes(1, 32, 8192, 8, 128, 2) == 2**30
    assert c.live_bytes == 0


def test_bf16_storage_is_widened_exactly():
    """Generator rounding + oracle widening equal torch's float32 -> bfloat16 -> float64."""
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(4096).astype(np.float32) * np.float32(3.0),
                        np.array([1.0, -2.5, 3.140625, 1e-30, 65280.0, 1.00390625, 1.01171875],
                                 np.float32)])   # the last two are exact bf16 ties
    got = direct.to_float64(W.to_bf16_bits(x), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# planted mistakes: each must make some pin above fail
# --------------------------------------------------------------------------

def _pins_pass():
    """Run the discriminating pins; return True only if all hold."""
    checks = [
        test_rectangle_mask_matches_printed_example,
        test_incremental_chunk_equals_full_exactly,
        test_head_labelled_values_pin_the_head_map,
        test_zero_query_gives_prefix_mean,
        test_dominant_key_selects_its_value_row,
        lambda: test_chunk_matches_torch_lower_right(4, 5, 37),
        test_verify_mask_counts,
    ]
    for f in checks:
        try:
            f()
        except Exception:
            return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


def test_planted_top_left_mask_is_caught(monkeypatch):
    monkeypatch.setattr(direct, "query_position", lambda length, n_new, t: t)
    assert not _pins_pass()
    # the top-left row 0 of the verify step sees key 0 only
    g = read_golden("mask_page_numbers.txt")
    m = direct.decode_causal_mask(g["verify_T"], g["verify_S"])
    assert m[0].sum() == g["topleft_row0_visible"]


def test_planted_top_left_gives_finite_large_error(monkeypatch):
    good_full, _ = _chunk_vs_full(37, 5)
    monkeypatch.setattr(direct, "query_position", lambda length, n_new, t: t)
    _, bad_inc = _chunk_vs_full(37, 5)
    assert np.isfinite(bad_inc).all()          # silent: no crash, no NaN
    assert np.abs(bad_inc - good_full).max() > 0.1


def test_planted_modulo_head_map_is_caught(monkeypatch):
    # h % Hkv for the 4-KV-head case of the head-labelled pin
    monkeypatch.setattr(direct, "kv_head_of", lambda h, G: h % 4)
    assert not _pins_pass()


def test_planted_missing_offset_is_caught(monkeypatch):
    monkeypatch.setattr(direct, "query_position", lambda length, n_new, t: length + t)
    assert not _pins_pass()


def test_planted_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(direct, "query_position", lambda length, n_new, t: length - n_new + t - 1)
    assert not _pins_pass()


def test_planted_missing_scale_is_caught(monkeypatch):
    real = direct.attend_one

    def unscaled(keys, values, q, head_dim):
        return real(keys, values, q * math.sqrt(head_dim), head_dim)

    monkeypatch.setattr(direct, "attend_one", unscaled)
    assert not _pins_pass()


def test_planted_length_before_write_is_caught(monkeypatch):
    """Advancing the length before the check leaves a failed append claiming tokens."""
    real = direct.Cache.append

    def early(self, k_new, v_new, n_new):
        for b in range(self.batch):
            self.lens[b] += int(n_new[b])
            if self.lens[b] > self.max_len:
                raise ValueError(f"row {b}: {int(self.lens[b])} tokens > max_len {self.max_len}")
        self.lens -= np.asarray(n_new, np.int64)
        return real(self, k_new, v_new, n_new)

    monkeypatch.setattr(direct.Cache, "append", early)
    with pytest.raises(AssertionError):
        test_overflow_on_last_row_raises_and_changes_nothing()
