"""Pins of the FP8 (E4M3, one scale per head) cache oracle (oracle/fp8.py).

[CH16] "16. Prefill, decode and the KV cache", exercise 4. The decoder is
pinned to values fixed by the format's fields (OCP E4M3: bias 7, largest
finite 448, subnormals m * 2^-9), the encoder to round trips, ties and
saturation, and the attention to the pinned linear-cache oracle applied to the
dequantized values.
"""

import numpy as np
import pytest

from oracle import direct, fp8


def test_decode_anchor_values():
    assert fp8.DECODE[0x00] == 0.0
    assert fp8.DECODE[0x01] == 2.0 ** -9            # smallest subnormal
    assert fp8.DECODE[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert fp8.DECODE[0x08] == 2.0 ** -6            # smallest normal
    assert fp8.DECODE[0x38] == 1.0                  # exponent 7 = bias, mantissa 0
    assert fp8.DECODE[0x39] == 1.125
    assert fp8.DECODE[0x40] == 2.0
    assert fp8.DECODE[0x7E] == 448.0                # largest finite
    assert np.isnan(fp8.DECODE[0x7F]) and np.isnan(fp8.DECODE[0xFF])
    assert fp8.DECODE[0xB8] == -1.0 and fp8.DECODE[0xFE] == -448.0
    finite = fp8.DECODE[:0x7F]
    assert (np.diff(finite) > 0).all()              # positive codes increase strictly
    assert np.array_equal(fp8.DECODE[0x80:0xFF], -finite)


def test_round_trip_of_every_finite_code():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        if c == 0x80:
            assert fp8.encode_one(np.float32(-0.0)) == 0x80
            continue
        assert fp8.encode_one(np.float32(fp8.DECODE[c])) == c, hex(c)


def test_ties_go_to_the_even_code_and_the_rest_to_the_nearest():
    for c in range(0x7E):
        lo, hi = fp8.DECODE[c], fp8.DECODE[c + 1]
        mid = np.float32((lo + hi) / 2)             # exact in float32 for these grids
        assert fp8.encode_one(mid) == (c if c % 2 == 0 else c + 1), hex(c)
        assert fp8.encode_one(np.float32(lo + (hi - lo) * 0.25)) == c
        assert fp8.encode_one(np.float32(lo + (hi - lo) * 0.75)) == c + 1


def test_saturation_and_tiny_values():
    assert fp8.encode_one(np.float32(1000.0)) == 0x7E
    assert fp8.encode_one(np.float32(-1e30)) == 0xFE
    assert fp8.encode_one(np.float32(460.0)) == 0x7E
    assert fp8.encode_one(np.float32(2.0 ** -11)) == 0x00     # below half the smallest subnormal
    assert fp8.encode_one(np.float32(-2.0 ** -11)) == 0x80
    assert fp8.encode_one(np.float32(0.75 * 2.0 ** -9)) == 0x01


def test_quantize_uses_the_float32_product():
    """x * (1/scale) is formed in float32 before rounding (the integer decision)."""
    x = np.float32(3.3)
    s = np.float32(0.37)
    inv = np.float32(1.0) / s
    assert fp8.quantize(np.array([x]), inv)[0] == fp8.encode_one(np.float32(x * inv))


def test_array_quantizer_equals_the_scalar_encoder():
    """quantize (whole arrays) takes the same decision as encode_one on the tie
    grid, random values across magnitudes, saturating values and signed zeros."""
    rng = np.random.default_rng(5)
    grid = []
    for c in range(0x7E):
        lo, hi = fp8.DECODE[c], fp8.DECODE[c + 1]
        grid += [lo, (lo + hi) / 2, lo + (hi - lo) * 0.3, lo + (hi - lo) * 0.7]
    x = np.concatenate([grid, rng.standard_normal(5000) * rng.choice([1e-3, 0.1, 3, 80, 900], 5000),
                        [0.0, 448, 460, 1e9, 2.0 ** -12]]).astype(np.float32)
    x = np.concatenate([x, -x])
    want = np.array([fp8.encode_one(v) for v in x], np.uint8)
    assert np.array_equal(fp8.quantize(x, np.float32(1.0)), want)


def test_quantization_error_is_within_half_a_step():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * 3
    codes = fp8.quantize(x, np.float32(1.0))
    err = np.abs(fp8.decode(codes) - x.astype(np.float64))
    # half the spacing at |x|: 2^(floor(log2|x|) - 4), and 2^-10 in the subnormal range
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
    assert (err <= 2.0 ** (e - 4) + 1e-12).all()


def _bf16(x):
    import workloads as W
    return W.to_bf16_bits(x)


def test_attention_is_the_plain_oracle_on_dequantized_values():
    """The FP8 cache's attention equals the linear-cache oracle fed the
    dequantized values, to 0.0 (power-of-two scales keep every code x scale
    exact in float32)."""
    rng = np.random.default_rng(1)
    B, hk, G, d, S = 2, 2, 3, 16, 40
    ks, vs = np.array([2.0 ** -6, 0.5], np.float32), np.array([0.125, 4.0], np.float32)
    c = fp8.Fp8Cache(B, hk, S, d, ks, vs)
    lin = direct.Cache(B, hk, S, d, "f32")
    for n in ([7, 3], [1, 1], [9, 0], [2, 5]):
        T = max(n)
        k = _bf16(rng.standard_normal((B, hk, T, d)).astype(np.float32) * ks[None, :, None, None] * 40)
        v = _bf16(rng.standard_normal((B, hk, T, d)).astype(np.float32) * vs[None, :, None, None] * 40)
        q = _bf16(rng.standard_normal((B, hk * G, T, d)).astype(np.float32))
        s0 = c.lens.copy()
        c.append(k, v, n)
        kd = np.zeros((B, hk, T, d), np.float32)
        vd = np.zeros_like(kd)
        for b in range(B):
            k64, v64 = c.dequantized(b)
            kd[b, :, :n[b]] = k64[:, s0[b]:s0[b] + n[b]]
            vd[b, :, :n[b]] = v64[:, s0[b]:s0[b] + n[b]]
        lin.append(kd, vd, n)
        assert np.array_equal(fp8.attention(c, q, n), _direct_bf16q(lin, q, n))


def _direct_bf16q(lin, q_bits, n):
    """direct.attention with bf16 queries widened to float32 (exact)."""
    import workloads as W
    return direct.attention(lin, W.bf16_bits_to_f32(q_bits), n)


def test_one_scale_per_head():
    """Head-labelled V (every element of KV head h is the code for 1.0) with
    v_scale[h] = h + 1: query head g reads KV head g // G, so its output is g // G + 1."""
    B, hk, G, d, S = 1, 3, 2, 8, 16
    c = fp8.Fp8Cache(B, hk, S, d, np.ones(hk, np.float32), np.arange(1, hk + 1, dtype=np.float32))
    rng = np.random.default_rng(2)
    k = _bf16(rng.standard_normal((B, hk, 5, d)).astype(np.float32))
    v = _bf16(np.broadcast_to(np.arange(1, hk + 1, dtype=np.float32)[None, :, None, None], (B, hk, 5, d)).copy())
    c.append(k, v, [5])
    assert (c.v[:, :, :5] == 0x38).all()          # each value / its scale is exactly 1.0
    q = _bf16(rng.standard_normal((B, hk * G, 5, d)).astype(np.float32))
    out = fp8.attention(c, q, [5])
    for h in range(hk * G):
        assert np.allclose(out[0, h, :5], h // G + 1, rtol=0, atol=1e-12)


def test_planted_missing_scale_fails():
    """Planted mistake: dequantizing without the head's scale changes the result."""
    rng = np.random.default_rng(3)
    c = fp8.Fp8Cache(1, 1, 8, 8, [0.05], [0.05])
    x = _bf16(rng.standard_normal((1, 1, 4, 8)).astype(np.float32))
    c.append(x, x, [4])
    q = _bf16(rng.standard_normal((1, 2, 4, 8)).astype(np.float32))
    good = fp8.attention(c, q, [4])
    k64, v64 = c.dequantized(0)
    bad = fp8.attention_row(k64 / 0.05, v64 / 0.05, 4, 4, q[0], "bf16", [(h, t) for h in range(2) for t in range(4)])
    assert np.abs(good[0] - bad).max() > 1e-2
