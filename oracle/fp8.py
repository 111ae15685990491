"""FP8 (E4M3) KV cache with one scale per head: the CPU reference.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/ and
``__graft_entry__.smoke()``.

Source: [CH16] "16. Prefill, decode and the KV cache" (inference.shantanugoel.com),
exercise 4 (store the cache in FP8, E4M3 with one scale per head, and
dequantize on read) and "How big is the cache?" / the bandwidth bullet
(decode reads the whole cache each step, which is what quantization buys).

Readings taken where the page is silent (each listed in the design notes):
  * E4M3 is the OCP 8-bit format: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent 0 holds subnormals m * 2^-9; the largest finite value is
    448 (0x7E); 0x7F/0xFF are NaN; there are no infinities.
  * "One scale per head": one float32 scale per KV head for K and one for V,
    fixed by the caller when the cache is made. A stored code c of head h
    stands for c * scale[h].
  * Quantization on append: y = float32(x) * float32(1 / scale) in float32,
    saturated to [-448, 448], rounded to the nearest E4M3 value, ties to the
    even code (the encoding is the integer decision, taken in float32 on
    both sides).

Arithmetic after decoding is float64; every E4M3 value is exact in float64.
"""

from __future__ import annotations

import numpy as np

from .direct import attend_one, kv_head_of, query_position, to_float64

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of one E4M3 code (int 0..255) from its fields, per the OCP format."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9              # subnormal: (m / 8) * 2^(1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# decode table: code -> float64 value
DECODE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes):
    """float64 values of an array of E4M3 codes (uint8)."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode_one(y):
    """E4M3 code of one float32 value: saturate to +-448, round to nearest,
    ties to the even code. Works from the value grid: the candidates are the
    two finite codes of the same sign around |y|."""
    y = float(np.float32(y))
    if y != y:
        return 0x7F
    sign = 0x80 if (y < 0 or (y == 0 and np.signbit(y))) else 0
    a = min(abs(y), E4M3_MAX)
    mags = DECODE[:0x7F]                      # codes 0x00 .. 0x7E, increasing values
    hi = int(np.searchsorted(mags, a, side="left"))
    if hi < len(mags) and mags[hi] == a:
        return sign | hi
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    if d_lo < d_hi:
        c = lo
    elif d_hi < d_lo:
        c = hi
    else:
        c = lo if lo % 2 == 0 else hi         # tie: the code whose mantissa is even
    return sign | c


def quantize(x_f32, inv_scale_f32):
    """Codes of float32 values x times the float32 reciprocal scale (the product
    in float32). The same rule as ``encode_one``, applied to whole arrays: the
    two finite codes around |y| (after saturation), the nearer one, on a tie
    the even one; the sign bit from y."""
    y = (np.asarray(x_f32, dtype=np.float32) * np.float32(inv_scale_f32)).astype(np.float32)
    mags = DECODE[:0x7F]
    a = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX)
    hi = np.minimum(np.searchsorted(mags, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    c = np.where(mags[hi] == a, hi,
                 np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi))))
    code = (c | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), code)


class Fp8Cache:
    """K and V codes [B, Hkv, max_len, d] (uint8) with per-KV-head scales.

    Appends take bfloat16 (uint16 bit patterns) or float32 inputs and store
    their E4M3 codes; everything else follows the linear cache of
    ``direct.Cache`` (validate every row, then write; lengths after the write).
    """

    def __init__(self, batch, kv_heads, max_len, head_dim, k_scale, v_scale, in_dtype="bf16"):
        self.k = np.zeros((batch, kv_heads, max_len, head_dim), np.uint8)
        self.v = np.zeros_like(self.k)
        self.lens = np.zeros(batch, np.int64)
        self.k_scale = np.asarray(k_scale, np.float32).reshape(kv_heads)
        self.v_scale = np.asarray(v_scale, np.float32).reshape(kv_heads)
        if not (np.isfinite(self.k_scale).all() and np.isfinite(self.v_scale).all()
                and (self.k_scale > 0).all() and (self.v_scale > 0).all()):
            raise ValueError("scales must be finite and positive")
        self.in_dtype = in_dtype

    @property
    def batch(self):
        return self.k.shape[0]

    @property
    def kv_heads(self):
        return self.k.shape[1]

    @property
    def max_len(self):
        return self.k.shape[2]

    def append(self, k_new, v_new, n_new):
        B, hk, S, d = self.k.shape
        T = k_new.shape[2]
        n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
        for b in range(B):
            n = int(n_new[b])
            if n < 0 or n > T:
                raise ValueError(f"row {b}: n_new {n} outside 0..{T}")
            if self.lens[b] + n > S:
                raise ValueError(f"row {b}: {int(self.lens[b]) + n} tokens > max_len {S}")
        kf = to_float64(k_new, self.in_dtype).astype(np.float32)
        vf = to_float64(v_new, self.in_dtype).astype(np.float32)
        for b in range(B):
            s, n = int(self.lens[b]), int(n_new[b])
            for h in range(hk):
                inv_k = np.float32(1.0) / self.k_scale[h]
                inv_v = np.float32(1.0) / self.v_scale[h]
                self.k[b, h, s:s + n] = quantize(kf[b, h, :n], inv_k)
                self.v[b, h, s:s + n] = quantize(vf[b, h, :n], inv_v)
        self.lens += n_new

    def truncate(self, new_lens):
        new = np.broadcast_to(np.asarray(new_lens, dtype=np.int64), self.lens.shape)
        if np.any(new < 0) or np.any(new > self.lens):
            raise ValueError("Invalid truncation length")
        self.lens = new.copy()

    def dequantized(self, b):
        """float64 K and V of row b: code value times the head's scale (dequantize on read)."""
        k = decode(self.k[b]) * self.k_scale.astype(np.float64)[:, None, None]
        v = decode(self.v[b]) * self.v_scale.astype(np.float64)[:, None, None]
        return k, v


def attention_row(k64, v64, length, n_new_b, q_row, q_dtype, pairs):
    """The plain definition on dequantized float64 K/V [Hkv, >= length, d] of one
    row, for the listed (head, t) pairs ([GQA] "A strong answer": head h reads
    KV head h // G; query t at length - n_new + t sees keys 0 .. that position)."""
    hk, _, d = k64.shape
    hq, T, _ = q_row.shape
    G = hq // hk
    out = np.zeros((hq, T, d), np.float64)
    for h, t in pairs:
        if t >= n_new_b:
            continue
        p = query_position(length, n_new_b, t)
        kvh = kv_head_of(h, G)
        out[h, t] = attend_one(k64[kvh, :p + 1], v64[kvh, :p + 1], to_float64(q_row[h, t], q_dtype), d)
    return out


def attention(cache: Fp8Cache, q, n_new):
    """GQA output [B, Hq, T, d] (float64) over the dequantized cache."""
    q = np.asarray(q)
    B, hq, T, d = q.shape
    n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
    out = np.zeros((B, hq, T, d), np.float64)
    for b in range(B):
        L, n = int(cache.lens[b]), int(n_new[b])
        if n < 0 or n > T or n > L:
            raise ValueError(f"row {b}: bad n_new {n}")
        if n == 0:
            continue
        k64, v64 = cache.dequantized(b)
        out[b] = attention_row(k64, v64, L, n, q[b], cache.in_dtype,
                               [(h, t) for h in range(hq) for t in range(n)])
    return out
