"""Shapes, seeded draws and call schedules for the GQA / KV-cache workloads.

Every value here is drawn from ``numpy.random.default_rng`` with an explicit
seed, as standard-normal float32, optionally scaled, then rounded once to the
storage type (bfloat16 by round-to-nearest-even, kept as uint16 bit patterns,
or float32 as is). Both the HIP path and the CPU oracle receive the same bits.

The workload shapes stand in for what the pages discuss:
  * the random trials and the S=37 / T=5 chunk of the two interview pages
    (tiny float32 cache, ``TINY_FP32``);
  * 4,096-token Llama-3.1-8B generation with 8,192-token reservations
    ("Implement grouped-query attention over a preallocated KV cache",
    section "A strong answer") -> ``LLAMA8B_DECODE``;
  * speculative verify, T=4 over S=4,096 ("Write the causal mask for a decode
    step with a KV cache", section "A strong answer") -> ``LLAMA8B_VERIFY``;
  * a chunk in the middle of a 10K prompt (same page, "What interviewers probe
    next") -> ``LLAMA8B_CHUNKED_PREFILL``;
  * batch 64 with very different row lengths (first page, the reversal
    paragraph and "What interviewers probe next") -> ``LLAMA8B_RAGGED``.
No weights and no dataset are involved: attention inputs are synthetic.
"""

from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np


# --------------------------------------------------------------------------
# storage types
# --------------------------------------------------------------------------

def storage_np_dtype(dtype: str):
    """numpy dtype that holds one stored element: float32, or bf16 bits."""
    if dtype == "f32":
        return np.float32
    if dtype == "bf16":
        return np.uint16
    raise ValueError(f"unknown storage dtype {dtype!r}")


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Standard-normal draw in float32, times ``scale``, stored as ``dtype``."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "f32":
        return x
    return to_bf16_bits(x)


def _nan_like(dtype: str):
    return np.float32("nan") if dtype == "f32" else np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    name: str
    dtype: str           # storage / compute dtype of q, k, v, out: "f32" or "bf16"
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    max_len: int
    value_scale: float = 1.0     # multiplier applied to every N(0,1) draw
    notes: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


TINY_FP32 = Shape("tiny_fp32", "f32", 2, 4, 2, 16, 64,
                  notes={"final_lens": (37, 20), "chunk": (1, 8)})
LLAMA8B_DECODE = Shape("llama8b_decode_b32_s4096", "bf16", 32, 32, 8, 128, 8192,
                       value_scale=1.0 / math.sqrt(128.0),
                       notes={"cached": 4096, "T": 1})
# Sliding window over a ring: max_len is the ring capacity (slots per row);
# 20,000 tokens precede the step, so the ring has wrapped twice and a decode
# query at position 20,000 reads keys 16,905 .. 20,000 through wrapped slots.
LLAMA8B_WINDOW_DECODE = Shape("llama8b_window_decode_b32_w4096_c8192", "bf16", 32, 32, 8, 128, 8192,
                              value_scale=1.0 / math.sqrt(128.0),
                              notes={"window": 4096, "cached": 20000, "T": 1})
LLAMA8B_VERIFY = Shape("llama8b_verify_b16_t4_s4096", "bf16", 16, 32, 8, 128, 8192,
                       notes={"cached": 4092, "T": 4})
LLAMA8B_CHUNKED_PREFILL = Shape("llama8b_chunked_prefill_b4_10240x512", "bf16", 4, 32, 8, 128, 16384,
                                notes={"prompt": 10240, "chunk": 512})
LLAMA8B_RAGGED = Shape("llama8b_ragged_b64", "bf16", 64, 32, 8, 128, 32768,
                       notes={"len_range": (1, 32000), "n_new_choices": (0, 1, 4, 256), "T": 256})



def llama8b_decode_shard(tp: int) -> Shape:
    """One GPU's share of the decode workload when tp GPUs split the heads:
    8/tp KV heads with their 32/tp query heads (group 4 kept), all 32 rows."""
    if tp not in (1, 2, 4, 8):
        raise ValueError(tp)
    return Shape(f"llama8b_decode_b32_s4096_tp{tp}", "bf16", 32, 32 // tp, 8 // tp, 128, 8192,
                 value_scale=1.0 / math.sqrt(128.0), notes={"cached": 4096, "T": 1, "tp": tp})


WORKLOADS = {s.name: s for s in (TINY_FP32, LLAMA8B_DECODE, LLAMA8B_VERIFY,
                                 LLAMA8B_CHUNKED_PREFILL, LLAMA8B_RAGGED)}


# --------------------------------------------------------------------------
# seeded tensors
# --------------------------------------------------------------------------

_TAG_PREFIX = 1
_TAG_STEP = 2


def prefix_kv(shape: Shape, seed: int, row: int, start: int, n_tokens: int):
    """K and V for tokens [start, start+n_tokens) of one row: [Hkv, n, d] each.

    Token i of row r is drawn from its own stream (seed, row, i), so any slice
    of a row's history can be regenerated on its own, and the GPU setup (which
    appends in chunks) and a sampled oracle check (which reads one row) see the
    same bits.
    """
    hk, d = shape.kv_heads, shape.head_dim
    k = np.empty((hk, n_tokens, d), storage_np_dtype(shape.dtype))
    v = np.empty_like(k)
    # one generator per 256-token block keeps this fast and still slice-stable
    blk = 256
    i = 0
    while i < n_tokens:
        tok = start + i
        b0 = (tok // blk) * blk
        rng = np.random.default_rng([seed, _TAG_PREFIX, row, b0])
        kk = draw(rng, (blk, hk, d), shape.dtype, shape.value_scale)
        vv = draw(rng, (blk, hk, d), shape.dtype, shape.value_scale)
        lo = tok - b0
        take = min(blk - lo, n_tokens - i)
        k[:, i:i + take] = kk[lo:lo + take].transpose(1, 0, 2)
        v[:, i:i + take] = vv[lo:lo + take].transpose(1, 0, 2)
        i += take
    return k, v


def step_inputs(shape: Shape, seed: int, step: int, T: int, n_new, pad: str = "nan"):
    """q [B,Hq,T,d], k_new and v_new [B,Hkv,T,d] for one call.

    Slots t >= n_new[b] are padding the method must never read; ``pad='nan'``
    fills them with NaN so that a leak shows, ``pad='normal'`` leaves the draw.
    """
    B, hq, hk, d = shape.batch, shape.q_heads, shape.kv_heads, shape.head_dim
    rng = np.random.default_rng([seed, _TAG_STEP, step])
    q = draw(rng, (B, hq, T, d), shape.dtype, shape.value_scale)
    k = draw(rng, (B, hk, T, d), shape.dtype, shape.value_scale)
    v = draw(rng, (B, hk, T, d), shape.dtype, shape.value_scale)
    if pad == "nan":
        n_new = np.asarray(n_new)
        for b in range(B):
            n = int(n_new[b])
            q[b, :, n:] = _nan_like(shape.dtype)
            k[b, :, n:] = _nan_like(shape.dtype)
            v[b, :, n:] = _nan_like(shape.dtype)
    elif pad != "normal":
        raise ValueError(pad)
    return q, k, v


# --------------------------------------------------------------------------
# call schedules
# --------------------------------------------------------------------------

def _chunk_schedule(rng, targets, t_max, start=None, max_calls=10_000):
    lens = list(start) if start is not None else [0] * len(targets)
    calls = []
    while any(l < t for l, t in zip(lens, targets)):
        T = int(rng.integers(1, t_max + 1))
        n = []
        for b, tgt in enumerate(targets):
            want = int(rng.integers(0, T + 1))
            n.append(min(want, tgt - lens[b]))
        calls.append({"T": T, "n_new": n})
        lens = [l + x for l, x in zip(lens, n)]
        if len(calls) > max_calls:
            raise RuntimeError("schedule did not converge")
    return calls


def tiny_schedule(seed: int = 0):
    """Call schedule for the tiny float32 cache (B=2, final lengths 37 and 20).

    The first call hits the empty cache with zero new tokens. Rows then grow in
    seeded chunks of 1..8 tokens, with some calls giving a row no tokens. The
    last call appends exactly 5 tokens to row 0 (32 -> 37) and none to row 1,
    so it reproduces the S=37, T=5 chunk used on the causal-mask page.
    """
    rng = np.random.default_rng([seed, 0xC0])
    calls = [{"T": 3, "n_new": [0, 0]}]
    calls += _chunk_schedule(rng, [32, 20], 8)
    calls.append({"T": 5, "n_new": [5, 0]})
    return calls


def schedule_to_lengths(calls, batch):
    lens = [0] * batch
    out = []
    for c in calls:
        lens = [l + n for l, n in zip(lens, c["n_new"])]
        out.append(list(lens))
    return out


def trial_spec(seed: int, head_dims=(16,)):
    """One random trial in the ranges of the first page's correctness report.

    1, 2 or 4 KV heads; group size 1..8; 1..3 rows; final row lengths 0..40;
    chunks of 1..8 tokens (so decode, chunked prefill with T < S and rows that
    get zero tokens in a call all occur).
    """
    rng = np.random.default_rng([seed, 0x7A1])
    hk = int(rng.choice([1, 2, 4]))
    g = int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    d = int(rng.choice(list(head_dims)))
    targets = [int(rng.integers(0, 41)) for _ in range(B)]
    calls = _chunk_schedule(rng, targets, 8)
    if not calls:
        calls = [{"T": int(rng.integers(1, 9)), "n_new": [0] * B}]
    shape = Shape(f"trial{seed}", "f32", B, hk * g, hk, d, 48)
    return shape, calls


def ragged_rows(seed: int = 4, batch: int = 64, lo: int = 1, hi: int = 32000,
                choices=(0, 1, 4, 256)):
    """Per-row cached lengths log-uniform in [lo, hi] and per-row n_new."""
    rng = np.random.default_rng([seed, 0x4A6])
    u = rng.uniform(math.log(lo), math.log(hi), size=batch)
    lens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)
    n_new = rng.choice(np.asarray(choices, dtype=np.int64), size=batch)
    return lens, n_new


def ring_schedule(seed, batch, capacity, window, steps, t_cap):
    """Seeded calls for a sliding-window ring: decode steps (T=1), short chunks
    (T=4) and chunks of t_cap, some rows idle, every row's n_new kept within
    what the ring accepts (any n while the row fits in the ring, at most
    capacity - window + 1 once it would wrap). Returns (calls, final lengths)."""
    rng = np.random.default_rng(seed)
    lens = np.zeros(batch, np.int64)
    calls = []
    for _ in range(steps):
        T = int(rng.choice([1, 1, 4, t_cap]))
        n = []
        for b in range(batch):
            lim = T if lens[b] + T <= capacity else min(T, capacity - window + 1)
            n.append(int(rng.integers(0, lim + 1)) if rng.random() < 0.8 else 0)
        calls.append({"T": T, "n_new": n})
        lens += np.asarray(n)
    return calls, lens
