#!/usr/bin/env python3
"""Benchmark: GQA decode over a preallocated KV cache on one MI355X.

One step = one pass of the whole hot path over one batch: in-place append of
each row's new token, grouped-query attention, and the rollback of the cache
length (so every step sees the same lengths). Workload: Llama-3.1-8B-shaped
decode, one layer, Hq=32, Hkv=8, d=128, bfloat16, B=32 rows of 4,096 cached
tokens in 8,192-token reservations, T=1 (attention over 4,097 keys). Inputs are
seeded synthetic N(0,1)/sqrt(d) values; no weights.

Prints one JSON line. `value` is decode-attention HBM throughput over whole
steps: algorithmic bytes per step (live K+V, q, out, and the append's read and
write) divided by the wall time per step. `roofline` reports the attention
call alone against MI355X's 8 TB/s, timed with HIP events on the stream the
kernels run on. `prefill` gives chunked-prefill TFLOP/s (B=4, 10,240-token
prompts fed as 512-token chunks) against the 2.5 PFLOP/s dense bf16 peak.
`cpu_baseline` times the float64 CPU oracle on the host.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama8b_b32_s4096_traffic.json")


def csrc_hash():
    """First 16 hex digits of the sha256 over the HIP library sources, in name order."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gqa_attention_preallocated_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy of known size), or None when the kernel
    sources changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return int(rec["traffic_bytes"]) if rec.get("csrc_sha256_16") == csrc_hash() else None


def dev_bf16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def attention_bytes(lens_after, n_new, hq, hkv, d, T, elem=2):
    """Algorithmic bytes of one attention call: live K+V, real q, every out slot."""
    kv = sum(int(s) for s in lens_after) * hkv * d * 2 * elem
    q = sum(int(n) for n in n_new) * hq * d * elem
    out = len(lens_after) * hq * T * d * elem
    return kv + q + out


def attention_flops(lens_after, n_new, hq, d):
    """4*d FLOP per visible (query, key) pair per query head."""
    pairs = 0
    for s, n in zip(lens_after, n_new):
        base = int(s) - int(n)
        pairs += sum(base + t + 1 for t in range(int(n)))
    return 4 * d * hq * pairs


def fill_decode_cache(torch, cache, shape, seed, tokens, chunk=2048):
    import workloads as W
    B = shape.batch
    hist = []
    for start in range(0, tokens, chunk):
        n = min(chunk, tokens - start)
        ks = np.empty((B, shape.kv_heads, n, shape.head_dim), np.uint16)
        vs = np.empty_like(ks)
        for b in range(B):
            ks[b], vs[b] = W.prefix_kv(shape, seed, b, start, n)
        hist.append((ks, vs))
        cache.append(dev_bf16(torch, ks), dev_bf16(torch, vs), [n] * B)
    return hist


def run_decode(torch, steps, warmup):
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_DECODE
    seed, cached = DECODE_SEED, DECODE_CACHED
    B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
    # two caches used in turn: each step streams 537 MB that the previous step
    # did not touch, so the 256 MB last-level cache cannot serve it
    caches = [KVCache(B, hkv, sh.max_len, d, device_lens=False) for _ in range(2)]
    hist = None
    for c in caches:
        hist = fill_decode_cache(torch, c, sh, seed, cached)
    n = [1] * B
    q, k, v = W.step_inputs(sh, seed, 10_000, 1, n, pad="normal")
    qd, kd, vd = dev_bf16(torch, q), dev_bf16(torch, k), dev_bf16(torch, v)
    out = torch.empty_like(qd)
    # workspace sized after the append (lengths 4,097)
    for c in caches:
        c.append(kd, vd, n)
    ws_bytes = max(c.workspace_bytes(hq, 1, n) for c in caches)
    for c in caches:
        c.truncate([cached] * B)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    # one decode step = append each row's new token, attend, roll back (so every
    # step sees 4,096 cached keys): kv_append_attention does the append and the
    # attention in the decode kernel's one launch (truncate launches nothing here)
    def step(i):
        c = caches[i & 1]
        append_attention(c, kd, vd, qd, n, out=out, workspace=ws)
        c.truncate([cached] * B)

    # the same step as two calls (kv_append, then gqa_attention), for comparison
    def step_two_calls(i):
        c = caches[i & 1]
        c.append(kd, vd, n)
        gqa_attention(qd, c, n, out=out, workspace=ws)
        c.truncate([cached] * B)

    walls = {}
    for name, fn in (("one_call", step), ("two_calls", step_two_calls)):
        # a short device spin first brings the clock up from idle (as the
        # other workloads' timing does); then the untimed warm-up steps
        torch.cuda._sleep(20_000_000)
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        walls[name] = (time.perf_counter() - t0) / steps

    # the step's kernel alone: back-to-back launches (alternating caches)
    # between two HIP events on the stream the library launches on (torch's
    # current stream, which the binding passes to every call). Like the wall
    # loop it starts behind a device spin and untimed warm-up steps, and it
    # times at least ROOFLINE_REPS launches whatever --steps is, so the host
    # has enqueued the launches before the GPU reaches them and the average
    # holds no first-launch or enqueue gap.
    reps = max(steps, ROOFLINE_REPS)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    for i in range(max(warmup, ROOFLINE_WARMUP)):
        step(i)
    e0.record()
    for i in range(reps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    att_avg = e0.elapsed_time(e1) / reps
    # per-call spread: each call between its own events (these include the
    # dispatch latency of an isolated launch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    att_ms = sorted(a.elapsed_time(b) for a, b in evs)

    lens_after = [cached + 1] * B
    # the launch reads every live key (the new one from k_new), q, and writes
    # out and the new K and V rows into the cache
    att_b = attention_bytes(lens_after, n, hq, hkv, d, 1)
    app_b = 2 * sum(n) * hkv * d * 2
    return {
        "shape": sh, "seed": seed, "q": q, "k": k, "v": v,
        "wall_s": walls["one_call"], "wall_two_calls_s": walls["two_calls"],
        "att_ms_avg": att_avg, "att_ms_p50": att_ms[len(att_ms) // 2],
        "att_ms_p10": att_ms[len(att_ms) // 10], "att_ms_p90": att_ms[(9 * len(att_ms)) // 10],
        "att_bytes": att_b, "append_bytes": app_b, "lens_after": lens_after,
    }


def run_prefill(torch, reps=3):
    """Chunked prefill: reset, then 20 x (append a 512-token chunk, attention T=512)."""
    from gqa_attention_preallocated_amd import KVCache, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_CHUNKED_PREFILL
    B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
    cache = KVCache(B, hkv, sh.max_len, d, device_lens=False)
    n = [512] * B
    chunks = []
    for c in range(20):
        q, k, v = W.step_inputs(sh, PREFILL_SEED, c, 512, n, pad="normal")
        chunks.append((dev_bf16(torch, q), dev_bf16(torch, k), dev_bf16(torch, v)))
    out = torch.empty_like(chunks[0][0])
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    flops = [attention_flops([512 * (c + 1)] * B, n, hq, d) for c in range(20)]
    times = np.zeros(20)
    for rep in range(reps + 1):
        cache.reset()
        evs = []
        # a short GPU spin first: the host enqueues all 20 chunks while it
        # runs, so each event pair brackets GPU work only, not host latency
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)
        for c, (qd, kd, vd) in enumerate(chunks):
            cache.append(kd, vd, n)
            need = cache.workspace_bytes(hq, 512, n)
            if need > ws.numel():
                ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gqa_attention(qd, cache, n, out=out, workspace=ws)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        if rep > 0:
            times += np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3
    times /= reps
    total_flops = float(sum(flops))
    total_s = float(times.sum())
    tflops = total_flops / total_s / 1e12
    return {
        "metric": "chunked prefill attention TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "peak": BF16_PEAK_TFLOPS, "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "ms_per_prompt": round(total_s * 1e3, 4),
        "flop_per_prompt": total_flops,
        "last_chunk_tflops": round(flops[-1] / times[-1] / 1e12, 2),
        "config": {"workload": sh.name, "batch": B, "prompt": 10240, "chunk": 512},
    }


def _fill_gpu_random(torch, cache, lens, seed, chunk=4096):
    """Seeded N(0,1) K/V history drawn on the GPU (fast set-up for timing runs)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    lens = [int(x) for x in lens]
    done = [0] * len(lens)
    B, hkv, d = cache.batch, cache.kv_heads, cache.head_dim
    while any(x < l for x, l in zip(done, lens)):
        n = [min(chunk, l - x) for x, l in zip(done, lens)]
        T = max(n)
        k = torch.randn(B, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        cache.append(k, v, n)
        done = [x + y for x, y in zip(done, n)]


def _time_calls(torch, fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)     # the host enqueues every call before the GPU reaches them
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e-3


def run_verify(torch, reps=30):
    """Speculative verify: B=16, 4,092 cached + 4 new tokens per row, T=4. The
    step: kv_append_attention of the 4 draft tokens, then a host-only rollback
    to 4,092 (two caches in turn); also the attention call alone."""
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_VERIFY
    B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
    cached = sh.notes["cached"]
    caches = [KVCache(B, hkv, sh.max_len, d, device_lens=False) for _ in range(2)]
    n = [4] * B
    for i, c in enumerate(caches):
        _fill_gpu_random(torch, c, [cached] * B, 20 + i)
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn(B, hq, 4, d, device="cuda", generator=g).to(torch.bfloat16)
    kn = torch.randn(B, hkv, 4, d, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty_like(q)
    caches[0].append(kn, kn, n)
    ws = torch.zeros(max(caches[0].workspace_bytes(hq, 4, n), 256), dtype=torch.uint8, device="cuda")
    caches[0].truncate([cached] * B)

    def step(i):
        c = caches[i & 1]
        append_attention(c, kn, kn, q, n, out=out, workspace=ws)
        c.truncate([cached] * B)

    t_step = _time_calls(torch, step, reps)
    for c in caches:
        c.append(kn, kn, n)
    t_att = _time_calls(torch, lambda i: gqa_attention(q, caches[i & 1], n, out=out, workspace=ws), reps)
    nbytes = attention_bytes([cached + 4] * B, n, hq, hkv, d, 4)
    step_bytes = nbytes + 2 * sum(n) * hkv * d * 2      # and the new K and V rows written
    return {"metric": "verify step HBM GB/s", "value": round(step_bytes / t_step / 1e9, 2), "unit": "GB/s",
            "frac_of_8TBs": round(step_bytes / t_step / 8e12, 4), "ms": round(t_step * 1e3, 5), "bytes": step_bytes,
            "attention_only": {"ms": round(t_att * 1e3, 5), "bytes": nbytes, "GB/s": round(nbytes / t_att / 1e9, 2)},
            "config": {"workload": sh.name, "batch": B, "T": 4, "cached": cached, "keys": cached + 4}}


def run_shard(torch, reps=40):
    """One GPU's share of the decode step when tp GPUs split the heads (tp = 1,
    2, 4, 8: Hkv = 8/tp and Hq = 32/tp, all 32 rows, 4,096 cached keys + 1):
    kv_append_attention then a host-only rollback, over 2*tp caches in turn so
    that each step reads 1/(2 tp) of 1.07 GB of K/V that the step before did
    not touch."""
    from gqa_attention_preallocated_amd import KVCache, append_attention
    import workloads as W
    shards = []
    for tp in (1, 2, 4, 8):
        sh = W.llama8b_decode_shard(tp)
        B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
        nc = 2 * tp
        caches = [KVCache(B, hkv, sh.max_len, d, device_lens=False) for _ in range(nc)]
        for i, c in enumerate(caches):
            _fill_gpu_random(torch, c, [4096] * B, 40 + i)
        n = [1] * B
        g = torch.Generator(device="cuda").manual_seed(13)
        q = (torch.randn(B, hq, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
        kn = (torch.randn(B, hkv, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
        vn = (torch.randn(B, hkv, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
        out = torch.empty_like(q)
        caches[0].append(kn, vn, n)
        ws_bytes = caches[0].workspace_bytes(hq, 1, n)
        caches[0].truncate([4096] * B)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

        def step(i):
            c = caches[i % nc]
            append_attention(c, kn, vn, q, n, out=out, workspace=ws)
            c.truncate([4096] * B)

        t = _time_calls(torch, step, reps)
        nbytes = attention_bytes([4097] * B, n, hq, hkv, d, 1) + 2 * B * hkv * d * 2
        shards.append({"tp": tp, "kv_heads": hkv, "q_heads": hq, "items": B * hkv, "ms": round(t * 1e3, 5),
                       "bytes": nbytes, "GB/s": round(nbytes / t / 1e9, 2), "frac_of_8TBs": round(nbytes / t / 8e12, 4)})
        del caches, ws
        torch.cuda.empty_cache()
    return {"metric": "decode step per GPU under head sharding, HBM GB/s", "value": shards[-1]["GB/s"], "unit": "GB/s",
            "shards": shards,
            "config": {"workload": "llama8b_decode_b32_s4096_tp{1,2,4,8}", "batch": 32, "keys": 4097, "T": 1}}


def run_stride(torch, reps=60):
    """The Llama decode step (B=32, 4,096 cached + 1 new token, one
    kv_append_attention call, two caches in turn) on linear caches of several
    max_len: the rows of a (row, KV head) sit max_len x 256 bytes apart."""
    from gqa_attention_preallocated_amd import KVCache, append_attention
    import workloads as W
    sh = W.LLAMA8B_DECODE
    B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
    n = [1] * B
    g = torch.Generator(device="cuda").manual_seed(3)
    q = (torch.randn(B, hq, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
    kn = (torch.randn(B, hkv, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
    out = torch.empty_like(q)
    nbytes = attention_bytes([DECODE_CACHED + 1] * B, n, hq, hkv, d, 1)
    res = {}
    for ml in (8192, 8256, 8448, 12288, 16384, 4160):
        caches = [KVCache(B, hkv, ml, d, device_lens=False) for _ in range(2)]
        for i, c in enumerate(caches):
            _fill_gpu_random(torch, c, [DECODE_CACHED] * B, 60 + i)

        def step(i):
            c = caches[i & 1]
            append_attention(c, kn, kn, q, n, out=out)
            c.truncate([DECODE_CACHED] * B)

        t = _time_calls(torch, step, reps)
        res[str(ml)] = {"us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1)}
        del caches
        torch.cuda.empty_cache()
    for v in res.values():
        v["vs_8192"] = round(v["us"] / res["8192"]["us"], 4)
    return {"metric": "decode step time against the cache's max_len (row stride)", "unit": "us",
            "max_len": res, "config": {"workload": "llama8b_decode_b32_s4096", "batch": B, "keys": DECODE_CACHED + 1}}


def run_window(torch, reps=30):
    """Sliding-window decode: B=32 rows, a 4,096-key window over an 8,192-slot ring
    after 20,000 tokens (the ring has wrapped twice), T=1. Two caches in turn."""
    from gqa_attention_preallocated_amd import KVCache, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_WINDOW_DECODE
    B, hq, hkv, d, C = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim, sh.max_len
    win, L = sh.notes["window"], sh.notes["cached"]
    caches = [KVCache(B, hkv, C, d, device_lens=False, window=win) for _ in range(2)]
    g = torch.Generator(device="cuda").manual_seed(11)
    for c in caches:
        done = 0
        while done < L + 1:
            n = min(4096, L + 1 - done)
            x = (torch.randn(B, hkv, n, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
            c.append(x, x, [n] * B)
            done += n
    q = (torch.randn(B, hq, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
    out = torch.empty_like(q)
    n = [1] * B
    ws = torch.zeros(max(max(c.workspace_bytes(hq, 1, n) for c in caches), 256), dtype=torch.uint8, device="cuda")
    t = _time_calls(torch, lambda i: gqa_attention(q, caches[i & 1], n, out=out, workspace=ws), reps)
    # live K+V of the window (4,096 keys per row), q and out
    nbytes = B * win * hkv * d * 2 * 2 + 2 * B * hq * d * 2
    return {"metric": "sliding-window decode attention HBM GB/s", "value": round(nbytes / t / 1e9, 2), "unit": "GB/s",
            "frac_of_8TBs": round(nbytes / t / 8e12, 4), "ms": round(t * 1e3, 5), "bytes": nbytes,
            "config": {"workload": sh.name, "batch": B, "window": win, "ring_slots": C, "position": L, "T": 1}}


def run_fp8(torch, reps=30):
    """Decode over an E4M3 cache: the Llama decode shape (B=32, 4,096 cached + 1,
    T=1) with K and V stored as codes and one scale per KV head. Two caches in turn."""
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_DECODE
    B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
    sc = [2.0 ** -9] * hkv
    caches = [KVCache(B, hkv, sh.max_len, d, device_lens=False, fp8_scales=(sc, sc)) for _ in range(2)]
    g = torch.Generator(device="cuda").manual_seed(12)
    for c in caches:
        for n in (2048, 2048):
            x = (torch.randn(B, hkv, n, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
            c.append(x, x, [n] * B)
    q = (torch.randn(B, hq, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
    kn = (torch.randn(B, hkv, 1, d, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
    out = torch.empty_like(q)
    n = [1] * B
    caches[0].append(kn, kn, n)
    ws = torch.zeros(max(caches[0].workspace_bytes(hq, 1, n), 256), dtype=torch.uint8, device="cuda")
    caches[0].truncate([4096] * B)

    # the decode step: kv_append_attention (the decode kernel quantizes and
    # stores the new token itself), then a host-only rollback to 4,096
    def step(i):
        c = caches[i & 1]
        append_attention(c, kn, kn, q, n, out=out, workspace=ws)
        c.truncate([4096] * B)

    t_step = _time_calls(torch, step, reps)
    for c in caches:
        c.append(kn, kn, n)
    t = _time_calls(torch, lambda i: gqa_attention(q, caches[i & 1], n, out=out, workspace=ws), reps)
    # live K+V codes (one byte each), q and out in bfloat16; the step also
    # writes the new codes
    nbytes = B * 4097 * hkv * d * 2 + 2 * B * hq * d * 2
    step_bytes = nbytes + 2 * B * hkv * d
    return {"metric": "E4M3-cache decode step HBM GB/s", "value": round(step_bytes / t_step / 1e9, 2), "unit": "GB/s",
            "frac_of_8TBs": round(step_bytes / t_step / 8e12, 4), "ms": round(t_step * 1e3, 5), "bytes": step_bytes,
            "attention_only": {"ms": round(t * 1e3, 5), "bytes": nbytes, "GB/s": round(nbytes / t / 1e9, 2)},
            "config": {"workload": "llama8b_fp8_decode_b32_s4096", "batch": B, "keys": 4097, "T": 1,
                       "cache": "e4m3, one scale per kv head"}}


def run_tree(torch, reps=30):
    """Tree-based speculative verify: B=16 rows of 4,092 committed tokens, 8 draft
    nodes per row in a tree (two branches off node 0 and a second root). The
    step: kv_append_attention_tree of the 8 nodes, then a host-only rollback to
    4,092 (two caches in turn); also the tree attention call alone."""
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_VERIFY
    B, hq, hkv, d, T = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim, 8
    cached = sh.notes["cached"]
    caches = [KVCache(B, hkv, sh.max_len, d, device_lens=False) for _ in range(2)]
    n = [T] * B
    for i, c in enumerate(caches):
        _fill_gpu_random(torch, c, [cached] * B, 40 + i)
    g = torch.Generator(device="cuda").manual_seed(13)
    q = torch.randn(B, hq, T, d, device="cuda", generator=g).to(torch.bfloat16)
    kn = torch.randn(B, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty_like(q)
    parents = [[-1, 0, 1, 2, 0, 4, -1, 6]] * B
    caches[0].append(kn, kn, n)
    ws = torch.zeros(max(caches[0].workspace_bytes(hq, T, n), 256), dtype=torch.uint8, device="cuda")
    caches[0].truncate([cached] * B)

    def step(i):
        c = caches[i & 1]
        append_attention(c, kn, kn, q, n, out=out, workspace=ws, parents=parents)
        c.truncate([cached] * B)

    t_step = _time_calls(torch, step, reps)
    for c in caches:
        c.append(kn, kn, n)
    t = _time_calls(torch, lambda i: gqa_attention(q, caches[i & 1], n, out=out, workspace=ws, parents=parents),
                    reps)
    nbytes = attention_bytes([cached + T] * B, n, hq, hkv, d, T)
    step_bytes = nbytes + 2 * sum(n) * hkv * d * 2
    return {"metric": "tree verify step HBM GB/s", "value": round(step_bytes / t_step / 1e9, 2), "unit": "GB/s",
            "frac_of_8TBs": round(step_bytes / t_step / 8e12, 4), "ms": round(t_step * 1e3, 5), "bytes": step_bytes,
            "attention_only": {"ms": round(t * 1e3, 5), "bytes": nbytes, "GB/s": round(nbytes / t / 1e9, 2)},
            "config": {"workload": "llama8b_tree_verify_b16_n8_s4100", "batch": B, "nodes": T, "keys": cached + T}}


def run_ragged(torch, seed=4, reps=20):
    """Ragged batch: 64 rows, log-uniform lengths in [1, 32000], n_new in {0, 1, 4, 256}, T=256.
    The step: kv_append_attention of every row's new tokens, then a host-only
    rollback; also the attention call alone."""
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_RAGGED
    B, hq, hkv, d, T = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim, 256
    lens, n_new = W.ragged_rows(seed)
    cache = KVCache(B, hkv, sh.max_len, d, device_lens=False)
    _fill_gpu_random(torch, cache, lens, 30)
    g = torch.Generator(device="cuda").manual_seed(8)
    kn = torch.randn(B, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn(B, hq, T, d, device="cuda", generator=g).to(torch.bfloat16)
    n = [int(x) for x in n_new]
    base = [int(x) for x in lens]
    out = torch.empty_like(q)
    cache.append(kn, kn, n)
    ws = torch.zeros(max(cache.workspace_bytes(hq, T, n), 256), dtype=torch.uint8, device="cuda")
    t_att = _time_calls(torch, lambda i: gqa_attention(q, cache, n, out=out, workspace=ws), reps)
    cache.truncate(base)

    def step(i):
        append_attention(cache, kn, kn, q, n, out=out, workspace=ws)
        cache.truncate(base)

    t = _time_calls(torch, step, reps)
    after = [l + x for l, x in zip(base, n)]
    nbytes = attention_bytes(after, n, hq, hkv, d, T) + 2 * sum(n) * hkv * d * 2
    flops = attention_flops(after, n, hq, d)
    t_bw, t_mm = nbytes / 8e12, flops / 2.5e15
    return {"metric": "ragged batch step (append + attention), lower bound / time",
            "value": round(max(t_bw, t_mm) / t, 4), "unit": "fraction", "ms": round(t * 1e3, 5),
            "bytes": nbytes, "flops": flops, "hbm_frac": round(t_bw / t, 4), "mfma_frac": round(t_mm / t, 4),
            "attention_only_ms": round(t_att * 1e3, 5),
            "rows_by_n_new": {str(k): int((n_new == k).sum()) for k in (0, 1, 4, 256)},
            "config": {"workload": sh.name, "seed": seed, "batch": B, "T": T, "sum_lens": int(sum(after))}}


def run_paged(torch, reps=30):
    """Paged cache ([GQA] reversal: a block table and a paged kernel): the Llama
    decode step (B=32, 4,096 cached + 1) with rows interleaved page by page in
    the pool, at page sizes 64 and 256, against the same step on the linear
    cache; and the three ragged batches in a pool of exactly the pages their
    lengths need, against the dense cache, with the bytes each holds."""
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    import workloads as W
    sh = W.LLAMA8B_DECODE
    B, hq, hkv, d = sh.batch, sh.q_heads, sh.kv_heads, sh.head_dim
    g = torch.Generator(device="cuda").manual_seed(9)
    q = torch.randn(B, hq, 1, d, device="cuda", generator=g).to(torch.bfloat16)
    kn = torch.randn(B, hkv, 1, d, device="cuda", generator=g).to(torch.bfloat16)
    n = [1] * B
    nbytes = attention_bytes([DECODE_CACHED + 1] * B, n, hq, hkv, d, 1)
    decode = {}
    for name, P in (("linear", None), ("page64", 64), ("page256", 256)):
        if P is None:
            cache = KVCache(B, hkv, sh.max_len, d, device_lens=False)
            _fill_gpu_random(torch, cache, [DECODE_CACHED] * B, 31)
        else:
            cache = KVCache(B, hkv, sh.max_len, d, device_lens=False, page_size=P,
                            num_pages=B * -(-(DECODE_CACHED + 1) // P))
            _fill_gpu_random(torch, cache, [DECODE_CACHED] * B, 31, chunk=P)     # rows alternate page by page
        cache.append(kn, kn, n)
        out = torch.empty_like(q)
        t = _time_calls(torch, lambda i: gqa_attention(q, cache, n, out=out), reps)
        decode[name] = {"ms": round(t * 1e3, 5), "GB/s": round(nbytes / t / 1e9, 1),
                        "cache_bytes": cache.bytes}
        del cache
    ragged = []
    rs = W.LLAMA8B_RAGGED
    for seed in (4, 5, 6):
        lens, n_new = W.ragged_rows(seed)
        nl = [int(x) for x in n_new]
        after = [int(l) + x for l, x in zip(lens, nl)]
        T = 256
        qr = torch.randn(rs.batch, rs.q_heads, T, d, device="cuda", generator=g).to(torch.bfloat16)
        kr = torch.randn(rs.batch, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        row = {"seed": seed}
        for name, P in (("dense", None), ("page256", 256)):
            if P is None:
                cache = KVCache(rs.batch, hkv, rs.max_len, d, device_lens=False)
            else:
                cache = KVCache(rs.batch, hkv, rs.max_len, d, device_lens=False, page_size=P,
                                num_pages=sum(-(-a // P) for a in after))
            _fill_gpu_random(torch, cache, lens, 30)
            cache.append(kr, kr, nl)
            out = torch.empty_like(qr)
            ws = torch.zeros(max(cache.workspace_bytes(rs.q_heads, T, nl), 256), dtype=torch.uint8, device="cuda")
            t = _time_calls(torch, lambda i: gqa_attention(qr, cache, nl, out=out, workspace=ws), 20)
            row[name] = {"ms": round(t * 1e3, 5), "cache_bytes": cache.bytes}
            del cache
        row["time_ratio"] = round(row["page256"]["ms"] / row["dense"]["ms"], 4)
        row["bytes_ratio"] = round(row["page256"]["cache_bytes"] / row["dense"]["cache_bytes"], 4)
        ragged.append(row)
    return {"metric": "paged decode attention HBM GB/s", "value": decode["page256"]["GB/s"], "unit": "GB/s",
            "decode": decode, "ragged": ragged,
            "config": {"workload": sh.name + " / " + rs.name, "batch": B, "keys": DECODE_CACHED + 1}}


def run_probe(torch, reps=10):
    """Streaming-read probe (bench_probe.hip, built beside the library): the HBM
    read rate of a plain 16-byte-load kernel, plain and non-temporal, over two
    alternating 1 GiB buffers (four times the MALL). The attention kernels'
    rates are quoted against it as the practical ceiling."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbench_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.probe_stream_read.restype = ctypes.c_int
    nbytes = 1 << 30
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda"), torch.full((nbytes,), 2, dtype=torch.uint8,
                                                                             device="cuda")]
    sink = torch.empty(32768 * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = {}
    for nt in (0, 1):
        for blocks in (2048, 4096, 8192, 16384):
            ts = []
            for r in range(reps + 2):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                rc = lib.probe_stream_read(ctypes.c_void_p(bufs[r & 1].data_ptr()), nbytes, blocks, nt,
                                           ctypes.c_void_p(sink.data_ptr()), stream)
                e1.record()
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"probe_stream_read returned {rc}")
                if r >= 2:
                    ts.append(e0.elapsed_time(e1) * 1e-3)
            gbs = nbytes / sorted(ts)[len(ts) // 2] / 1e9
            key = "nontemporal" if nt else "plain"
            if gbs > best.get(key, (0, 0))[0]:
                best[key] = (gbs, blocks)
    del bufs, sink
    return {"plain_GB/s": round(best["plain"][0], 1), "plain_blocks": best["plain"][1],
            "nontemporal_GB/s": round(best["nontemporal"][0], 1), "nontemporal_blocks": best["nontemporal"][1],
            "bytes": nbytes, "note": "median of %d reads per launch shape; best shape reported" % reps}


DECODE_SEED, DECODE_CACHED = 1, 4096
# the event-timed roofline loop: untimed warm-up steps and timed launches, at
# least these many whatever --steps and --warmup are
ROOFLINE_WARMUP, ROOFLINE_REPS = 200, 400
# chunked-prefill oracle baseline: the chunk in the middle of the 10,240-token
# prompt (keys 0 .. 5,631), prompt seed as in run_prefill
PREFILL_SEED, PREFILL_CPU_CHUNK = 3, 10


def _oracle_worker(rank, nproc, reps, budget_s, barrier, results):
    """One host process of the CPU baseline: regenerate this worker's rows of the
    decode step from the seeded generators, wait for the others, then run the
    float64 oracle over them `reps` times on one thread, or until budget_s of
    compute has passed (checked after each row)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:       # pragma: no cover
        pass
    import workloads as W
    from oracle import direct
    sh = W.LLAMA8B_DECODE
    rows = list(range(rank, sh.batch, nproc))
    n = [1] * sh.batch
    q, k, v = W.step_inputs(sh, DECODE_SEED, 10_000, 1, n, pad="normal")
    data = []
    for b in rows:
        kh, vh = W.prefix_kv(sh, DECODE_SEED, b, 0, DECODE_CACHED)
        data.append((b, np.concatenate([kh, k[b, :, :1]], axis=1), np.concatenate([vh, v[b, :, :1]], axis=1)))
    # one untimed call: the first in a fresh interpreter pays one-off set-up (about 2 s)
    b0, k0, v0 = data[0]
    direct.attention_row(k0, v0, k0.shape[1], 1, q[b0], "bf16", [(0, 0)])
    barrier.wait()
    t0 = time.perf_counter()
    done = 0
    for _ in range(reps):
        for b, kr, vr in data:
            direct.attention_row(kr, vr, kr.shape[1], 1, q[b], "bf16", [(h, 0) for h in range(sh.q_heads)])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            continue
        break
    t1 = time.perf_counter()
    results.put((rank, done, t0, t1))


def _oracle_prefill_worker(rank, nproc, budget_s, barrier, results):
    """One host process of the chunked-prefill CPU baseline: regenerate the
    prompt up to chunk PREFILL_CPU_CHUNK, then run the float64 oracle over
    (row, query) units of that chunk (all 32 heads each), units dealt
    round-robin over the processes in a strided order over the chunk's
    queries, until budget_s of compute has passed (checked after each unit)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:       # pragma: no cover
        pass
    import workloads as W
    from oracle import direct
    sh = W.LLAMA8B_CHUNKED_PREFILL
    c = PREFILL_CPU_CHUNK
    n = [512] * sh.batch
    ks, vs = [], []
    for i in range(c + 1):
        q, k, v = W.step_inputs(sh, PREFILL_SEED, i, 512, n, pad="normal")
        ks.append(k)
        vs.append(v)
    L = 512 * (c + 1)
    kr = np.concatenate(ks, axis=2)                    # [B, Hkv, L, d]
    vr = np.concatenate(vs, axis=2)
    # units (b, t): t in a stride-67 order over the chunk so every worker's
    # sample spreads over early and late queries
    units = [(b, (67 * j) % 512) for j in range(512) for b in range(sh.batch)][rank::nproc]
    heads = range(sh.q_heads)
    direct.attention_row(kr[0], vr[0], L, 512, q[0], "bf16", [(0, 0)])     # one-off set-up, untimed
    barrier.wait()
    t0 = time.perf_counter()
    done, flop = 0, 0
    for b, t in units:
        direct.attention_row(kr[b], vr[b], L, 512, q[b], "bf16", [(h, t) for h in heads])
        done += 1
        flop += 4 * sh.head_dim * sh.q_heads * (L - 512 + t + 1)
        if time.perf_counter() - t0 > budget_s:
            break
    t1 = time.perf_counter()
    results.put((rank, done, t0, t1, flop))


def cpu_baseline_prefill(budget_s=1.5, max_procs=16):
    """The float64 oracle on the host over a sample of the chunked-prefill
    workload: (row, query) units of the middle chunk of the 10,240-token
    prompt, every head, over one single-threaded process per host core (at
    most max_procs). Reported in GFLOP/s of the same algorithmic count (4 d
    FLOP per visible pair and head)."""
    import multiprocessing as mp
    import workloads as W
    sh = W.LLAMA8B_CHUNKED_PREFILL
    nproc = max(1, min(max_procs, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(nproc), ctx.Queue()
    procs = [ctx.Process(target=_oracle_prefill_worker, args=(r, nproc, budget_s, barrier, results))
             for r in range(nproc)]
    for pr in procs:
        pr.start()
    got = [results.get(timeout=600) for _ in procs]
    for pr in procs:
        pr.join()
    units = sum(g[1] for g in got)
    flop = sum(g[4] for g in got)
    wall = max(g[3] for g in got) - min(g[2] for g in got)
    cpu_s = sum(g[3] - g[2] for g in got)
    total = sh.batch * 512
    return {"value": round(flop / wall / 1e9, 4), "unit": "GFLOP/s", "cores": nproc, "kind": "oracle",
            "sample": f"{units} of the {total} (row, query) units of chunk {PREFILL_CPU_CHUNK} "
                      f"(keys 0..{512 * (PREFILL_CPU_CHUNK + 1) - 1}) of the 10,240-token prompt "
                      f"({units / total:.1%}), each over all 32 heads; {flop / 1e9:.1f} GFLOP, "
                      f"{cpu_s:.1f} s of CPU over {nproc} single-threaded processes, {wall:.2f} s wall, "
                      f"float64 numpy"}


def cpu_baseline(reps=20, budget_s=1.5, max_procs=16):
    """The float64 oracle on the host: the whole decode step (32 rows x 32 heads)
    up to `reps` times, rows dealt over one single-threaded process per host core
    (at most max_procs), each stopping after budget_s of compute. Runs before
    this process touches the GPU; the workers are fresh interpreters that never
    do."""
    import multiprocessing as mp
    import workloads as W
    sh = W.LLAMA8B_DECODE
    nproc = max(1, min(max_procs, len(os.sched_getaffinity(0)), sh.batch))
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(nproc), ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(r, nproc, reps, budget_s, barrier, results)) for r in range(nproc)]
    for pr in procs:
        pr.start()
    got = [results.get(timeout=600) for _ in procs]
    for pr in procs:
        pr.join()
    rows = sum(g[1] for g in got)
    wall = max(g[3] for g in got) - min(g[2] for g in got)
    cpu_s = sum(g[3] - g[2] for g in got)
    b_per_row = attention_bytes([DECODE_CACHED + 1], [1], sh.q_heads, sh.kv_heads, sh.head_dim, 1)
    return {"value": round(rows * b_per_row / wall / 1e9, 4), "unit": "GB/s", "cores": nproc, "kind": "oracle",
            "sample": f"{rows} row-steps of the decode step (each: one row, all 32 heads, 4,097 keys; "
                      f"rows dealt round-robin, at most {reps} passes over the 32 rows), "
                      f"{cpu_s:.1f} s of CPU over {nproc} single-threaded processes, {wall:.2f} s wall, float64 numpy"}


def run_append(torch, reps=20):
    """Append bandwidth: B=32 rows, Llama KV shape, T in {1, 512, 2048, 4096} new tokens per row."""
    from gqa_attention_preallocated_amd import KVCache
    B, hkv, d = 32, 8, 128
    cache = KVCache(B, hkv, 8192, d, device_lens=False)
    g = torch.Generator(device="cuda").manual_seed(9)
    out = {}
    for T in (1, 512, 2048, 4096):
        k = torch.randn(B, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        n = [T] * B

        def call(i):
            cache.append(k, v, n)
            cache.truncate(0)
        t = _time_calls(torch, call, reps)
        nbytes = 2 * 2 * B * hkv * T * d * 2          # K and V, read once and written once
        out[str(T)] = {"us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1), "bytes": nbytes}
    return {"metric": "append HBM GB/s (K+V read + written)", "unit": "GB/s", "by_T": out,
            "config": {"workload": "llama8b_append_b32", "batch": B, "kv_heads": hkv, "head_dim": d}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "verify", "ragged", "append", "window", "fp8", "tree",
                                       "paged", "shard", "stride", "probe", "cpu"],
                    default=None,
                    help="time one workload only (for profiling); prints its own JSON line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run one plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.only == "cpu":
        print(json.dumps({"cpu_baseline": cpu_baseline(), "prefill_cpu_baseline": cpu_baseline_prefill()}),
              flush=True)
        return
    # the CPU baseline runs first, while no GPU context exists in this process
    cpu = cpu_pre = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline()
        if not args.no_prefill:
            cpu_pre = cpu_baseline_prefill()
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
        # the scale for the attention kernel's counters
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only == "ragged":
        print(json.dumps({"ragged": [run_ragged(torch, seed) for seed in (4, 5, 6)]}), flush=True)
        return
    if args.only in ("prefill", "verify", "append", "window", "fp8", "tree", "paged", "shard", "stride", "probe"):
        fn = {"prefill": run_prefill, "verify": run_verify, "append": run_append, "window": run_window,
              "fp8": run_fp8, "tree": run_tree, "paged": run_paged, "shard": run_shard, "stride": run_stride,
              "probe": run_probe}[args.only]
        print(json.dumps({args.only: fn(torch)}), flush=True)
        return
    res = run_decode(torch, args.steps, args.warmup)
    if args.only == "decode":
        args.no_prefill = True
        args.no_cpu_baseline = True
    step_bytes = res["att_bytes"] + res["append_bytes"]
    value = step_bytes / res["wall_s"] / 1e9
    achieved = step_bytes / (res["att_ms_avg"] * 1e-3) / 1e9
    line = {
        "metric": "decode attn HBM GB/s (% peak), Llama-8B shape B=32 S=4096; prefill TFLOP/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_s"] * 1e3, 4),
        "ms_per_step_two_calls": round(res["wall_two_calls_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(d) q, k, v; no weights)",
        "config": {"workload": res["shape"].name, "batch": 32, "q_heads": 32, "kv_heads": 8,
                   "head_dim": 128, "cached": 4096, "keys": 4097, "T": 1, "max_len": 8192,
                   "layers": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "decode_kernel (one launch per kv_append_attention call: the step)",
                     "bytes_per_launch": step_bytes,
                     "ms_avg": round(res["att_ms_avg"], 5),
                     "isolated_call_ms": {"p10": round(res["att_ms_p10"], 5), "p50": round(res["att_ms_p50"], 5),
                                          "p90": round(res["att_ms_p90"], 5)}},
    }
    if not args.no_prefill:
        line["prefill"] = run_prefill(torch)
        if cpu_pre is not None:
            line["prefill"]["cpu_baseline"] = cpu_pre
        probe = run_probe(torch)
        if probe is not None:
            probe["decode_kernel_frac"] = round(achieved / probe["nontemporal_GB/s"], 4)
            line["read_probe"] = probe
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
