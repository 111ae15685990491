"""Helpers for the GPU tests: moving seeded storage arrays to and from the device
and comparing against the CPU oracle at the contract tolerances."""

from __future__ import annotations

import numpy as np
import torch

import workloads as W

# Contract tolerances (max absolute error against the float64 oracle):
# float32 inputs 1e-5; bfloat16 inputs with float32 accumulation 2e-2.
TOL_ABS = {"f32": 1e-5, "bf16": 2e-2}
# Internal gate on top of the contract: at these magnitudes an all-zero output
# would pass 2e-2, so the worst error must also be small next to the largest
# reference value. bf16 rounds P and the output to 8 significant bits
# (relative 2^-9 each), so a correct kernel sits near 0.4%; 1e-2 leaves margin.
TOL_REL = {"f32": 1e-5, "bf16": 1e-2}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> storage array (float32, or bf16 bit patterns as uint16)."""
    h = t.detach().cpu().contiguous()
    if dtype == "f32":
        return h.numpy()
    return h.view(torch.int16).numpy().view(np.uint16)


def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return stored.astype(np.float64)
    return W.bf16_bits_to_f32(stored).astype(np.float64)


def out_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return widen(from_dev(t, dtype), dtype)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if got.size == 0:
        return
    err = float(np.abs(got - ref).max())
    scale = float(np.abs(ref).max())
    assert err <= TOL_ABS[dtype], f"{what}: max abs error {err:.3e} > {TOL_ABS[dtype]}"
    if scale > 0:
        assert err <= TOL_REL[dtype] * scale, f"{what}: max error {err:.3e} vs max |ref| {scale:.3e}"
    return err


def same_bytes(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                                 np.ascontiguousarray(b).view(np.uint8))


def fill_rows(cache, shape, seed, lens, chunk=2048):
    """Append each row's seeded history (prefix_kv) until row b holds lens[b]
    tokens (into each cache of a list, when given one)."""
    caches = cache if isinstance(cache, (list, tuple)) else [cache]
    lens = np.asarray(lens)
    B, hk, d = shape.batch, shape.kv_heads, shape.head_dim
    start = 0
    while start < lens.max():
        n = np.clip(lens - start, 0, chunk)
        T = int(n.max())
        k = np.zeros((B, hk, T, d), W.storage_np_dtype(shape.dtype))
        v = np.zeros_like(k)
        for b in range(B):
            if n[b] > 0:
                k[b, :, :n[b]], v[b, :, :n[b]] = W.prefix_kv(shape, seed, b, start, int(n[b]))
        kd, vd = to_dev(k, shape.dtype), to_dev(v, shape.dtype)
        for c in caches:
            c.append(kd, vd, n.tolist())
        start += chunk


def row_history(shape, seed, b, length, extra_k=None, extra_v=None):
    k, v = W.prefix_kv(shape, seed, b, 0, length)
    if extra_k is not None:
        k = np.concatenate([k, extra_k], axis=1)
        v = np.concatenate([v, extra_v], axis=1)
    return k, v
