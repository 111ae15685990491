"""Rows of the split-K decode kernel split across work groups.

A (row, KV head, query tile) split into at most 64 work groups is merged by
the last of them to finish, inside the decode kernel, after counting arrivals
on a word of the workspace; a row split further (only a small keys-per-split
policy asks for that) goes through the combine kernel. Both paths against the
oracle, in one call and across policies; and the merge against whatever the
workspace held before the call: zeros, random bytes, all-ones, the words an
earlier call left, or the leftovers of a call with another plan.
"""

import numpy as np
import pytest
import torch

from oracle import direct
import workloads as W
from gpu_util import assert_close, fill_rows, out_f64, row_history, to_dev

pytestmark = pytest.mark.gpu

SHAPE = W.Shape("merge", "bf16", 3, 8, 2, 128, 8192 + 64)
LENS = [8191, 5000, 333]
SEED = 31


def _setup():
    from gqa_attention_preallocated_amd import KVCache
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sh = SHAPE
    cache = KVCache(sh.batch, sh.kv_heads, sh.max_len, sh.head_dim)
    fill_rows(cache, sh, SEED, LENS)
    return cache


def _step(cache, T, n, r):
    """Append the step's tokens; returns (q as stored, k, v, q on the device)."""
    q, k, v = W.step_inputs(SHAPE, SEED, 10_000 + r, T, n, pad="nan")
    cache.append(to_dev(k, "bf16"), to_dev(v, "bf16"), n)
    return q, k, v, to_dev(q, "bf16")


@pytest.mark.parametrize("policy", [(1, 64), (1, 128), (1, 1024), (0, 0)],
                         ids=["combine_and_merge", "64_splits", "8_splits", "auto"])
def test_split_rows_against_oracle(policy):
    """(1, 64): rows of 8,192 and 5,001 keys split into 128 and 79 work groups
    (combine kernel) beside a row of 334 keys in 6 (merged in the decode
    kernel), in one call; (1, 128): 64 splits, the most the in-kernel merge
    takes. Every row and head of a decode step and of a verify step (T = 4)."""
    from gqa_attention_preallocated_amd import gqa_attention
    cache = _setup()
    cache.set_policy(*policy)
    for r, T in enumerate((1, 4)):
        n = [T] * SHAPE.batch
        q, k, v, qd = _step(cache, T, n, r)
        got = out_f64(gqa_attention(qd, cache, n), "bf16")
        for b in range(SHAPE.batch):
            L = cache.lens[b]
            kr, vr = row_history(SHAPE, SEED, b, L - T, k[b, :, :T], v[b, :, :T])
            ref = direct.attention_row(kr, vr, L, T, q[b], "bf16",
                                       [(h, t) for h in range(SHAPE.q_heads) for t in range(T)])
            assert_close(got[b], ref, "bf16", f"policy {policy} T {T} row {b}")
        cache.truncate(LENS)


def test_merge_ignores_prior_workspace_contents():
    """The output bits do not depend on what the workspace held: the merge
    reads the partials in split order whichever work group is last, and a
    counter word no call left behind counts as zero arrivals. Calls on one
    workspace in a row (the second finds the words the first left), and a
    call with another plan in between, give the bits of a zeroed workspace."""
    from gqa_attention_preallocated_amd import gqa_attention
    cache = _setup()
    cache.set_policy(1, 512)                                   # up to 17 splits per row
    hq = SHAPE.q_heads
    n1, n4 = [1] * SHAPE.batch, [4] * SHAPE.batch
    _, _, _, q1 = _step(cache, 1, n1, 0)
    size = max(cache.workspace_bytes(hq, 1, n1), 256)
    cache.truncate(LENS)
    _, _, _, q4 = _step(cache, 4, n4, 1)
    size = max(size, cache.workspace_bytes(hq, 4, n4))
    cache.truncate(LENS)

    def run(q, T, n, ws, r):
        _step(cache, T, n, r)                                  # the same k/v as before
        out = gqa_attention(q, cache, n, workspace=ws)
        cache.truncate(LENS)
        torch.cuda.synchronize()
        return out.view(torch.int16).clone()

    fresh = lambda: torch.zeros(size, dtype=torch.uint8, device="cuda")
    want1, want4 = run(q1, 1, n1, fresh(), 0), run(q4, 4, n4, fresh(), 1)
    g = torch.Generator(device="cuda").manual_seed(5)
    noise = torch.randint(0, 256, (size,), dtype=torch.uint8, device="cuda", generator=g)
    ones = torch.full((size,), 255, dtype=torch.uint8, device="cuda")
    for name, ws in (("random bytes", noise), ("all ones", ones)):
        assert torch.equal(run(q1, 1, n1, ws, 0), want1), f"{name}: first call"
        assert torch.equal(run(q1, 1, n1, ws, 0), want1), f"{name}: second call on the same workspace"
        assert torch.equal(run(q4, 4, n4, ws, 1), want4), f"{name}: verify plan after decode"
        assert torch.equal(run(q1, 1, n1, ws, 0), want1), f"{name}: decode after verify"
