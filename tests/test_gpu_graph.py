"""HIP graph capture of the library's calls.

Every call enqueues only kernel launches (and, for mixed batches, an event
fork and join with the handle's side stream): no copies, memsets or device
allocations, so a serving loop can capture a step into a HIP graph and replay
it without the host work of the call. A captured call replays the lengths it
was captured with (the host state moves once, at capture), which fits the
step the benchmark times: append at a fixed length, attend, roll back.

Each test captures one step, then replays it several times with new q, k_new
and v_new copied into the captured buffers, with eager reference calls on a
second cache and synchronizations between the replays, and checks every replay
against the eager result bit for bit (output and cache bytes).
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import fill_rows, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    from gqa_attention_preallocated_amd import KVCache, append_attention, gqa_attention
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return KVCache, append_attention, gqa_attention


CASES = [
    # (name, T, n_new per row, policy)
    ("decode", 1, [1, 1, 1, 1], (0, 0)),
    ("decode_split", 1, [1, 1, 1, 1], (1, 64)),
    ("verify_padded", 4, [4, 4, 2, 0], (0, 0)),
    ("prefill_chunk", 128, [128, 128, 128, 128], (0, 0)),
    ("mixed", 128, [1, 4, 128, 0], (0, 0)),
]


@pytest.mark.parametrize("name,T,n,policy", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("one_call", [True, False], ids=["one_call", "two_calls"])
def test_captured_step_replays_match_eager(name, T, n, policy, one_call):
    KVCache, append_attention, gqa_attention = _lib()
    B, hk, G, d, S = 4, 2, 4, 128, 2048
    shape = W.Shape("graph", "bf16", B, hk * G, hk, d, S)
    lens = [1000, 1537, 64, 700]
    cap, ref = KVCache(B, hk, S, d), KVCache(B, hk, S, d)
    fill_rows([cap, ref], shape, 81, lens)
    for c in (cap, ref):
        c.set_policy(*policy)
    q0, k0, v0 = W.step_inputs(shape, 81, 0, T, n, pad="normal")
    q, k, v = to_dev(q0, "bf16"), to_dev(k0, "bf16"), to_dev(v0, "bf16")
    out = torch.empty_like(q)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    ws_ref = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")

    def step():
        if one_call:
            append_attention(cap, k, v, q, n, out=out, workspace=ws)
        else:
            cap.append(k, v, n)
            gqa_attention(q, cap, n, out=out, workspace=ws)

    # one eager step first (a mixed call creates the side stream here), rolled back
    step()
    cap.truncate(lens)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    cap.truncate(lens)                       # the host state moved once, at capture
    torch.cuda.synchronize()
    for r in range(1, 4):
        qn, kn, vn = W.step_inputs(shape, 81, r, T, n, pad="normal")
        q.copy_(to_dev(qn, "bf16"))
        k.copy_(to_dev(kn, "bf16"))
        v.copy_(to_dev(vn, "bf16"))
        g.replay()
        ref.append(k, v, n)
        want = gqa_attention(q, ref, n, workspace=ws_ref)
        ref.truncate(lens)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"{name} replay {r}: output bits"
        assert torch.equal(cap.k.view(torch.int16), ref.k.view(torch.int16)), f"{name} replay {r}: K bytes"
        assert torch.equal(cap.v.view(torch.int16), ref.v.view(torch.int16)), f"{name} replay {r}: V bytes"
        # the replay left the device lengths at the captured post-append values
        want_dev = torch.tensor([L + x for L, x in zip(lens, n)], dtype=torch.int32)
        assert torch.equal(cap.lens_dev[:B].cpu(), want_dev), f"{name} replay {r}: device lengths"
        assert cap.lens == lens
    del g
