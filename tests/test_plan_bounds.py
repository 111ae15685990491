"""CPU replay of every launch the library plans, checked for bounds and coverage.

The library's real host code (validation, lengths, work planning) is linked
against a simulator of the kernel launchers (tests/hostcheck/launch_sim.cpp)
that walks every block and column with the kernels' own indexing functions.
Each workload below is run through append + attention on fake addresses, and
the simulator must report no access outside a buffer, every output row written
exactly once per call, every appended slot written once, and the device lengths
equal to the host lengths.
"""

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session")
def sim(hostcheck_lib):
    lib = hostcheck_lib
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.kv_cache_create.argtypes = [I32, I32, I32, I32, ctypes.c_int, P, P, P, P, ctypes.POINTER(P)]
    lib.kv_cache_create_ring.argtypes = [I32, I32, I32, I32, ctypes.c_int, I32, P, P, P, P, ctypes.POINTER(P)]
    FP = ctypes.POINTER(ctypes.c_float)
    lib.kv_cache_create_fp8.argtypes = [I32, I32, I32, I32, FP, FP, P, P, P, P, ctypes.POINTER(P)]
    lib.kv_cache_create_paged.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.c_int, P, P, P, P, P,
                                          ctypes.POINTER(P)]
    lib.kv_get_block_table.argtypes = [P, I32P]
    lib.kv_free_pages.argtypes = [P]
    lib.kv_append.argtypes = [P, P, P, I32, I32P, P]
    lib.gqa_attention_workspace_size.argtypes = [P, I32, I32, I32P, ctypes.POINTER(ctypes.c_size_t)]
    lib.gqa_attention.argtypes = [P, P, I32, I32, I32P, P, P, ctypes.c_size_t, P]
    lib.gqa_attention_tree.argtypes = [P, P, I32, I32, I32P, I32P, P, P, ctypes.c_size_t, P]
    lib.kv_append_attention.argtypes = [P, P, P, P, I32, I32, I32P, P, P, ctypes.c_size_t, P]
    lib.kv_append_attention_workspace_size.argtypes = [P, I32, I32, I32P, ctypes.POINTER(ctypes.c_size_t)]
    lib.kv_append_attention_tree.argtypes = [P, P, P, P, I32, I32, I32P, I32P, P, P, ctypes.c_size_t, P]
    lib.kv_truncate.argtypes = [P, I32P, P]
    lib.kv_cache_set_policy.argtypes = [P, I32, I32]
    lib.kv_cache_destroy.argtypes = [P]
    lib.kv_last_error.restype = ctypes.c_char_p
    lib.hostcheck_region.argtypes = [ctypes.c_uint64, ctypes.c_size_t, ctypes.c_char_p]
    lib.hostcheck_error.restype = ctypes.c_char_p
    lib.hostcheck_out_row_writes.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64]
    lib.hostcheck_out_rows_total.restype = ctypes.c_int64
    lib.hostcheck_appended_chunks.restype = ctypes.c_int64
    lib.hostcheck_appended_dupes.restype = ctypes.c_int64
    lib.hostcheck_launches.restype = ctypes.c_int64
    lib.hostcheck_table.argtypes = [ctypes.c_int64]
    return lib


def _i32(vals):
    vals = [int(x) for x in vals]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


class SimCache:
    """A cache on fake, non-overlapping addresses inside the simulator."""

    GAP = 1 << 44

    def __init__(self, lib, B, hk, max_len, d, dtype, hq, t_max, window=None, paged=None):
        self.lib, self.B, self.hk, self.max_len, self.d, self.hq = lib, B, hk, max_len, d, hq
        self.elem = 4 if dtype == "f32" else 2                  # q, out, k_new, v_new
        cache_elem = {"f32": 4, "bf16": 2, "fp8": 1}[dtype]       # K, V
        lib.hostcheck_reset()
        self.addr = {}
        # paged = (page_size, num_pages): K and V are one pool, plus a block table
        self.paged = paged
        rows = B * max_len if paged is None else paged[1] * paged[0]
        self.max_blocks = 0 if paged is None else max_len // paged[0]
        sizes = {
            "k": rows * hk * d * cache_elem, "v": rows * hk * d * cache_elem,
            "table": 4 * max(B * self.max_blocks, 1),
            "lens": 4 * max(B, 1),
            "k_new": B * hk * t_max * d * self.elem, "v_new": B * hk * t_max * d * self.elem,
            "q": B * hq * t_max * d * self.elem, "out": B * hq * t_max * d * self.elem,
            "ws": 1 << 34,
        }
        for i, (name, size) in enumerate(sizes.items()):
            base = (i + 1) * self.GAP
            self.addr[name] = base
            lib.hostcheck_region(base, max(size, 1), name.encode())
        h = ctypes.c_void_p()
        bufs = (ctypes.c_void_p(self.addr["k"]), ctypes.c_void_p(self.addr["v"]), ctypes.c_void_p(self.addr["lens"]))
        if paged is not None:
            st = lib.kv_cache_create_paged(B, hk, paged[1], paged[0], self.max_blocks, d, 0 if dtype == "f32" else 1,
                                           *bufs[:2], ctypes.c_void_p(self.addr["table"]), bufs[2], None,
                                           ctypes.byref(h))
        elif dtype == "fp8":
            sc = (ctypes.c_float * max(hk, 1))(*([0.05] * hk))
            st = lib.kv_cache_create_fp8(B, hk, max_len, d, sc, sc, *bufs, None, ctypes.byref(h))
        elif window is None:
            st = lib.kv_cache_create(B, hk, max_len, d, 0 if dtype == "f32" else 1, *bufs, None, ctypes.byref(h))
        else:
            st = lib.kv_cache_create_ring(B, hk, max_len, d, 0 if dtype == "f32" else 1, window, *bufs, None,
                                          ctypes.byref(h))
        assert st == 0, lib.kv_last_error()
        self.window = window
        self.h = h
        self.lens = np.zeros(B, np.int64)
        self.appended = 0
        self.rewrote = False     # set after a rollback: slots get written again

    def append(self, T, n_new):
        st = self.lib.kv_append(self.h, ctypes.c_void_p(self.addr["k_new"]), ctypes.c_void_p(self.addr["v_new"]),
                                T, _i32(n_new), None)
        assert st == 0, self.lib.kv_last_error()
        self.lens += np.asarray(n_new)
        self.appended += int(np.sum(n_new)) * self.hk * self.d * self.elem // 16
        if (self.lens > self.max_len).any():
            self.rewrote = True              # a ring has wrapped: slots are written again

    def attention(self, T, n_new):
        size = ctypes.c_size_t()
        assert self.lib.gqa_attention_workspace_size(self.h, self.hq, T, _i32(n_new), ctypes.byref(size)) == 0
        assert size.value < (1 << 34)
        self.lib.hostcheck_begin_call()
        st = self.lib.gqa_attention(self.h, ctypes.c_void_p(self.addr["q"]), self.hq, T, _i32(n_new),
                                    ctypes.c_void_p(self.addr["out"]), ctypes.c_void_p(self.addr["ws"]),
                                    size.value, None)
        assert st == 0, self.lib.kv_last_error()
        return size.value

    def append_attention(self, T, n_new):
        """kv_append_attention; returns its workspace size, which must equal
        gqa_attention's for the lengths after the append."""
        size = ctypes.c_size_t()
        assert self.lib.kv_append_attention_workspace_size(self.h, self.hq, T, _i32(n_new), ctypes.byref(size)) == 0
        assert size.value < (1 << 34)
        self.lib.hostcheck_begin_call()
        a = self.addr
        st = self.lib.kv_append_attention(self.h, ctypes.c_void_p(a["k_new"]), ctypes.c_void_p(a["v_new"]),
                                          ctypes.c_void_p(a["q"]), self.hq, T, _i32(n_new), ctypes.c_void_p(a["out"]),
                                          ctypes.c_void_p(a["ws"]), size.value, None)
        assert st == 0, self.lib.kv_last_error()
        self.lens += np.asarray(n_new)
        self.appended += int(np.sum(n_new)) * self.hk * self.d * self.elem // 16
        if (self.lens > self.max_len).any():
            self.rewrote = True
        after = ctypes.c_size_t()
        assert self.lib.gqa_attention_workspace_size(self.h, self.hq, T, _i32(n_new), ctypes.byref(after)) == 0
        assert after.value == size.value
        return size.value

    def block_table(self):
        arr = (ctypes.c_int32 * max(1, self.B * self.max_blocks))()
        assert self.lib.kv_get_block_table(self.h, arr) == 0
        return np.array(list(arr)[: self.B * self.max_blocks], np.int64).reshape(self.B, self.max_blocks)

    def check(self, T=None):
        lib = self.lib
        errs = [lib.hostcheck_error(i).decode() for i in range(lib.hostcheck_error_count())]
        assert not errs, errs[:5]
        if not self.rewrote:
            assert lib.hostcheck_appended_dupes() == 0
            assert lib.hostcheck_appended_chunks() == self.appended
        for b in range(self.B):
            assert lib.hostcheck_lens_dev(b) == self.lens[b]
        if self.paged is not None:
            # the device table the kernels read equals the library's host table
            host = self.block_table()
            dev = [lib.hostcheck_table(i) for i in range(self.B * self.max_blocks)]
            assert host.reshape(-1).tolist() == dev
        if T is not None and self.B > 0 and T > 0:
            rows = self.B * self.hq * T
            row_bytes = self.d * self.elem
            assert lib.hostcheck_out_rows_total() == rows
            for i in range(rows):
                assert lib.hostcheck_out_row_writes(self.addr["out"], i, row_bytes) == 1, i


def _run(sim, B, hk, G, d, max_len, dtype, calls, policy=(0, 0)):
    t_max = max([c["T"] for c in calls] + [1])
    c = SimCache(sim, B, hk, max_len, d, dtype, hk * G, t_max)
    sim.kv_cache_set_policy(c.h, policy[0], policy[1])
    for call in calls:
        c.append(call["T"], call["n_new"])
        c.attention(call["T"], call["n_new"])
        c.check(call["T"])
    return c


@pytest.mark.parametrize("policy", [(0, 0), (1, 0), (2, 0), (1, 32), (2, 64)])
def test_tiny_schedule(sim, policy):
    sh = W.TINY_FP32
    _run(sim, sh.batch, sh.kv_heads, sh.group, sh.head_dim, sh.max_len, "f32", W.tiny_schedule(0), policy)


@pytest.mark.parametrize("kps", [2**31 - 1, 2**31 - 32, 2**31 - 64, 2**31 - 65, 10**9])
@pytest.mark.parametrize("path", [1, 2])
def test_huge_keys_per_split_means_one_split(sim, path, kps):
    """A split length near INT32_MAX ("never split") gives every row one split:
    rounding it up to the key tile must not wrap to a negative length and
    leave a row with no work items (its outputs unwritten, its fused append
    skipped)."""
    sh = W.TINY_FP32
    _run(sim, sh.batch, sh.kv_heads, sh.group, sh.head_dim, sh.max_len, "f32", W.tiny_schedule(0), (path, kps))
    # Llama-shaped rows: 4,097 keys each, decode and prefill kernels, one call
    # through kv_append_attention (the fused append writes every new token once)
    B, hk, hq, d = 4, 8, 32, 128
    c = SimCache(sim, B, hk, 8192, d, "bf16", hq, 4096)
    sim.kv_cache_set_policy(c.h, path, kps)
    for call in _prefix_calls([4096] * B):
        c.append(call["T"], call["n_new"])
    for T in (1, 64):
        ws = c.append_attention(T, [T] * B)
        assert ws == 0                           # one split per row: no partials
        c.check(T)
        sim.kv_truncate(c.h, _i32([4096] * B), None)
        c.lens[:] = 4096
        c.rewrote = True


def test_sanitized_replay():
    """The host library (abi.cpp with the launch simulator) under AddressSanitizer
    and UndefinedBehaviorSanitizer: the smaller simulator cases of this file and
    the host ABI checks, in a child process that preloads the ASan runtime. Any
    report aborts the child."""
    if os.environ.get("GQAKV_HOSTCHECK_SANITIZE") == "1":
        pytest.skip("already the sanitized run")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime for g++ here")
    env = dict(os.environ)
    env.update({"GQAKV_HOSTCHECK_SANITIZE": "1", "LD_PRELOAD": asan,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    sel = ("tiny_schedule or random_trials or huge_keys or ring_schedules or paged_random or mqa "
           "or more_rows or append_attention_trials or tree_verify or refus or invalid "
           "or capacity_error or argument_checks or truncate_rules or paged_create")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-p", "no:xdist",
           os.path.join(ROOT, "tests", "test_plan_bounds.py"), os.path.join(ROOT, "tests", "test_abi_host.py"),
           "-k", sel]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail


@pytest.mark.parametrize("seed", range(40))
def test_random_trials(sim, seed):
    shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
    for policy in [(0, 0), (1, 32), (2, 64)]:
        _run(sim, shape.batch, shape.kv_heads, shape.group, shape.head_dim, shape.max_len,
             "bf16" if seed % 2 else "f32", calls, policy)


def _prefix_calls(lens, chunk=4096):
    """Appends that bring every row to lens[b] (chunks of at most `chunk`)."""
    lens = np.asarray(lens)
    done = np.zeros_like(lens)
    calls = []
    while (done < lens).any():
        n = np.minimum(lens - done, chunk)
        calls.append({"T": int(n.max()), "n_new": n.tolist()})
        done += n
    return calls


def _setup(sim, shape, lens, t_max):
    c = SimCache(sim, shape.batch, shape.kv_heads, shape.max_len, shape.head_dim, shape.dtype,
                 shape.q_heads, max(t_max, 4096))
    for call in _prefix_calls(lens):
        c.append(call["T"], call["n_new"])
    return c


def test_llama_decode(sim):
    sh = W.LLAMA8B_DECODE
    c = _setup(sim, sh, [4096] * sh.batch, 1)
    for _ in range(2):
        c.append(1, [1] * sh.batch)
        ws = c.attention(1, [1] * sh.batch)
        c.check(1)
        sim.kv_truncate(c.h, _i32([4096] * sh.batch), None)
        c.lens[:] = 4096
        c.rewrote = True
        c.check()
    assert ws == 0            # 256 (row, kv head) items fill the chip: no cross-group split


def test_llama_verify(sim):
    sh = W.LLAMA8B_VERIFY
    c = _setup(sim, sh, [4092] * sh.batch, 4)
    c.append(4, [4] * sh.batch)
    c.attention(4, [4] * sh.batch)
    c.check(4)


def test_llama_chunked_prefill(sim):
    sh = W.LLAMA8B_CHUNKED_PREFILL
    c = SimCache(sim, sh.batch, sh.kv_heads, sh.max_len, sh.head_dim, "bf16", sh.q_heads, 512)
    for chunk in range(20):
        c.append(512, [512] * sh.batch)
        c.attention(512, [512] * sh.batch)
        c.check(512)
    assert c.lens.tolist() == [10240] * sh.batch


@pytest.mark.parametrize("seed", [4, 5, 6])
def test_llama_ragged(sim, seed):
    sh = W.LLAMA8B_RAGGED
    lens, n_new = W.ragged_rows(seed)
    c = _setup(sim, sh, lens, 256)
    c.append(256, n_new)
    c.attention(256, n_new)
    c.check(256)


def test_more_rows_than_one_launch_table(sim):
    B = 150
    rng = np.random.default_rng(0)
    lens = rng.integers(1, 300, B)
    c = SimCache(sim, B, 2, 512, 64, "bf16", 8, 300)
    for call in _prefix_calls(lens, 128):
        c.append(call["T"], call["n_new"])
    n_new = rng.choice([0, 1, 3, 40], B)
    n_new = np.minimum(n_new, c.lens)
    c.attention(40, n_new)
    c.check(40)
    sim.kv_truncate(c.h, _i32(c.lens // 2), None)
    c.lens = c.lens // 2
    c.rewrote = True
    c.check()


def test_mqa_and_mha_shapes(sim):
    for hk, G in [(1, 32), (1, 64), (1, 128), (8, 1), (2, 3)]:
        c = SimCache(sim, 2, hk, 256, 128, "bf16", hk * G, 64)
        c.append(64, [64, 30])
        c.attention(64, [64, 30])
        c.check(64)
        c.append(3, [1, 3])
        c.attention(3, [1, 3])
        c.check(3)


@pytest.mark.parametrize("d,C,win", [(16, 64, 1), (64, 128, 50), (128, 128, 128), (128, 192, 64), (32, 256, 200)])
def test_ring_schedules(sim, d, C, win):
    """Sliding-window rings: every launch stays inside its buffers, reads only
    held keys through slots that never wrap inside a tile, and writes every
    output row once, over many wraps, under every kernel selection."""
    calls, lens = W.ring_schedule(d * 1000 + C + win, 3, C, win, 200, min(40, C - win + 1))
    assert lens.max() > C + 8                     # the schedule wraps the ring
    for policy in [(0, 0), (1, 0), (2, 0), (1, 32), (2, 64)]:
        c = SimCache(sim, 3, 2, C, d, "bf16", 8, max(x["T"] for x in calls), window=win)
        sim.kv_cache_set_policy(c.h, *policy)
        for call in calls:
            c.append(call["T"], call["n_new"])
            if max(call["n_new"]) > 0:
                c.attention(call["T"], call["n_new"])
                c.check(call["T"])


def test_ring_capacity_and_rollback_rules(sim):
    """An append that would evict a key its first new query needs, and a rollback
    below what the ring still holds, are refused and change nothing."""
    C, W = 128, 64
    c = SimCache(sim, 1, 1, C, 64, "bf16", 4, 128, window=W)
    c.append(128, [128])
    assert sim.kv_append(c.h, ctypes.c_void_p(c.addr["k_new"]), ctypes.c_void_p(c.addr["v_new"]), 128,
                         _i32([66]), None) == 2          # KV_ERR_CAPACITY: 66 > C - W + 1
    assert b"evict" in sim.kv_last_error()
    c.append(65, [65])                                   # the limit: the ring now holds positions 65..192
    # a rollback to n' needs keys from n' - 63 on: 127 needs key 64 (evicted), 128 needs 65 (held)
    assert sim.kv_truncate(c.h, _i32([127]), None) == 1
    assert b"Invalid truncation length" in sim.kv_last_error()
    assert sim.kv_truncate(c.h, _i32([128]), None) == 0
    c.lens[:] = 128
    c.rewrote = True
    c.check()
    c.append(65, [65])
    c.attention(65, [65])
    c.check(65)


@pytest.mark.parametrize("seed", range(12))
def test_fp8_random_trials(sim, seed):
    """E4M3 caches: appends write one code byte per element inside the cache,
    and attention reads 1-byte rows, at every head dim and kernel selection."""
    shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
    for policy in [(0, 0), (1, 32), (2, 64)]:
        _run(sim, shape.batch, shape.kv_heads, shape.group, shape.head_dim, shape.max_len, "fp8", calls, policy)


def test_llama_fp8_decode(sim):
    sh = W.LLAMA8B_DECODE
    c = SimCache(sim, sh.batch, sh.kv_heads, sh.max_len, sh.head_dim, "fp8", sh.q_heads, 4096)
    for call in _prefix_calls([4096] * sh.batch):
        c.append(call["T"], call["n_new"])
    c.append(1, [1] * sh.batch)
    assert c.attention(1, [1] * sh.batch) == 0
    c.check(1)


def test_tree_verify_launches_and_rules(sim):
    """Tree verify plans decode launches only, inside every buffer, one write
    per output row; bad parents, too many nodes, rings and a forced prefill
    kernel are refused."""
    sh = W.LLAMA8B_VERIFY
    c = SimCache(sim, sh.batch, sh.kv_heads, sh.max_len, sh.head_dim, "bf16", sh.q_heads, 4096)
    for call in _prefix_calls([4092] * sh.batch):
        c.append(call["T"], call["n_new"])
    T = 8
    n = [8] * (sh.batch - 2) + [5, 0]
    c.append(T, n)
    parents = [-1, 0, 1, 2, 0, 4, -1, 6] * sh.batch
    size = ctypes.c_size_t()
    assert sim.gqa_attention_workspace_size(c.h, sh.q_heads, T, _i32(n), ctypes.byref(size)) == 0
    sim.hostcheck_begin_call()
    st = sim.gqa_attention_tree(c.h, ctypes.c_void_p(c.addr["q"]), sh.q_heads, T, _i32(n), _i32(parents),
                                ctypes.c_void_p(c.addr["out"]), ctypes.c_void_p(c.addr["ws"]), size.value, None)
    assert st == 0, sim.kv_last_error()
    c.check(T)

    def call(par, T_=T, n_=n):
        return sim.gqa_attention_tree(c.h, ctypes.c_void_p(c.addr["q"]), sh.q_heads, T_, _i32(n_), _i32(par),
                                      ctypes.c_void_p(c.addr["out"]), ctypes.c_void_p(c.addr["ws"]), 1 << 30,
                                      None)
    bad = list(parents)
    bad[3] = 3                                  # a node cannot be its own parent
    assert call(bad) == 1 and b"parent" in sim.kv_last_error()
    assert call([-1] * (sh.batch * 17), 17, [0] * sh.batch) == 3       # more than 16 nodes
    sim.kv_cache_set_policy(c.h, 2, 0)
    assert call(parents) == 3


def _paged_pair(sim, B, hk, G, d, max_len, dtype, t_max, P, pages):
    """A simulated paged cache and the oracle's page bookkeeping (K/V of width 1)."""
    from oracle import paged as opaged
    c = SimCache(sim, B, hk, max_len, d, dtype, hk * G, t_max, paged=(P, pages))
    ref = opaged.PagedCache(B, 1, pages, P, max_len // P, 1)
    return c, ref


def _ref_append(ref, n_new):
    n = np.asarray(n_new)
    T = max(int(n.max()), 1) if len(n) else 1
    z = np.zeros((len(n), 1, T, 1), np.float32)
    ref.append(z, z, n)


@pytest.mark.parametrize("seed", range(16))
def test_paged_random_trials(sim, seed):
    """Paged caches: every append writes through pages the block table gives the
    row, every attention tile reads one page of the row, and the table the
    kernels see equals the host table and the oracle's page assignment (lowest
    free page first), under every kernel selection, with rollbacks freeing
    pages along the way."""
    shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
    P = (64, 128, 256)[seed % 3]
    S = -(-shape.max_len // P) * P
    pages = shape.batch * (S // P)            # enough for every row at once
    t_max = max([c["T"] for c in calls] + [1])
    for policy in [(0, 0), (1, 32), (2, 64)]:
        c, ref = _paged_pair(sim, shape.batch, shape.kv_heads, shape.group, shape.head_dim, S,
                             "bf16" if seed % 2 else "f32", t_max, P, pages)
        sim.kv_cache_set_policy(c.h, *policy)
        for i, call in enumerate(calls):
            c.append(call["T"], call["n_new"])
            _ref_append(ref, call["n_new"])
            c.attention(call["T"], call["n_new"])
            c.check(call["T"])
            assert np.array_equal(c.block_table(), ref.table)
            assert sim.kv_free_pages(c.h) == len(ref.free)
            if i % 3 == 2:                     # roll every row back by a third
                new = c.lens - c.lens // 3
                assert sim.kv_truncate(c.h, _i32(new), None) == 0
                ref.truncate(new)
                c.lens = new.copy()
                c.rewrote = True
                c.check()
                assert np.array_equal(c.block_table(), ref.table)


def test_paged_pool_rules(sim):
    """A pool that cannot give a call all its pages refuses it and changes
    nothing; so does a row past max_blocks; page sizes outside the rules and
    E4M3 storage are refused at creation."""
    c, ref = _paged_pair(sim, 2, 1, 4, 64, 256, "bf16", 256, 64, 5)
    c.append(130, [130, 64])                   # 3 + 1 pages
    _ref_append(ref, [130, 64])
    before = (c.block_table().copy(), sim.kv_free_pages(c.h))
    k = ctypes.c_void_p(c.addr["k_new"])
    assert sim.kv_append(c.h, k, k, 70, _i32([70, 70]), None) == 2      # 1 + 2 pages > 1 free
    assert b"pages needed" in sim.kv_last_error()
    assert sim.kv_append(c.h, k, k, 130, _i32([127, 0]), None) == 2     # 257 > 4 blocks of 64
    assert np.array_equal(c.block_table(), before[0]) and sim.kv_free_pages(c.h) == before[1]
    c.check()
    assert sim.kv_truncate(c.h, _i32([64, 64]), None) == 0             # row 0 frees 2 pages
    ref.truncate([64, 64])
    c.lens[:] = [64, 64]
    c.rewrote = True
    c.append(70, [70, 60])                     # 2 + 1 pages: the pool's last three
    _ref_append(ref, [70, 60])
    assert np.array_equal(c.block_table(), ref.table) and sim.kv_free_pages(c.h) == 0
    c.attention(70, [70, 60])
    c.check(70)
    h = ctypes.c_void_p()
    a = ctypes.c_void_p(c.addr["k"])
    t = ctypes.c_void_p(c.addr["table"])
    for P, pages, blocks, dt in [(32, 4, 4, 1), (96, 4, 4, 1), (64, 0, 4, 1), (64, 4, 0, 1), (64, 4, 4, 2)]:
        st = sim.kv_cache_create_paged(2, 1, pages, P, blocks, 64, dt, a, a, t, None, None, ctypes.byref(h))
        assert st in (1, 3), (P, pages, blocks, dt)


def test_paged_llama_ragged(sim):
    """The 64 ragged Llama-shaped rows (1 .. 32,000 cached, 0 to 256 new) in a
    pool of exactly the pages their lengths need: decode and prefill launches
    stay inside the pool, and the pool is a fraction of the dense reservation."""
    sh = W.LLAMA8B_RAGGED
    lens, n_new = W.ragged_rows(4)
    P = 256
    pages = int(sum(-(-int(L + n) // P) for L, n in zip(lens, n_new)))
    c = SimCache(sim, sh.batch, sh.kv_heads, sh.max_len, sh.head_dim, "bf16", sh.q_heads, 4096, paged=(P, pages))
    for call in _prefix_calls(lens):
        c.append(call["T"], call["n_new"])
    c.append(int(max(n_new)), n_new)
    assert sim.kv_free_pages(c.h) == 0
    c.attention(int(max(n_new)), n_new)
    c.check(int(max(n_new)))
    assert pages * P < 0.6 * sh.batch * sh.max_len


@pytest.mark.parametrize("seed", range(24))
def test_append_attention_trials(sim, seed):
    """kv_append_attention: every new token written once (by the copy kernel or
    by the decode kernel's items, never both), every k_new read inside the
    row's new tokens, lens_dev and every output row set, under each policy and
    cache kind."""
    shape, calls = W.trial_spec(seed, head_dims=(16, 32, 64, 128))
    kind = ["f32", "bf16", "ring", "paged", "fp8", "bf16"][seed % 6]
    for policy in [(0, 0), (1, 32), (2, 64)]:
        t_max = max([c["T"] for c in calls] + [1])
        hq = shape.kv_heads * shape.group
        if kind == "paged":
            P = 64
            max_len = -(-shape.max_len // P) * P
            pages = shape.batch * (max_len // P)
            c = SimCache(sim, shape.batch, shape.kv_heads, max_len, shape.head_dim, "bf16", hq, t_max,
                         paged=(P, pages))
        elif kind == "ring":
            c = SimCache(sim, shape.batch, shape.kv_heads, 64, shape.head_dim, "bf16", hq, t_max,
                         window=64 - t_max + 1)
        else:
            c = SimCache(sim, shape.batch, shape.kv_heads, shape.max_len, shape.head_dim, kind, hq, t_max)
        sim.kv_cache_set_policy(c.h, policy[0], policy[1])
        for call in calls:
            c.append_attention(call["T"], call["n_new"])
            c.check(call["T"])


def test_append_attention_llama_decode_and_ragged(sim):
    """Llama-3.1-8B shapes: a decode step over 32 rows of 8191 keys, and a
    mixed batch (decode, verify and prefill rows) in one call, on linear and
    paged caches."""
    for paged in (None, (256, 32 * 34)):
        c = SimCache(sim, 32, 8, 8704, 128, "bf16", 32, 4096, paged=paged)
        for call in _prefix_calls([8191] * 32):
            c.append(call["T"], call["n_new"])
        c.append_attention(1, [1] * 32)
        c.check(1)
        n = [1, 4, 512, 0] * 8
        c.append_attention(512, n)
        c.check(512)


@pytest.mark.parametrize("d,C,win", [(64, 128, 50), (128, 192, 64)])
def test_append_attention_ring_wraps(sim, d, C, win):
    """kv_append_attention on a sliding-window ring over many wraps."""
    calls, lens = W.ring_schedule(d * 1000 + C + win + 1, 3, C, win, 200, min(40, C - win + 1))
    assert lens.max() > C + 8
    for policy in [(0, 0), (1, 32)]:
        c = SimCache(sim, 3, 2, C, d, "bf16", 8, max(x["T"] for x in calls), window=win)
        sim.kv_cache_set_policy(c.h, *policy)
        for call in calls:
            c.append_attention(call["T"], call["n_new"])
            c.check(call["T"])


def test_append_attention_tree(sim):
    """kv_append_attention_tree: the tree's tokens written exactly once by the
    decode kernel's items, every output row once, lens_dev set; the tree rules
    refuse a bad parent before anything is written."""
    sh = W.LLAMA8B_VERIFY
    c = SimCache(sim, sh.batch, sh.kv_heads, sh.max_len, sh.head_dim, "bf16", sh.q_heads, 4096)
    for call in _prefix_calls([4092] * sh.batch):
        c.append(call["T"], call["n_new"])
    T = 8
    n = [8] * (sh.batch - 2) + [5, 0]
    parents = [-1, 0, 1, 2, 0, 4, -1, 6] * sh.batch
    size = ctypes.c_size_t()
    assert sim.kv_append_attention_workspace_size(c.h, sh.q_heads, T, _i32(n), ctypes.byref(size)) == 0
    a = c.addr

    def call(par):
        sim.hostcheck_begin_call()
        return sim.kv_append_attention_tree(c.h, ctypes.c_void_p(a["k_new"]), ctypes.c_void_p(a["v_new"]),
                                            ctypes.c_void_p(a["q"]), sh.q_heads, T, _i32(n), _i32(par),
                                            ctypes.c_void_p(a["out"]), ctypes.c_void_p(a["ws"]), size.value, None)
    bad = list(parents)
    bad[3] = 3
    launches = sim.hostcheck_launches()
    assert call(bad) == 1 and b"parent" in sim.kv_last_error()
    assert sim.hostcheck_launches() == launches          # refused before any launch
    assert call(parents) == 0, sim.kv_last_error()
    c.lens += np.asarray(n)
    c.appended += int(np.sum(n)) * c.hk * c.d * c.elem // 16
    c.check(T)


def test_append_attention_tree_wide_rows(sim):
    """A tree call with 48 columns a row (G=4, T=12). The automatic plan gives
    rows that wide to the prefill kernel; a tree call keeps them on the split-K
    decode kernel, and the workspace query covers that plan: the call succeeds
    with exactly the queried bytes and writes every new token once. At 24 rows
    x 8 KV heads (192 items) the prefill plan needs no split, and with it no
    workspace, while the decode plan splits each row in two."""
    B, hk, hq, d, T = 24, 8, 32, 128, 12
    c = SimCache(sim, B, hk, 8192, d, "bf16", hq, 4096)
    for call in _prefix_calls([4092] * B):
        c.append(call["T"], call["n_new"])
    n = [T] * (B - 1) + [7]
    parents = list(range(-1, T - 1)) * B
    size = ctypes.c_size_t()
    assert sim.kv_append_attention_workspace_size(c.h, hq, T, _i32(n), ctypes.byref(size)) == 0
    assert size.value > 0                       # split-K partials of the decode plan
    a = c.addr
    sim.hostcheck_begin_call()
    st = sim.kv_append_attention_tree(c.h, ctypes.c_void_p(a["k_new"]), ctypes.c_void_p(a["v_new"]),
                                      ctypes.c_void_p(a["q"]), hq, T, _i32(n), _i32(parents),
                                      ctypes.c_void_p(a["out"]), ctypes.c_void_p(a["ws"]), size.value, None)
    assert st == 0, sim.kv_last_error()
    c.lens += np.asarray(n)
    c.appended += int(np.sum(n)) * c.hk * c.d * c.elem // 16
    c.check(T)


def test_noalloc_entry_point(sim):
    """kv_append_attention_noalloc: the same launches as kv_append_attention with
    the library's scratch as workspace (the simulator maps it onto the
    registered workspace region), every kernel on one stream; a call whose
    partials need more than the scratch is refused before anything is
    enqueued, with nothing changed."""
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    sim.kv_append_attention_noalloc.argtypes = [P, P, P, P, I32, I32, ctypes.POINTER(I32), P, P]
    B, hk, hq, d = 16, 8, 32, 128
    c = SimCache(sim, B, hk, 8192, d, "bf16", hq, 4096)
    for call in _prefix_calls([4092] * B):
        c.append(call["T"], call["n_new"])
    a = c.addr
    for T in (4, 1):                            # verify, then a smaller decode call: both split rows
        size = ctypes.c_size_t()
        assert sim.kv_append_attention_workspace_size(c.h, hq, T, _i32([T] * B), ctypes.byref(size)) == 0
        assert 0 < size.value <= 16 << 20
        sim.hostcheck_begin_call()
        st = sim.kv_append_attention_noalloc(c.h, P(a["k_new"]), P(a["v_new"]), P(a["q"]), hq, T, _i32([T] * B),
                                             P(a["out"]), None)
        assert st == 0, sim.kv_last_error()
        c.lens += T
        c.appended += B * T * hk * d * c.elem // 16
        c.check(T)
    # a prefill row forced into 64-key splits needs far more than 16 MiB of partials
    sim.kv_cache_set_policy(c.h, 2, 64)
    launches = sim.hostcheck_launches()
    st = sim.kv_append_attention_noalloc(c.h, P(a["k_new"]), P(a["v_new"]), P(a["q"]), hq, 256, _i32([256] * B),
                                         P(a["out"]), None)
    assert st == 4
    assert "16777216 bytes of scratch" in sim.kv_last_error().decode()
    assert sim.hostcheck_launches() == launches
    lens = (ctypes.c_int32 * B)()
    assert sim.kv_get_lens(c.h, lens) == 0 and list(lens) == c.lens.tolist()


@pytest.mark.parametrize("kps, splits, combine", [(0, 32, False), (1024, 8, False), (128, 64, False),
                                                  (64, 128, True)])
def test_split_decode_rows_merge(sim, kps, splits, combine):
    """Decode rows split into at most 64 work groups are merged by the last of
    them in the decode kernel (after every partial of its group was written,
    with the group's arrival counter in the workspace past the partials): no
    combine launch. Rows split further, which only a small keys-per-split
    policy asks for, go through the combine kernel. Either way every output
    row is written exactly once."""
    B, hk, hq, d = 4, 2, 8, 128
    c = SimCache(sim, B, hk, 8192 + 64, d, "bf16", hq, 4096)
    for call in _prefix_calls([8191] * B):
        c.append(call["T"], call["n_new"])
    sim.kv_cache_set_policy(c.h, 1, kps)
    c.append(1, [1] * B)
    launches = sim.hostcheck_launches()
    ws = c.attention(1, [1] * B)
    c.check(1)
    assert sim.hostcheck_launches() - launches == (2 if combine else 1)
    # partials (d + 2 floats per record, 16 columns per group and split), then
    # one counter word per group and split, each region 256-byte aligned
    records = B * hk * splits * 16
    up = lambda x: (x + 255) // 256 * 256
    assert ws == up(up(records * d * 4) + records * 8) + records // 16 * 8


@pytest.mark.parametrize("G, T, want", [(4, 16, 2), (4, 8, 2), (4, 4, 1), (8, 8, 2), (64, 1, 4)])
def test_float32_d128_decode_subtiles(sim, G, T, want):
    """A float32 cache at d = 128 runs the decode kernel with at most two
    16-column subtiles when the group allows (its four-subtile instance spills
    registers): a tree call over G*T > 32 columns gets more query tiles
    instead, each reading the row's keys. Every output is still written once."""
    B, hk, d = 2, 2, 128
    c = SimCache(sim, B, hk, 1024, d, "f32", hk * G, 512)
    for call in _prefix_calls([300, 77]):
        c.append(call["T"], call["n_new"])
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    sim.gqa_attention_tree.argtypes = [P, P, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32), P, P,
                                       ctypes.c_size_t, P]
    sim.hostcheck_last_decode_nsub.restype = ctypes.c_int
    c.append(T, [T] * B)
    size = ctypes.c_size_t()
    assert sim.gqa_attention_workspace_size(c.h, hk * G, T, _i32([T] * B), ctypes.byref(size)) == 0
    parents = [t - 1 for t in range(T)] * B                     # a chain per row
    sim.hostcheck_begin_call()
    a = c.addr
    st = sim.gqa_attention_tree(c.h, P(a["q"]), hk * G, T, _i32([T] * B), _i32(parents), P(a["out"]),
                                P(a["ws"]), size.value, None)
    assert st == 0, sim.kv_last_error()
    c.check(T)
    assert sim.hostcheck_last_decode_nsub() == want
