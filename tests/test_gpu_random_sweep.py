"""Seeded random sweep over the whole call surface, against the oracle.

Each case draws its own shape and batch:
- dtype, head_dim, group size, KV heads and window;
- a ragged batch: some sequences with no history and some past the first lap of the
  ring, chunks longer than the window, an occasional empty sequence, and a permuted map
  of cache rows with unused rows.

It then runs, through the C ABI, what one layer does with such a batch:
- the history goes in with swa_cache_write;
- swa_prefill_chunk runs, and then the chunk's own cache write;
- a decode batch at random positions runs as write-then-attend (swa_cache_write +
  swa_decode) or as the fused swa_decode_step.

Every output is compared with the oracle's attention over the unrolled history. Every
ring is compared bytewise with the oracle's ring simulator. The windows straddle 512
slots, where the decode starts to split a window across workgroups, so the batches
also reach the split and stream plans and their merges.

The rules checked are those of Mistral 7B (Chinese translation), section 2: the
paragraph "Sliding Window Attention" (a query attends to the last W positions), the
paragraph "Rolling Buffer Cache" (position i in slot i mod W) and the paragraph
"Pre-fill and Chunking" (a chunk attends to the cache and causally to itself).
"""
import numpy as np
import pytest

import oracle
import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import make_workload, to_f32
from helpers import (check_close, dev, empty, host_raw, new_batch, oracle_seq, poisoned_cache,
                     write_history)

N_CASES = 128
WINDOWS = [1, 2, 5, 31, 64, 100, 257, 511, 512, 700, 1024]


def draw_case(i):
    rng = np.random.default_rng(9000 + i)
    c = {"case": i}
    c["dtype"] = "f32" if rng.random() < 0.25 else "bf16"
    c["d"] = int(rng.choice([16, 64, 128]))
    c["G"] = int(rng.choice([1, 2, 4, 8]))
    c["hkv"] = int(rng.choice([1, 2, 4]))
    w = int(rng.choice(WINDOWS))
    c["window"] = w

    def start():
        r = rng.random()
        if r < 0.3:
            return 0
        if r < 0.6:
            return int(rng.integers(1, w + 1))
        return int(rng.integers(w, 3 * w + 2))

    n_pre = int(rng.integers(1, 7))
    budget = 384
    spec = []
    for _ in range(n_pre):
        r = rng.random()
        if r < 0.1:
            n_new = 0
        elif r < 0.35:
            n_new = int(rng.integers(w, 2 * w + 3))       # a chunk as long as the window or longer
        else:
            n_new = int(rng.integers(1, min(w, 96) + 1))
        n_new = min(n_new, budget)
        budget -= n_new
        spec.append((start(), n_new))
    c["prefill"] = spec
    c["prefill_extra_rows"] = int(rng.integers(0, 3))
    n_dec = int(rng.choice([1, 2, 3, 5, 9, 16]))
    c["decode"] = [(start(), 1) for _ in range(n_dec)]
    c["decode_extra_rows"] = int(rng.integers(0, 3))
    c["fused"] = bool(rng.random() < 0.5)
    c["mirrors"] = bool(rng.random() < 0.75)
    c["rows_seed"] = int(rng.integers(1 << 30))
    return c


def permuted_rows(n, extra, seed):
    """Cache rows for n sequences out of n + extra, in a seeded random order."""
    return [int(x) for x in np.random.default_rng(seed).permutation(n + extra)[:n]]


def ring_reference(cache, wl, batches):
    """The oracle's rings after the poisoned start and the given (rows_k, rows_v, lengths, starts) writes."""
    ring_k = host_raw(cache.k, wl.dtype).copy()
    ring_v = host_raw(cache.v, wl.dtype).copy()
    for kk, vv, lens, starts in batches:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        oracle.ring_write(ring_k, kk, cu, starts, wl.cache_idx)
        oracle.ring_write(ring_v, vv, cu, starts, wl.cache_idx)
    return ring_k, ring_v


def assert_rings(cache, wl, ring_k, ring_v, what):
    gk, gv = host_raw(cache.k, wl.dtype), host_raw(cache.v, wl.dtype)
    assert np.array_equal(gk.view(np.uint8), ring_k.view(np.uint8)), f"{what}: K ring differs"
    assert np.array_equal(gv.view(np.uint8), ring_v.view(np.uint8)), f"{what}: V ring differs"


def make(c, name, spec, extra, seed):
    rows = permuted_rows(len(spec), extra, c["rows_seed"] + seed)
    return make_workload(name, 10_000 * c["case"] + seed, spec, window=c["window"],
                         n_q_heads=c["G"] * c["hkv"], n_kv_heads=c["hkv"], head_dim=c["d"],
                         dtype=c["dtype"], cache_rows=rows, n_cache=len(spec) + extra)


def history_batch(wl):
    lens = [s.start_pos - s.hist_lo for s in wl.seqs]
    return wl.hist_packed("k"), wl.hist_packed("v"), lens, [s.hist_lo for s in wl.seqs]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    import torch
    c = draw_case(i)
    tag = str(c)
    print(f"[sweep] {tag}", flush=True)
    d, w, dtype = c["d"], c["window"], c["dtype"]

    # ---- prefill: history, attend, then the chunk's own write
    wl = make(c, "sweep-prefill", c["prefill"], c["prefill_extra_rows"], 1)
    cache = poisoned_cache(wl.n_cache, wl.n_kv_heads, w, d, dtype)
    hist = history_batch(wl)
    ring_k, ring_v = ring_reference(cache, wl, [hist])
    write_history(cache, wl)
    assert_rings(cache, wl, ring_k, ring_v, f"history write, {tag}")
    if wl.total_tokens > 0:
        q, kn, vn = dev(wl.q, dtype), dev(wl.k_new, dtype), dev(wl.v_new, dtype)
        out = empty((wl.total_tokens, wl.n_q_heads, d), dtype)
        out.fill_(float("nan"))
        batch = new_batch(wl, mirrors=c["mirrors"])
        swa.swa_prefill_chunk(cache, batch, q, wl.n_q_heads, kn, vn, wl.scale, out)
        got = to_f32(host_raw(out, dtype), dtype)
        ref = np.concatenate([oracle_seq(wl, b) for b in range(wl.num_seqs)])
        check_close(got, ref, dtype, f"prefill, {tag}")
        swa.swa_cache_write(cache, batch, kn, vn)
        cu = wl.cu_seqlens
        oracle.ring_write(ring_k, wl.k_new, cu, wl.start_pos, wl.cache_idx)
        oracle.ring_write(ring_v, wl.v_new, cu, wl.start_pos, wl.cache_idx)
        assert_rings(cache, wl, ring_k, ring_v, f"chunk write, {tag}")

    # ---- decode: one token per sequence, write then attend (or the fused step)
    wd = make(c, "sweep-decode", c["decode"], c["decode_extra_rows"], 2)
    cache = poisoned_cache(wd.n_cache, wd.n_kv_heads, w, d, dtype)
    ring_k, ring_v = ring_reference(cache, wd, [history_batch(wd)])
    write_history(cache, wd)
    batch = new_batch(wd, mirrors=c["mirrors"])
    q, kn, vn = dev(wd.q, dtype), dev(wd.k_new, dtype), dev(wd.v_new, dtype)
    out = empty((wd.num_seqs, wd.n_q_heads, d), dtype)
    out.fill_(float("nan"))
    ws_bytes = swa.swa_decode_workspace_size(cache, wd.num_seqs, wd.n_q_heads)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    if c["fused"]:
        swa.swa_decode_step(cache, batch, q, wd.n_q_heads, kn, vn, wd.scale, out, ws, ws_bytes)
    else:
        swa.swa_cache_write(cache, batch, kn, vn)
        swa.swa_decode(cache, batch, q, wd.n_q_heads, wd.scale, out, ws, ws_bytes)
    got = to_f32(host_raw(out, dtype), dtype)
    ref = np.concatenate([oracle_seq(wd, b) for b in range(wd.num_seqs)])
    check_close(got, ref, dtype, f"decode ({'fused step' if c['fused'] else 'write + decode'}), {tag}")
    cu = np.arange(wd.num_seqs + 1, dtype=np.int32)
    oracle.ring_write(ring_k, wd.k_new, cu, wd.start_pos, wd.cache_idx)
    oracle.ring_write(ring_v, wd.v_new, cu, wd.start_pos, wd.cache_idx)
    assert_rings(cache, wd, ring_k, ring_v, f"decode write, {tag}")


def test_sweep_reaches_every_plan_and_shape():
    """The drawn cases cover every dtype, head_dim and group size, windows on both sides
    of 512 slots, and decode batches of one and of several sequences (host logic only)."""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert {c["dtype"] for c in cases} == {"bf16", "f32"}
    assert {c["d"] for c in cases} == {16, 64, 128}
    assert {c["G"] for c in cases} == {1, 2, 4, 8}
    assert any(c["window"] >= 512 and len(c["decode"]) >= 2 and c["dtype"] == "bf16" for c in cases)
    assert any(c["window"] < 512 for c in cases)
    assert any(len(c["decode"]) == 1 for c in cases) and any(c["fused"] for c in cases)
    assert any(any(n >= c["window"] for _, n in c["prefill"]) for c in cases)
