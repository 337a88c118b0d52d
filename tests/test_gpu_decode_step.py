"""GPU checks of swa_decode_step, the fused decode step.

Mistral 7B (Chinese translation), section 2, paragraphs "Rolling Buffer Cache"
and "Pre-fill and Chunking": a generated token's keys and values are stored in
slot pos mod W, then the token attends to the window.  swa_decode_step does
both in one launch, so it must reproduce swa_cache_write followed by
swa_decode bit for bit (outputs and cache contents), and match the fp64 oracle
within the usual tolerance.  A step is also captured in a HIP graph and
replayed with new tokens and advanced positions.
"""
import numpy as np
import pytest

import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import batched_decode, make_workload
from helpers import check_close, dev, host_f32, host_raw, oracle_all, poisoned_cache, torch, write_history

pytestmark = pytest.mark.gpu


def clone_cache(c):
    return swa.Cache(c.k.clone(), c.v.clone())


def workspace(cache, n, hq):
    nb = swa.swa_decode_workspace_size(cache, n, hq)
    return torch().empty(max(nb, 16), dtype=torch().uint8, device="cuda"), nb


def separate_and_fused(wl, cache):
    """Run write + decode on one copy of the cache and the fused step on another."""
    t = torch()
    c_sep, c_fus = clone_cache(cache), clone_cache(cache)
    batch = swa.Batch([1] * wl.num_seqs, [s.start_pos for s in wl.seqs], wl.cache_idx)
    q, kn, vn = dev(wl.q, wl.dtype), dev(wl.k_new, wl.dtype), dev(wl.v_new, wl.dtype)
    ws, nb = workspace(cache, wl.num_seqs, wl.n_q_heads)
    dt = t.bfloat16 if wl.dtype == "bf16" else t.float32
    o_sep = t.full((wl.num_seqs, wl.n_q_heads, wl.head_dim), float("nan"), dtype=dt, device="cuda")
    o_fus = t.full_like(o_sep, float("nan"))
    swa.swa_cache_write(c_sep, batch, kn, vn)
    swa.swa_decode(c_sep, batch, q, wl.n_q_heads, wl.scale, o_sep, ws, nb)
    swa.swa_decode_step(c_fus, batch, q, wl.n_q_heads, kn, vn, wl.scale, o_fus, ws, nb)
    t.cuda.synchronize()
    return (c_sep, o_sep), (c_fus, o_fus)


def assert_same_bits(a, b, what):
    t = torch()
    iv = t.int16 if a.dtype == t.bfloat16 else t.int32
    assert t.equal(a.view(iv), b.view(iv)), what


@pytest.mark.parametrize("dtype,window,group", [("bf16", 4096, 4), ("bf16", 100, 8), ("bf16", 1, 1),
                                                ("bf16", 4096, 1), ("bf16", 1000, 1), ("bf16", 300, 2),
                                                ("f32", 64, 4), ("f32", 5, 1)])
@pytest.mark.parametrize("d", [128, 64, 16])
def test_fused_step_equals_write_then_decode(dtype, window, group, d):
    hkv = 2
    positions = sorted({0, 1, max(0, window - 2), window - 1, window, window + 1, 3 * window + 5, 9000})
    wl = make_workload("step", 70 + window, [(p, 1) for p in positions], window=window, n_q_heads=hkv * group,
                       n_kv_heads=hkv, head_dim=d, dtype=dtype, cache_rows=list(reversed(range(len(positions)))))
    cache = poisoned_cache(wl.n_cache, hkv, window, d, dtype)
    write_history(cache, wl)
    (c_sep, o_sep), (c_fus, o_fus) = separate_and_fused(wl, cache)
    assert_same_bits(o_sep, o_fus, "output")
    assert_same_bits(c_sep.k, c_fus.k, "cache K")
    assert_same_bits(c_sep.v, c_fus.v, "cache V")
    check_close(host_f32(o_fus, dtype), oracle_all(wl), dtype, f"fused step W={window}")


@pytest.mark.parametrize("group,batch", [(1, 16), (1, 64)])
def test_fused_step_full_size_other_groups(group, batch):
    """Full 4096-slot rings with 32 query heads over 32 / G KV heads.  G = 1 runs on
    the VALU kernel: 16 sequences x 32 KV heads split every window in 4, so the new
    token's slot lands in a split sp > 0 for most sequences; 64 sequences need no split."""
    hkv = 32 // group
    pos = np.random.default_rng(1300 + group + batch).integers(4096, 32768, size=batch)
    wl = make_workload(f"step-g{group}", 1400 + group + batch, [(int(p), 1) for p in pos], window=4096,
                       n_q_heads=32, n_kv_heads=hkv, head_dim=128, dtype="bf16")
    cache = poisoned_cache(batch, hkv, 4096, 128, "bf16")
    write_history(cache, wl)
    (c_sep, o_sep), (c_fus, o_fus) = separate_and_fused(wl, cache)
    assert_same_bits(o_sep, o_fus, "output")
    assert_same_bits(c_sep.k, c_fus.k, "cache K")
    assert_same_bits(c_sep.v, c_fus.v, "cache V")
    check_close(host_f32(o_fus, "bf16"), oracle_all(wl), "bf16", f"fused step G={group} B={batch}")


@pytest.mark.parametrize("batch", [64, 8])
def test_fused_step_full_size_batched_decode(batch):
    """Sequences at positions in [4096, 32768), full 4096-slot rings: 64 sequences (one
    workgroup per ring) and 8 (split windows, workspace and merge)."""
    wl = batched_decode(1004, batch=batch)
    cache = poisoned_cache(batch, 8, 4096, 128, "bf16")
    write_history(cache, wl)
    (c_sep, o_sep), (c_fus, o_fus) = separate_and_fused(wl, cache)
    assert_same_bits(o_sep, o_fus, "output")
    assert_same_bits(c_sep.k, c_fus.k, "cache K")
    assert_same_bits(c_sep.v, c_fus.v, "cache V")
    check_close(host_f32(o_fus, "bf16"), oracle_all(wl), "bf16", "fused step, batched decode")


@pytest.mark.parametrize("group", [2, 8])
def test_fused_step_full_size_group_sizes(group):
    """16 sequences, full 4096-slot rings, 32 query heads over 32 / G KV heads (split plans)."""
    hkv = 32 // group
    pos = np.random.default_rng(1300 + group).integers(4096, 32768, size=16)
    wl = make_workload(f"step-g{group}", 1400 + group, [(int(p), 1) for p in pos], window=4096, n_q_heads=32,
                       n_kv_heads=hkv, head_dim=128, dtype="bf16")
    cache = poisoned_cache(16, hkv, 4096, 128, "bf16")
    write_history(cache, wl)
    (c_sep, o_sep), (c_fus, o_fus) = separate_and_fused(wl, cache)
    assert_same_bits(o_sep, o_fus, "output")
    assert_same_bits(c_sep.k, c_fus.k, "cache K")
    assert_same_bits(c_sep.v, c_fus.v, "cache V")
    check_close(host_f32(o_fus, "bf16"), oracle_all(wl), "bf16", f"fused step G={group}")


@pytest.mark.parametrize("start", [[5000, 4096, 4200, 12345], [2044, 100, 2047, 3000]])
def test_graph_captured_step_replays_match_eager_steps(start):
    """Capture one fused step (split plan, with workspace), then replay it for
    several generated tokens: between replays the inputs are refilled and the
    device positions advance.  Every replay must equal the same step run
    eagerly on a second cache, output and cache bit for bit.  The second set of
    positions starts below W: two sequences cross 2048 valid slots while the
    graph replays, which changes how their slots are spread over the splits."""
    t = torch()
    n, hq, hkv, d, window = 4, 32, 8, 128, 4096
    rng = np.random.default_rng(123)
    wl = make_workload("graph", 124, [(p, 1) for p in start], window=window, n_q_heads=hq, n_kv_heads=hkv,
                       head_dim=d, dtype="bf16")
    cache_g = poisoned_cache(n, hkv, window, d, "bf16")
    write_history(cache_g, wl)
    cache_e = clone_cache(cache_g)

    batch_g = swa.Batch([1] * n, start, list(range(n)))
    batch_e = swa.Batch([1] * n, start, list(range(n)))
    q = t.empty((n, hq, d), dtype=t.bfloat16, device="cuda")
    kn = t.empty((n, hkv, d), dtype=t.bfloat16, device="cuda")
    vn = t.empty((n, hkv, d), dtype=t.bfloat16, device="cuda")
    out_g = t.empty((n, hq, d), dtype=t.bfloat16, device="cuda")
    out_e = t.empty_like(out_g)
    ws_g, nb = workspace(cache_g, n, hq)
    ws_e, _ = workspace(cache_g, n, hq)
    assert nb > 0

    def refill():
        q.copy_(t.from_numpy(rng.standard_normal((n, hq, d), dtype=np.float32)).to(t.bfloat16))
        kn.copy_(t.from_numpy(rng.standard_normal((n, hkv, d), dtype=np.float32)).to(t.bfloat16))
        vn.copy_(t.from_numpy(rng.standard_normal((n, hkv, d), dtype=np.float32)).to(t.bfloat16))

    refill()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):  # warm-up launch outside the capture, on a scratch cache
        scratch = clone_cache(cache_g)
        swa.swa_decode_step(scratch, batch_g, q, hq, kn, vn, wl.scale, out_g, ws_g, nb)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    del scratch

    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        swa.swa_decode_step(cache_g, batch_g, q, hq, kn, vn, wl.scale, out_g, ws_g, nb)
    for step in range(5):
        if step > 0:
            refill()
            batch_g.sp.add_(1)
            batch_e.sp.add_(1)
            batch_e.h_sp += 1
        graph.replay()
        t.cuda.synchronize()
        swa.swa_decode_step(cache_e, batch_e, q, hq, kn, vn, wl.scale, out_e, ws_e, nb)
        t.cuda.synchronize()
        assert_same_bits(out_g, out_e, f"replay {step}: output")
        assert_same_bits(cache_g.k, cache_e.k, f"replay {step}: cache K")
        assert_same_bits(cache_g.v, cache_e.v, f"replay {step}: cache V")
        assert not t.isnan(out_g.float()).any()
