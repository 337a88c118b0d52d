"""GPU parity of swa_decode against the fp64 oracle.

Mistral 7B (Chinese translation), section 2: after the prompt, tokens are
generated one at a time (paragraph "Pre-fill and Chunking"); each reads the W
most recent positions from the rolling buffer (paragraphs "Sliding Window
Attention", "Rolling Buffer Cache").  The new token is written first.
"""
import math

import numpy as np
import pytest

import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import batched_decode, make_workload
from helpers import (check_close, dev, expected_hist, host_f32, host_raw, one_hot_v, oracle_all, poisoned_cache,
                     run_decode, torch, write_history)

pytestmark = pytest.mark.gpu


def decode_case(seed, positions, window, hq, hkv, d, dtype, rows=None):
    n = len(positions)
    wl = make_workload("dec", seed, [(p, 1) for p in positions], window=window, n_q_heads=hq, n_kv_heads=hkv,
                       head_dim=d, dtype=dtype, cache_rows=rows)
    cache = poisoned_cache(wl.n_cache, hkv, window, d, dtype)
    write_history(cache, wl)
    got = host_f32(run_decode(wl, cache), dtype)
    return check_close(got, oracle_all(wl), dtype, f"decode W={window} n={n}")


@pytest.mark.parametrize("window", [1, 3, 64, 100, 1000, 4096])
def test_bf16_positions_around_the_window(window):
    positions = sorted({0, 1, max(0, window - 2), window - 1, window, window + 1, 3 * window + 5, 20000})
    decode_case(window, positions, window, 32, 8, 128, "bf16", rows=list(reversed(range(len(positions)))))


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_bf16_groups(group):
    hkv = 2
    decode_case(40 + group, [0, 17, 300, 5000], 512, hkv * group, hkv, 128, "bf16")


@pytest.mark.parametrize("d", [16, 64, 128])
def test_fp32(d):
    decode_case(50 + d, [0, 5, 64, 65, 1000], 64, 8, 2, d, "f32")


def test_window_one_is_exact():
    wl = make_workload("w1", 3, [(p, 1) for p in (0, 9, 100)], window=1, n_q_heads=8, n_kv_heads=2,
                       head_dim=128, dtype="bf16")
    cache = poisoned_cache(3, 2, 1, 128, "bf16")
    got = host_raw(run_decode(wl, cache), "bf16")
    for h in range(8):
        assert np.array_equal(got[:, h, :], wl.v_new[:, h // 4, :])


@pytest.mark.parametrize("batch", [64, 8])
def test_full_size_batched_decode(batch):
    """Sequences at positions in [4096, 32768), full 4096-slot rings, 32 q / 8 kv heads.
    64 sequences take one workgroup per ring; 8 sequences split each window (workspace and merge)."""
    wl = batched_decode(1004, batch=batch)
    cache = poisoned_cache(batch, 8, 4096, 128, "bf16")
    write_history(cache, wl)
    got = host_f32(run_decode(wl, cache), "bf16")
    check_close(got, oracle_all(wl), "bf16", "batched decode")


@pytest.mark.parametrize("group,batch", [(1, 16), (2, 16), (8, 16), (8, 64)])
def test_full_size_group_sizes(group, batch):
    """Full 4096-slot rings at the other group sizes: 32 query heads over 32 / G KV heads.
    (1, 16): the VALU kernel, 4 splits per ring; matrix-core kernel: (2, 16) 2 splits per ring,
    (8, 16) 8 splits, (8, 64) 2 splits."""
    hkv = 32 // group
    pos = np.random.default_rng(1100 + group + batch).integers(4096, 32768, size=batch)
    wl = make_workload(f"groups-{group}-{batch}", 1200 + group + batch, [(int(p), 1) for p in pos], window=4096,
                       n_q_heads=32, n_kv_heads=hkv, head_dim=128, dtype="bf16")
    cache = poisoned_cache(batch, hkv, 4096, 128, "bf16")
    write_history(cache, wl)
    assert swa.swa_decode_workspace_size(cache, batch, 32) > 0
    got = host_f32(run_decode(wl, cache), "bf16")
    check_close(got, oracle_all(wl), "bf16", f"decode G={group} B={batch}")


def test_many_short_sequences_single_split_plan():
    # enough (sequence, head) pairs that the plan uses no workspace
    positions = list(np.random.default_rng(2).integers(0, 300, size=300))
    wl = make_workload("many", 4, [(int(p), 1) for p in positions], window=256, n_q_heads=32, n_kv_heads=8,
                       head_dim=128, dtype="bf16")
    assert swa.swa_decode_workspace_size(poisoned_cache(1, 8, 256, 128, "bf16"), 300, 32) == 0
    cache = poisoned_cache(300, 8, 256, 128, "bf16")
    write_history(cache, wl)
    got = host_f32(run_decode(wl, cache), "bf16")
    check_close(got, oracle_all(wl), "bf16", "many short")


def test_deterministic_bitwise():
    wl = make_workload("det", 5, [(p, 1) for p in (10, 5000, 4095)], window=4096, n_q_heads=32, n_kv_heads=8,
                       head_dim=128, dtype="bf16")
    cache = poisoned_cache(3, 8, 4096, 128, "bf16")
    write_history(cache, wl)
    a = host_raw(run_decode(wl, cache), "bf16")
    b = host_raw(run_decode(wl, cache, write_first=False), "bf16")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_position_next_to_int32_max(dtype):
    d = 128 if dtype == "bf16" else 16
    decode_case(61, [2**31 - 2, 2**31 - 5000], 4096 if dtype == "bf16" else 64, 8, 2, d, dtype)


MASK_POSITIONS = [0, 1, 127, 128, 511, 512, 513, 2047, 4094, 4095, 4096, 9000, 255, 256, 1023, 1024]


def mask_workload(positions, group, seed):
    """Q = 0 and K = 0 give every valid slot the weight 1/|J(pos)|; V of position j is
    one-hot(j mod 64) + one-hot(64 + (j // 64) mod 64), so O * |J(pos)| is the exact
    histogram of the positions the query attended to."""
    hkv = 32 // group
    wl = make_workload("dmask", seed, [(p, 1) for p in positions], window=4096, n_q_heads=32, n_kv_heads=hkv,
                       head_dim=128, dtype="bf16")
    wl.q[:] = 0
    wl.k_new[:] = 0
    wl.v_new = np.concatenate([one_hot_v(1, hkv, 128, "bf16", base=p) for p in positions])
    for b, s in enumerate(wl.seqs):
        wl.hist_k[b][:] = 0
        wl.hist_v[b] = one_hot_v(s.start_pos - s.hist_lo, hkv, 128, "bf16", base=s.hist_lo)
    return wl


def assert_mask_histograms(got, wl, group, what):
    for b, s in enumerate(wl.seqs):
        exp, cnt = expected_hist(s.start_pos, 4096)
        for h in sorted({0, group - 1, group % 32, 31}):
            hist = np.rint(got[b, h].astype(np.float64) * cnt)
            assert np.array_equal(hist, exp), (what, s.start_pos, h)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("batch", [8, 16])
@pytest.mark.parametrize("fused", [False, True])
def test_mask_extraction_at_split_boundaries(group, batch, fused):
    """W = 4096 with 8 or 16 sequences: the plan splits every window (4 to 16 splits),
    and each sequence spreads its valid slots over the splits, so positions next to
    127/128, 511/512, 2047, 4095/4096 put the window edge and the new token's slot
    on split boundaries.  One slot dropped or counted twice changes the histogram."""
    hkv = 32 // group
    assert swa.swa_decode_workspace_size(poisoned_cache(1, hkv, 4096, 128, "bf16"), batch, 32) > 0
    for part in range(0, len(MASK_POSITIONS), batch):
        positions = MASK_POSITIONS[part:part + batch]
        wl = mask_workload(positions, group, seed=900 + part)
        cache = poisoned_cache(batch, hkv, 4096, 128, "bf16")
        write_history(cache, wl)
        t = torch()
        bt = swa.Batch([1] * batch, positions, list(range(batch)))
        q, kn, vn = dev(wl.q, "bf16"), dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
        out = t.full((batch, 32, 128), float("nan"), dtype=t.bfloat16, device="cuda")
        nb = swa.swa_decode_workspace_size(cache, batch, 32)
        ws = t.empty(nb, dtype=t.uint8, device="cuda")
        if fused:
            swa.swa_decode_step(cache, bt, q, 32, kn, vn, wl.scale, out, ws, nb)
        else:
            swa.swa_cache_write(cache, bt, kn, vn)
            swa.swa_decode(cache, bt, q, 32, wl.scale, out, ws, nb)
        assert_mask_histograms(host_f32(out, "bf16"), wl, group, f"G={group} B={batch} fused={fused}")


@pytest.mark.parametrize("group", [1, 4, 8])
def test_workspace_of_the_stated_size_is_enough(group):
    """swa_decode uses no byte past swa_decode_workspace_size(): the bytes after it
    keep a guard pattern, and the result matches the oracle."""
    hkv = 32 // group
    positions = [4100, 77, 20000]
    wl = make_workload("guard", 31 + group, [(p, 1) for p in positions], window=4096, n_q_heads=32,
                       n_kv_heads=hkv, head_dim=128, dtype="bf16")
    cache = poisoned_cache(3, hkv, 4096, 128, "bf16")
    write_history(cache, wl)
    t = torch()
    nb = swa.swa_decode_workspace_size(cache, 3, 32)
    assert nb > 0
    buf = t.full((nb + 4096,), 0xA5, dtype=t.uint8, device="cuda")
    bt = swa.Batch([1] * 3, positions)
    swa.swa_cache_write(cache, bt, dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16"))
    out = t.full((3, 32, 128), float("nan"), dtype=t.bfloat16, device="cuda")
    swa.swa_decode(cache, bt, dev(wl.q, "bf16"), 32, wl.scale, out, buf, nb)
    t.cuda.synchronize()
    assert bool((buf[nb:] == 0xA5).all())
    check_close(host_f32(out, "bf16"), oracle_all(wl), "bf16", f"guarded workspace G={group}")


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_bf16_small_head_dims(d, group):
    """head_dim 16 and 64 run on the matrix-core kernel at every G (G = 1 too)."""
    hkv = 8 if group < 8 else 4
    for window in (100, 4096):
        positions = sorted({0, 1, window - 1, window, window + 1, 3 * window + 5, 20000})
        decode_case(60 + d + group + window, positions, window, hkv * group, hkv, d, "bf16",
                    rows=list(reversed(range(len(positions)))))


@pytest.mark.parametrize("d,window", [(64, 4096), (16, 512)])
@pytest.mark.parametrize("group", [1, 4])
@pytest.mark.parametrize("fused", [False, True])
def test_mask_extraction_small_head_dims(d, window, group, fused):
    """Exact histograms at head_dim 64 and 16 with split plans (8 sequences)."""
    hkv = 32 // group
    positions = [0, 1, 127, 128, window - 2, window - 1, window, 9000]
    wl = make_workload("dmask-d", 950 + d, [(p, 1) for p in positions], window=window, n_q_heads=32,
                       n_kv_heads=hkv, head_dim=d, dtype="bf16")
    wl.q[:] = 0
    wl.k_new[:] = 0
    wl.v_new = np.concatenate([one_hot_v(1, hkv, d, "bf16", base=p) for p in positions])
    for b, s in enumerate(wl.seqs):
        wl.hist_k[b][:] = 0
        wl.hist_v[b] = one_hot_v(s.start_pos - s.hist_lo, hkv, d, "bf16", base=s.hist_lo)
    cache = poisoned_cache(8, hkv, window, d, "bf16")
    write_history(cache, wl)
    t = torch()
    bt = swa.Batch([1] * 8, positions, list(range(8)))
    q, kn, vn = dev(wl.q, "bf16"), dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
    out = t.full((8, 32, d), float("nan"), dtype=t.bfloat16, device="cuda")
    nb = swa.swa_decode_workspace_size(cache, 8, 32)
    assert nb > 0
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    if fused:
        swa.swa_decode_step(cache, bt, q, 32, kn, vn, wl.scale, out, ws, nb)
    else:
        swa.swa_cache_write(cache, bt, kn, vn)
        swa.swa_decode(cache, bt, q, 32, wl.scale, out, ws, nb)
    got = host_f32(out, "bf16")
    for b, p in enumerate(positions):
        exp, cnt = expected_hist(p, window, d)
        for h in sorted({0, group - 1, group % 32, 31}):
            assert np.array_equal(np.rint(got[b, h].astype(np.float64) * cnt), exp), (d, p, h)


def stream_positions(batch, seed):
    """Positions for the stream plan: 0, 1, the window edges and log-uniform contexts up to
    8 windows, in a shuffled order so that short and long pairs alternate in the slot stream."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 4095, 4096, 30000][:batch]
    rest = np.exp(rng.uniform(np.log(2), np.log(32768), batch - len(fixed))).astype(int).tolist()
    pos = fixed + rest
    rng.shuffle(pos)
    return [int(p) for p in pos]


@pytest.mark.parametrize("group,d,batch", [(4, 128, 8), (8, 128, 64), (2, 128, 5), (4, 64, 20), (8, 64, 33),
                                           (2, 64, 2), (1, 64, 7)])
@pytest.mark.parametrize("fused", [False, True])
def test_stream_plan_ragged_contexts(group, d, batch, fused):
    """2 to 64 sequences on the matrix-core kernel: the stream plan cuts the batch's
    valid slots into equal workgroup ranges, which split pairs at arbitrary slots and
    hold several short pairs each.  Output against the oracle; the fused step's cache
    rows bit for bit."""
    hkv = 32 // group
    pos = stream_positions(batch, 600 + 7 * group + d + batch)
    wl = make_workload("stream", 610 + group + d + batch, [(p, 1) for p in pos], window=4096, n_q_heads=32,
                       n_kv_heads=hkv, head_dim=d, dtype="bf16", cache_rows=list(reversed(range(batch))))
    cache = poisoned_cache(batch, hkv, 4096, d, "bf16")
    nb = swa.swa_decode_workspace_size(cache, batch, 32)
    assert nb > 0 and nb % (2 * group * (d + 2) * 4) == 0 and nb // (2 * group * (d + 2) * 4) <= 512
    write_history(cache, wl)
    if fused:
        t = torch()
        out = t.full((batch, 32, d), float("nan"), dtype=t.bfloat16, device="cuda")
        ws = t.empty(nb, dtype=t.uint8, device="cuda")
        kn, vn = dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
        swa.swa_decode_step(cache, swa.Batch([1] * batch, pos, wl.cache_idx), dev(wl.q, "bf16"), 32, kn, vn,
                            wl.scale, out, ws, nb)
        t.cuda.synchronize()
        for b, p in enumerate(pos):
            row = wl.cache_idx[b]
            assert t.equal(cache.k[row, :, p % 4096].view(t.int16), kn[b].view(t.int16)), (b, p)
            assert t.equal(cache.v[row, :, p % 4096].view(t.int16), vn[b].view(t.int16)), (b, p)
    else:
        out = run_decode(wl, cache)
    check_close(host_f32(out, "bf16"), oracle_all(wl), "bf16", f"stream G={group} d={d} B={batch} fused={fused}")


@pytest.mark.parametrize("fused", [False, True])
def test_stream_plan_mask_extraction_at_64_sequences(fused):
    """64 sequences with 4 KV heads (G = 8), the largest stream batch: every slot of every
    window counted exactly once, whatever range boundary or new-token slot it falls on."""
    group, batch = 8, 64
    rng = np.random.default_rng(77)
    positions = MASK_POSITIONS + [int(p) for p in rng.integers(0, 20000, batch - len(MASK_POSITIONS))]
    wl = mask_workload(positions, group, seed=978)
    cache = poisoned_cache(batch, 32 // group, 4096, 128, "bf16")
    nb = swa.swa_decode_workspace_size(cache, batch, 32)
    assert nb > 0 and nb % (2 * group * 130 * 4) == 0
    write_history(cache, wl)
    t = torch()
    bt = swa.Batch([1] * batch, positions, list(range(batch)))
    q, kn, vn = dev(wl.q, "bf16"), dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
    out = t.full((batch, 32, 128), float("nan"), dtype=t.bfloat16, device="cuda")
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    if fused:
        swa.swa_decode_step(cache, bt, q, 32, kn, vn, wl.scale, out, ws, nb)
    else:
        swa.swa_cache_write(cache, bt, kn, vn)
        swa.swa_decode(cache, bt, q, 32, wl.scale, out, ws, nb)
    assert_mask_histograms(host_f32(out, "bf16"), wl, group, f"stream B=64 fused={fused}")


def long_window_cache(positions, window, d=128):
    """Rings of one KV head holding, for each sequence, the window ending at its position:
    K = 0 and V of position j = one-hot(j mod 64) + one-hot(64 + (j // 256) mod 64)."""
    t = torch()
    n = len(positions)
    k = t.zeros((n, 1, window, d), dtype=t.bfloat16, device="cuda")
    v = t.zeros((n, 1, window, d), dtype=t.bfloat16, device="cuda")
    slots = t.arange(window, device="cuda", dtype=t.int64)
    for b, pos in enumerate(positions):
        j = pos - t.remainder(pos - slots, window)          # position held by each slot
        valid = j >= 0
        rows = slots[valid]
        jj = j[valid]
        v[b, 0, rows, jj % 64] = 1.0
        v[b, 0, rows, 64 + (jj // 256) % 64] = 1.0
    return swa.Cache(k, v)


def expected_long_window(pos, window):
    lo = max(0, pos - window + 1)
    j = np.arange(lo, pos + 1)
    o = np.zeros(128)
    np.add.at(o, j % 64, 1.0)
    np.add.at(o, 64 + (j // 256) % 64, 1.0)
    return o / len(j)


@pytest.mark.parametrize("positions", [[256 * 200 - 1], [256 * 300 - 1, 256 * 280 - 1], [30000, 256 * 300 - 1]])
def test_merge_of_more_than_64_partials(positions):
    """W = 32768 with one KV head (G = 2): one sequence takes the split plan with 128 parts;
    two sequences take the stream plan, where each window spans ~128 workgroup ranges (the
    second case starts the second window inside a range).  Both merges then loop over their
    partials in chunks of 64.  Q = K = 0 weighs every key equally, and with windows that end
    at 256k - 1 every bin of the one-hot V holds exactly 512 of the 32768 keys: the output is
    exactly 1/64.  One 256-slot piece dropped or counted twice changes it."""
    t = torch()
    W, hq, d = 32768, 2, 128
    n = len(positions)
    cache = long_window_cache(positions, W, d)
    nb = swa.swa_decode_workspace_size(cache, n, hq)
    if n == 1:
        assert nb == 128 * hq * (d + 2) * 4         # split plan: 128 parts of 256 slots
    else:
        assert nb == 256 * 2 * hq * (d + 2) * 4     # stream plan: 256 workgroups, ranges of 256 slots
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    q = t.zeros((n, hq, d), dtype=t.bfloat16, device="cuda")
    out = t.full((n, hq, d), float("nan"), dtype=t.bfloat16, device="cuda")
    swa.swa_decode(cache, swa.Batch([1] * n, positions, list(range(n))), q, hq, 1.0 / math.sqrt(d), out, ws, nb)
    got = host_f32(out, "bf16")
    for b, pos in enumerate(positions):
        exp = expected_long_window(pos, W)
        for h in range(hq):
            if (pos + 1) % 256 == 0 and pos + 1 >= W:
                assert np.array_equal(got[b, h], exp.astype(np.float32)), (pos, h)
            else:
                assert np.abs(got[b, h] - exp).max() <= 2e-3, (pos, h)
