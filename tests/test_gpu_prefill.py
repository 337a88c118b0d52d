"""GPU parity of swa_prefill_chunk against the fp64 oracle.

Mistral 7B (Chinese translation), section 2: paragraphs "Sliding Window
Attention", "Rolling Buffer Cache", "Pre-fill and Chunking" and Figures 1-3;
section 1 for grouped-query attention.  Tolerances: max-abs 2e-2 (bf16), 1e-4
(fp32); structural cases (W = 1, mask extraction) are exact.
"""
import math

import numpy as np
import pytest

import oracle
import sliding_window_gqa_swa_amd as swa
from oracle.brute import brute_masked_attention
from sliding_window_gqa_swa_amd.workloads import make_workload, tiny_prefill, to_f32
from helpers import (check_close, dev, empty, expected_hist, host_f32, host_raw, new_batch, one_hot_v, oracle_all,
                     poisoned_cache, run_prefill, torch, write_history)

pytestmark = pytest.mark.gpu


def prefill_case(seed, seqs, window, hq, hkv, d, dtype, n_cache=None):
    wl = make_workload("case", seed, seqs, window=window, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, dtype=dtype,
                       n_cache=n_cache)
    cache = poisoned_cache(wl.n_cache, hkv, window, d, dtype)
    write_history(cache, wl)
    out = run_prefill(wl, cache)
    got = host_f32(out, dtype)
    ref = oracle_all(wl)
    return check_close(got, ref, dtype, f"seed={seed} W={window} seqs={seqs}")


def test_tiny_config_fp32_against_bruteforce():
    wl = tiny_prefill(1001)
    cache = poisoned_cache(1, 2, 8, 16, "f32")
    out = run_prefill(wl, cache)
    got = host_f32(out, "f32")
    ref = brute_masked_attention(to_f32(wl.q, "f32"), to_f32(wl.k_new, "f32"), to_f32(wl.v_new, "f32"), 8, 0.25)
    assert np.abs(got - ref).max() <= 1e-4
    check_close(got, oracle_all(wl), "f32", "tiny")


@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 777])
@pytest.mark.parametrize("window", [1, 3, 64, 100, 129, 1000])
def test_bf16_single_sequence_from_start(n, window):
    prefill_case(10 * n + window, [(0, n)], window, 32, 8, 128, "bf16")


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_bf16_groups_with_history(group):
    hkv = 16 // group if group < 8 else 2
    prefill_case(500 + group, [(300, 200), (5, 70), (1000, 1)], 256, hkv * group, hkv, 128, "bf16")


@pytest.mark.parametrize("d", [16, 64, 128])
def test_fp32_with_history(d):
    prefill_case(600 + d, [(40, 77), (0, 30), (150, 3)], 50, 8, 2, d, "f32")


def test_bf16_partial_caches_are_never_read_past_their_history():
    # histories shorter than W: the never-written slots hold NaN and must stay unread
    prefill_case(77, [(10, 300), (1, 1), (200, 130), (0, 64)], 512, 32, 8, 128, "bf16")


def test_bf16_chunk_longer_than_window():
    prefill_case(78, [(0, 700), (900, 333)], 100, 32, 8, 128, "bf16")


def test_bf16_window_at_least_length_is_causal():
    # W >= N: the oracle is causal attention; run the same inputs at two windows
    a = prefill_case(79, [(0, 500)], 500, 32, 8, 128, "bf16")
    b = prefill_case(79, [(0, 500)], 4096, 32, 8, 128, "bf16")
    assert a <= 2e-2 and b <= 2e-2


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("bf16", 16), ("f32", 16)])
def test_window_one_is_exact(dtype, d):
    wl = make_workload("w1", 9, [(0, 150), (37, 20)], window=1, n_q_heads=8, n_kv_heads=2, head_dim=d, dtype=dtype)
    cache = poisoned_cache(2, 2, 1, d, dtype)
    write_history(cache, wl)
    got = host_raw(run_prefill(wl, cache), dtype)
    for h in range(8):
        assert np.array_equal(got[:, h, :], wl.v_new[:, h // 4, :])


def mask_extraction(window, group, d, cases):
    """Q = 0 makes every weight 1/|J(i)|; one-hot V turns O * |J(i)| into the exact
    histogram of the attended positions, so any off-by-one at the window edge or the
    diagonal shows, also through the ring (history) and the chunk boundary."""
    hkv = 2
    hq = hkv * group
    for start, n_new in cases:
        hist_lo = max(0, start - window + 1)
        wl = make_workload("mask", 1, [(start, n_new)], window=window, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                           dtype="bf16")
        wl.q[:] = 0
        wl.k_new[:] = 0
        wl.hist_k[0][:] = 0
        wl.v_new = one_hot_v(n_new, hkv, d, "bf16", base=start)
        wl.hist_v[0] = one_hot_v(start - hist_lo, hkv, d, "bf16", base=hist_lo)
        cache = poisoned_cache(1, hkv, window, d, "bf16")
        write_history(cache, wl)
        got = host_f32(run_prefill(wl, cache), "bf16")
        for r in range(n_new):
            exp, cnt = expected_hist(start + r, window, d)
            for h in sorted({0, group - 1, group % hq, hq - 1}):
                hist = np.rint(got[r, h].astype(np.float64) * cnt)
                assert np.array_equal(hist, exp), (d, window, start, r, h)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("window", [1, 2, 3, 4, 8, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 4096])
def test_mask_extraction_bf16(window, group):
    """Every compiled group size: a workgroup spans 256 / G query positions, so the
    band loop bounds differ per G."""
    mask_extraction(window, group, 128, [(0, 300), (200, 190), (5000, 70), (4000, 600)])


SMALL_D_WINDOWS = [(d, w) for d in (16, 64) for w in (1, 3, 17, 64, 65, 129, 256, 512, 4096)
                   if not (d == 16 and w > 512)]


@pytest.mark.parametrize("group", [1, 4, 8])
@pytest.mark.parametrize("d,window", SMALL_D_WINDOWS)
def test_mask_extraction_bf16_small_head_dims(d, window, group):
    """head_dim 64 (32-position codes) and 16 (8-position codes; their counts reach
    W / 8, and a bf16 output resolves them exactly only up to W = 512)."""
    mask_extraction(window, group, d, [(0, 300), (200, 190), (5000, 70), (4000, 300)])


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_bf16_small_head_dims_with_history(d, group):
    hkv = 16 // group if group < 8 else 2
    for window in (37, 256):
        prefill_case(700 + d + group + window, [(300, 200), (5, 70), (1000, 1), (0, 129)], window, hkv * group, hkv,
                     d, "bf16")


@pytest.mark.parametrize("d", [16, 64])
def test_bf16_small_head_dims_long_chunk_through_ring(d):
    """A 2000-token chunk after 3000 positions of history at W = 1024, 32 q / 8 kv heads."""
    prefill_case(800 + d, [(3000, 2000), (0, 700)], 1024, 32, 8, d, "bf16")


def test_figure3_chunks_through_the_ring():
    """Three chunks of four tokens with W = 4: the third chunk (positions 8..11)
    attends {5-8}, {6-9}, {7-10}, {8-11} and never positions 0..4."""
    hkv, d, window = 1, 128, 4
    cache = poisoned_cache(1, hkv, window, d, "bf16")
    table = {8: [5, 6, 7, 8], 9: [6, 7, 8, 9], 10: [7, 8, 9, 10], 11: [8, 9, 10, 11]}
    for s in (0, 4, 8):
        batch = swa.Batch([4], [s], [0])
        q = dev(np.zeros((4, 4, d), np.uint16), "bf16")
        kn = dev(np.zeros((4, hkv, d), np.uint16), "bf16")
        vn = dev(one_hot_v(4, hkv, d, "bf16", base=s), "bf16")
        out = empty((4, 4, d), "bf16")
        swa.swa_prefill_chunk(cache, batch, q, 4, kn, vn, 1 / math.sqrt(d), out)
        swa.swa_cache_write(cache, batch, kn, vn)
    got = host_f32(out, "bf16")
    for r, i in enumerate(range(8, 12)):
        attended = [j for j in range(12) if round(float(got[r, 0, j]) * 4) == 1]
        assert attended == table[i]


@pytest.mark.parametrize("chunk", [64, 128, 256, 512])
def test_chunked_through_ring_equals_unchunked(chunk):
    """Chunked prefill through the rolling buffer reproduces unchunked SWA, for
    chunks of W/4, W/2, W and 2W (the pages advise chunk = window; a chunk
    longer than W also applies the window inside itself, and its cache write
    keeps only the last W tokens)."""
    rng_seed, n, window = 31, 1200, 256
    hq, hkv, d = 32, 8, 128
    full = make_workload("full", rng_seed, [(0, n), (0, n)], window=window, n_q_heads=hq, n_kv_heads=hkv,
                         head_dim=d, dtype="bf16")
    ref = oracle_all(full)
    cache = poisoned_cache(2, hkv, window, d, "bf16")
    q, kn, vn = dev(full.q, "bf16"), dev(full.k_new, "bf16"), dev(full.v_new, "bf16")
    out = empty((2 * n, hq, d), "bf16")
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        idx = torch().cat([torch().arange(s, s + c), torch().arange(n + s, n + s + c)]).cuda()
        batch = swa.Batch([c, c], [s, s], [0, 1])
        qo = empty((2 * c, hq, d), "bf16")
        kc, vc = kn[idx].contiguous(), vn[idx].contiguous()
        swa.swa_prefill_chunk(cache, batch, q[idx].contiguous(), hq, kc, vc, full.scale, qo)
        swa.swa_cache_write(cache, batch, kc, vc)
        out[idx] = qo
    check_close(host_f32(out, "bf16"), ref, "bf16", f"chunked ({chunk}) vs unchunked")


def test_deterministic_bitwise():
    wl = make_workload("det", 12, [(100, 500), (0, 64)], window=300, n_q_heads=32, n_kv_heads=8, head_dim=128,
                       dtype="bf16")
    cache = poisoned_cache(2, 8, 300, 128, "bf16")
    write_history(cache, wl)
    a = host_raw(run_prefill(wl, cache), "bf16")
    b = host_raw(run_prefill(wl, cache), "bf16")
    assert np.array_equal(a, b)


def test_cache_is_not_written_by_prefill():
    wl = make_workload("ro", 13, [(50, 100)], window=128, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16")
    cache = poisoned_cache(1, 8, 128, 128, "bf16")
    write_history(cache, wl)
    before = host_raw(cache.k, "bf16").copy(), host_raw(cache.v, "bf16").copy()
    run_prefill(wl, cache)
    torch().cuda.synchronize()
    assert np.array_equal(host_raw(cache.k, "bf16").view(np.uint8), before[0].view(np.uint8))
    assert np.array_equal(host_raw(cache.v, "bf16").view(np.uint8), before[1].view(np.uint8))


def test_no_cache_pointers_when_every_sequence_starts_at_zero():
    wl = make_workload("nocache", 14, [(0, 90), (0, 17)], window=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                       dtype="bf16")
    c = swa.cache_struct(None, None, 2, 8, 128, 64, swa.SWA_DTYPE_BF16)
    q, kn, vn = dev(wl.q, "bf16"), dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
    out = empty((wl.total_tokens, 32, 128), "bf16")
    swa.swa_prefill_chunk(c, new_batch(wl), q, 32, kn, vn, wl.scale, out)
    check_close(host_f32(out, "bf16"), oracle_all(wl), "bf16", "no cache")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_positions_next_to_int32_max(dtype):
    # the last position of the chunk is 2^31 - 2: every position sum stays in range
    d = 128 if dtype == "bf16" else 64
    top = 2**31 - 1
    prefill_case(91, [(top - 301, 300), (top - 70, 69)], 100, 8, 2, d, dtype)


def test_empty_sequence_inside_a_batch():
    prefill_case(92, [(0, 130), (40, 0), (500, 77), (3, 0)], 64, 32, 8, 128, "bf16")


@pytest.mark.parametrize("group,d", [(4, 128), (1, 128), (8, 128), (4, 64), (2, 16)])
def test_no_tile_skip_variant_is_bitwise_identical(group, d):
    """swa_prefill_chunk_no_tile_skip visits every key tile from position 0 and
    masks the keys outside the window; the extra keys get weight exactly 0, so
    the output equals swa_prefill_chunk bit for bit (and matches the oracle)."""
    hkv = 2
    wl = make_workload("noskip", 40 + group + d, [(0, 1500), (3000, 700), (100, 33)], window=256,
                       n_q_heads=hkv * group, n_kv_heads=hkv, head_dim=d, dtype="bf16")
    cache = poisoned_cache(wl.n_cache, hkv, 256, d, "bf16")
    write_history(cache, wl)
    ref = run_prefill(wl, cache)
    q, kn, vn = dev(wl.q, "bf16"), dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
    out = empty((wl.total_tokens, wl.n_q_heads, d), "bf16")
    out.fill_(float("nan"))
    swa.swa_prefill_chunk_no_tile_skip(cache, new_batch(wl), q, wl.n_q_heads, kn, vn, wl.scale, out)
    t = torch()
    t.cuda.synchronize()
    assert t.equal(out.view(t.int16), ref.view(t.int16))
    check_close(host_f32(out, "bf16"), oracle_all(wl), "bf16", "no tile skip")
