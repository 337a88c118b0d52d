"""GPU parity of swa_cache_write against the oracle's ring simulator: bit-exact.

Mistral 7B (Chinese translation), section 2, paragraph "Rolling Buffer Cache"
and Figure 2: position i goes to slot i mod W; later positions overwrite.
"""
import numpy as np
import pytest

import oracle
import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import randn
from helpers import dev, host_raw, poisoned_cache

pytestmark = pytest.mark.gpu


def gpu_vs_oracle_ring(seed, window, n_cache, hkv, d, dtype, calls):
    """calls: list of (lengths, start_pos, cache_idx) applied in order."""
    rng = np.random.default_rng(seed)
    cache = poisoned_cache(n_cache, hkv, window, d, dtype)
    ring_k = host_raw(cache.k, dtype).copy()
    ring_v = host_raw(cache.v, dtype).copy()
    for lens, starts, rows in calls:
        total = int(sum(lens))
        kn = randn(rng, (total, hkv, d), dtype)
        vn = randn(rng, (total, hkv, d), dtype)
        batch = swa.Batch(lens, starts, rows)
        swa.swa_cache_write(cache, batch, dev(kn, dtype), dev(vn, dtype))
        cu = np.concatenate([[0], np.cumsum(lens)])
        oracle.ring_write(ring_k, kn, cu, starts, rows)
        oracle.ring_write(ring_v, vn, cu, starts, rows)
    gk, gv = host_raw(cache.k, dtype), host_raw(cache.v, dtype)
    assert np.array_equal(gk.view(np.uint8), ring_k.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), ring_v.view(np.uint8))


@pytest.mark.parametrize("window", [3, 4])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 16)])
def test_ring_illustration_one_by_one_and_in_chunks(window, dtype, d):
    # positions 0..11 written one at a time, then in chunks of W, then all at once
    one = [([1], [p], [0]) for p in range(12)]
    chunks = [([window], [p], [0]) for p in range(0, 12, window)]
    whole = [([12], [0], [0])]
    for calls in (one, chunks, whole):
        gpu_vs_oracle_ring(100 + window, window, 1, 2, d, dtype, calls)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 128), ("f32", 16)])
def test_ragged_batch_with_cache_rows_and_long_chunks(dtype, d):
    # chunk longer than W (only the last W land), ragged lengths, permuted rows,
    # an empty sequence, starts inside and past the first lap of the ring
    window = 37
    calls = [([5, 100, 0, 37, 38], [0, 11, 4, 70, 1000], [3, 0, 4, 1, 2]),
             ([1, 1, 1, 1, 1], [5, 111, 4, 107, 1038], [3, 0, 4, 1, 2])]
    gpu_vs_oracle_ring(7, window, 6, 3, d, dtype, calls)


def test_decode_shaped_write_full_size():
    # 64 sequences, one token each, into a W = 4096 cache with 8 KV heads
    rng = np.random.default_rng(1004)
    pos = rng.integers(4096, 32768, size=64)
    gpu_vs_oracle_ring(1004, 4096, 64, 8, 128, "bf16", [([1] * 64, list(pos), list(range(64)))])


def test_chunk_shaped_write_full_size():
    # 4 sequences x 4096-token chunk at position 8192, W = 4096
    gpu_vs_oracle_ring(1003, 4096, 4, 8, 128, "bf16", [([4096] * 4, [8192] * 4, [0, 1, 2, 3])])


def test_window_one_keeps_only_last():
    gpu_vs_oracle_ring(5, 1, 2, 1, 128, "bf16", [([9, 3], [0, 4], [1, 0])])
