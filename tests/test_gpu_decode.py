"""GPU parity of swa_decode against the fp64 oracle.

Mistral 7B (Chinese translation), section 2: after the prompt, tokens are
generated one at a time (paragraph "Pre-fill and Chunking"); each reads the W
most recent positions from the rolling buffer (paragraphs "Sliding Window
Attention", "Rolling Buffer Cache").  The new token is written first.
"""
import numpy as np
import pytest

import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import batched_decode, make_workload
from helpers import check_close, host_f32, host_raw, oracle_all, poisoned_cache, run_decode, write_history

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
