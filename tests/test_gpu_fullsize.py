"""Full-size GPU parity on the benchmark workloads, in the launch configuration
bench.py times, against the fp64 oracle.

The 16K-token prefill at W = 4096 is compared on every output row and head.
Elsewhere the compared rows are every row of the query tiles at the start and
end of each sequence and on both sides of every chunk boundary and window
edge, plus seeded random rows (4096 per sequence where the oracle time allows).
Mistral 7B (Chinese translation), section 2 ("Sliding Window Attention",
"Rolling Buffer Cache", "Pre-fill and Chunking").
"""
import numpy as np
import pytest

import oracle
import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import (batched_decode, chunked_sequences, mistral_prefill, ragged_mixed,
                                                  to_f32)
from helpers import (check_close, dev, empty, host_f32, new_batch, oracle_all, oracle_seq, poisoned_cache,
                     run_decode, run_prefill, torch, write_history)

pytestmark = pytest.mark.gpu

TILE = 64  # query positions of one workgroup at G = 4 (the widest at G = 1 is 256)


def edge_tile_rows(n, boundaries, width=256):
    """Every row within `width` positions of the sequence ends and of each boundary."""
    rows = set(range(min(width, n))) | set(range(max(0, n - width), n))
    for bnd in boundaries:
        rows |= {r for r in range(bnd - width, bnd + width) if 0 <= r < n}
    return rows


def sample_rows(n, rng, boundaries=(), n_random=4096, width=256):
    rows = edge_tile_rows(n, boundaries, width)
    rows |= set(rng.choice(n, size=min(n, n_random), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def test_mistral_prefill_16k_w4096_every_row():
    """The benchmark prefill (1 x 16384 tokens, 32 q / 8 kv heads, W = 4096): all
    16384 x 32 output rows against the oracle."""
    wl = mistral_prefill(1002, window=4096)
    cache = poisoned_cache(1, 8, 4096, 128, "bf16")
    got = host_f32(run_prefill(wl, cache), "bf16")
    ref = oracle_all(wl)
    check_close(got, ref, "bf16", "16K prefill W=4096, all rows")


def test_mistral_prefill_16k_causal():
    """W = 16384 >= N: causal attention.  Every row of the first and last query
    tiles and around positions 4096 / 8192, plus 4096 seeded random rows."""
    wl = mistral_prefill(1002, window=16384)
    cache = poisoned_cache(1, 8, 16384, 128, "bf16")
    got = host_f32(run_prefill(wl, cache), "bf16")
    rows = sample_rows(16384, np.random.default_rng(16384), boundaries=[4096, 8192])
    check_close(got[rows], oracle_seq(wl, 0, rows), "bf16", "16K prefill W=16384")


def test_chunked_prefill_4x32k_through_the_ring():
    """4 sequences x 32768 tokens in 8 chunks of 4096 through a 4096-slot ring.
    Sequence 0: every row within 256 positions of each chunk boundary and of its
    ends, plus 4096 random rows; sequences 1-3: the boundary rows and 256 random."""
    B, N, C, W = 4, 32768, 4096, 4096
    q, k, v = chunked_sequences(1003, batch=B, n=N, window=W)
    t = torch()
    cache = poisoned_cache(B, 8, W, 128, "bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")  # [B, N, H, D]
    out = empty((B, N, 32, 128), "bf16")
    for s in range(0, N, C):
        batch = swa.Batch([C] * B, [s] * B, list(range(B)))
        qc = qd[:, s:s + C].reshape(B * C, 32, 128).contiguous()
        kc = kd[:, s:s + C].reshape(B * C, 8, 128).contiguous()
        vc = vd[:, s:s + C].reshape(B * C, 8, 128).contiguous()
        oc = empty((B * C, 32, 128), "bf16")
        swa.swa_prefill_chunk(cache, batch, qc, 32, kc, vc, 1 / np.sqrt(128), oc)
        swa.swa_cache_write(cache, batch, kc, vc)
        out[:, s:s + C] = oc.view(B, C, 32, 128)
    t.cuda.synchronize()
    rng = np.random.default_rng(7)
    for b in range(B):
        rows = sample_rows(N, rng, boundaries=list(range(C, N, C)), n_random=4096 if b == 0 else 256,
                           width=TILE if b else 256)
        got = host_f32(out[b][t.from_numpy(rows).cuda()], "bf16")
        ref = oracle.attend(to_f32(q[b, rows], "bf16"), rows, to_f32(k[b], "bf16"), to_f32(v[b], "bf16"), 0, W,
                            1 / np.sqrt(128))
        check_close(got, ref, "bf16", f"chunked seq {b} ({len(rows)} rows)")
    # the ring holds exactly the last W positions of every sequence, bit for bit
    ring_k = cache.k.view(t.int16).cpu().numpy().view(np.uint16)
    ring_v = cache.v.view(t.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        slots = np.arange(N - W, N) % W
        assert np.array_equal(ring_k[b][:, slots, :], k[b, N - W:].transpose(1, 0, 2))
        assert np.array_equal(ring_v[b][:, slots, :], v[b, N - W:].transpose(1, 0, 2))


@pytest.mark.parametrize("variant", [False, True])
def test_ragged_mixed_batch(variant):
    """16 prefill + 32 decode sequences in one 48-row cache (rows permuted).
    Prefill: the first and last 256 rows of every sequence, the rows around
    positions where the window starts to slide, plus 512 random rows each."""
    wp, wd = ragged_mixed(1005, variant=variant)
    cache = poisoned_cache(48, 8, 4096, 128, "bf16")
    write_history(cache, wp)
    write_history(cache, wd)
    gp = host_f32(run_prefill(wp, cache), "bf16")
    rng = np.random.default_rng(11 + variant)
    for b, s in enumerate(wp.seqs):
        # relative row where the query position crosses W (the window starts sliding)
        edge = [4096 - s.start_pos] if 0 < 4096 - s.start_pos < s.n_new else []
        rows = sample_rows(s.n_new, rng, boundaries=edge, n_random=512)
        sl = wp.seq_tokens(b)
        check_close(gp[sl][rows], oracle_seq(wp, b, rows), "bf16",
                    f"mixed prefill seq {b} (L={s.start_pos + s.n_new})")
    gd = host_f32(run_decode(wd, cache), "bf16")
    check_close(gd, oracle_all(wd), "bf16", "mixed decode")


def test_batched_decode_full_size_bitwise_repeatable():
    wl = batched_decode(1004)
    cache = poisoned_cache(64, 8, 4096, 128, "bf16")
    write_history(cache, wl)
    a = run_decode(wl, cache)
    b = run_decode(wl, cache, write_first=False)
    torch().cuda.synchronize()
    assert torch().equal(a.view(torch().int16), b.view(torch().int16))
