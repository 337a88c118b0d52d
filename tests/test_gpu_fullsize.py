"""Full-size GPU parity on the benchmark workloads, in the launch configuration
bench.py times, against the fp64 oracle on sampled output rows.

Sampled rows always include the first and last rows of the sequence, the rows
around every window edge and chunk boundary, plus seeded random rows.
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


def sample_rows(n, rng, boundaries=(), n_random=192, halo=3):
    rows = set(range(min(halo, n))) | set(range(max(0, n - halo), n))
    for bnd in boundaries:
        rows |= {r for r in range(bnd - halo, bnd + halo) if 0 <= r < n}
    rows |= set(rng.integers(0, n, size=min(n, n_random)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("window", [4096, 16384])
def test_mistral_prefill_16k(window):
    wl = mistral_prefill(1002, window=window)
    cache = poisoned_cache(1, 8, window, 128, "bf16")
    got = host_f32(run_prefill(wl, cache), "bf16")
    rng = np.random.default_rng(window)
    rows = sample_rows(16384, rng, boundaries=[window, 4096, 8192])
    ref = oracle_seq(wl, 0, rows)
    check_close(got[rows], ref, "bf16", f"16K prefill W={window}")


def test_chunked_prefill_4x32k_through_the_ring():
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
        rows = sample_rows(N, rng, boundaries=list(range(C, N, C)), n_random=96)
        got = host_f32(out[b][t.from_numpy(rows).cuda()], "bf16")
        ref = oracle.attend(to_f32(q[b, rows], "bf16"), rows, to_f32(k[b], "bf16"), to_f32(v[b], "bf16"), 0, W,
                            1 / np.sqrt(128))
        check_close(got, ref, "bf16", f"chunked seq {b}")
    # the ring holds exactly the last W positions of every sequence, bit for bit
    ring_k = cache.k.view(t.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        expect = k[b, N - W:]                       # positions N-W .. N-1
        slots = np.arange(N - W, N) % W
        assert np.array_equal(ring_k[b][:, slots, :], expect.transpose(1, 0, 2))


@pytest.mark.parametrize("variant", [False, True])
def test_ragged_mixed_batch(variant):
    wp, wd = ragged_mixed(1005, variant=variant)
    cache = poisoned_cache(48, 8, 4096, 128, "bf16")
    write_history(cache, wp)
    write_history(cache, wd)
    gp = host_f32(run_prefill(wp, cache), "bf16")
    rng = np.random.default_rng(11 + variant)
    for b, s in enumerate(wp.seqs):
        rows = sample_rows(s.n_new, rng, boundaries=[64, 256], n_random=48)
        sl = wp.seq_tokens(b)
        check_close(gp[sl][rows], oracle_seq(wp, b, rows), "bf16", f"mixed prefill seq {b} (L={s.start_pos + s.n_new})")
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
