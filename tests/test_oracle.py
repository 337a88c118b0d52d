"""Pins of the CPU oracle against facts fixed by the paper and by mathematics.

Nothing here touches the GPU path.  Each test names what it pins:
  * brute force with an explicit N x N mask matrix (tiny sizes);
  * W >= N reduces to causal attention (torch's fp64 CPU attention routine);
  * W = 1 gives V exactly; constant V gives that constant (convex combination);
  * mask extraction: Q = 0 and one-hot V expose the exact attended set;
  * chunked prefill through the ring equals unchunked sliding-window attention;
  * ring contents after each write for W = 3 and W = 4 (golden tables);
  * Figure 3 chunk mask (golden); Figure 1 receptive field k (W - 1);
  * the cache stops growing at W slots: 32k positions in a 4096-slot ring is 8x.
Source: Mistral 7B (Chinese translation), section 2 "Architectural details".
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle.brute import band_mask, brute_masked_attention

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=True)


def rnd(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


def full_attend(q, k, v, window, scale):
    n = q.shape[0]
    return oracle.attend(q, np.arange(n), k, v, 0, window, scale)


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("n", [1, 5, 17, 64, 130])
@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("d", [4, 16])
def test_matches_dense_mask_bruteforce(n, group, d):
    rng = np.random.default_rng(1000 + 7 * n + group + d)
    hkv = 2
    hq = hkv * group
    for window in sorted({1, 2, 3, 4, 7, max(1, n - 1), n, n + 3}):
        q, k, v = rnd(rng, (n, hq, d)), rnd(rng, (n, hkv, d)), rnd(rng, (n, hkv, d))
        scale = 1.0 / math.sqrt(d)
        ref = brute_masked_attention(q, k, v, window, scale)
        got = full_attend(q, k, v, window, scale)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_band_mask_counts():
    # every row has exactly min(i + 1, W) keys and always includes itself
    for n, w in [(12, 4), (12, 3), (30, 1), (9, 20)]:
        m = band_mask(n, w)
        assert all(m[i, i] for i in range(n))
        assert list(m.sum(axis=1)) == [min(i + 1, w) for i in range(n)]


# ----------------------------------------------------------------------------- special cases

@pytest.mark.parametrize("group", [1, 4])
def test_window_at_least_length_is_causal_attention(group):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(42 + group)
    n, hkv, d = 48, 2, 16
    hq = hkv * group
    q, k, v = rnd(rng, (n, hq, d)), rnd(rng, (n, hkv, d)), rnd(rng, (n, hkv, d))
    scale = 1.0 / math.sqrt(d)
    tq = torch.from_numpy(q).double().permute(1, 0, 2)                          # [hq, n, d]
    tk = torch.from_numpy(k).double().permute(1, 0, 2).repeat_interleave(group, 0)
    tv = torch.from_numpy(v).double().permute(1, 0, 2).repeat_interleave(group, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    ref = ref.permute(1, 0, 2).numpy()
    for window in (n, n + 1, 4 * n):
        got = full_attend(q, k, v, window, scale)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_one_returns_own_value_exactly():
    rng = np.random.default_rng(7)
    n, hkv, group, d = 33, 2, 4, 16
    q, k, v = rnd(rng, (n, hkv * group, d)), rnd(rng, (n, hkv, d)), rnd(rng, (n, hkv, d))
    got = full_attend(q, k, v, 1, 0.25)
    for h in range(hkv * group):
        assert np.array_equal(got[:, h, :], v[:, h // group, :].astype(np.float64))


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(8)
    n, hkv, group, d = 40, 2, 2, 16
    q, k = rnd(rng, (n, hkv * group, d)) * 3, rnd(rng, (n, hkv, d)) * 3
    c = rnd(rng, (hkv, d))
    v = np.broadcast_to(c, (n, hkv, d)).copy()
    for window in (1, 5, 40):
        got = full_attend(q, k, v, window, 0.3)
        for h in range(hkv * group):
            np.testing.assert_allclose(got[:, h, :], np.broadcast_to(c[h // group], (n, d)), rtol=1e-14, atol=1e-14)


def one_hot_positions(n, hkv, d):
    """V row j = one-hot code of j (dims 0..d/2-1: j mod d/2, rest: (j // (d/2)) mod d/2)."""
    half = d // 2
    v = np.zeros((n, hkv, d), dtype=np.float32)
    for j in range(n):
        v[j, :, j % half] = 1.0
        v[j, :, half + (j // half) % half] = 1.0
    return v


def decode_one_hot(o_row, count, d):
    """Recover the attended positions from O * |J| when they span < (d/2)^2 and are contiguous."""
    half = d // 2
    lo_part = np.rint(o_row[:half] * count).astype(int)
    hi_part = np.rint(o_row[half:] * count).astype(int)
    return lo_part, hi_part


@pytest.mark.parametrize("window", [1, 2, 3, 4, 8, 17])
def test_mask_extraction_exposes_exact_band(window):
    n, hkv, d = 60, 1, 16
    q = np.zeros((n, 2, d), dtype=np.float32)
    k = np.ones((n, hkv, d), dtype=np.float32)
    v = one_hot_positions(n, hkv, d)
    got = full_attend(q, k, v, window, 1.0)
    half = d // 2
    for i in range(n):
        band = list(range(max(0, i - window + 1), i + 1))
        exp_lo = np.zeros(half, int)
        exp_hi = np.zeros(half, int)
        for j in band:
            exp_lo[j % half] += 1
            exp_hi[(j // half) % half] += 1
        lo_part, hi_part = decode_one_hot(got[i, 0], len(band), d)
        assert np.array_equal(lo_part, exp_lo) and np.array_equal(hi_part, exp_hi), (i, window)


def test_mask_extraction_detects_a_planted_off_by_one():
    # the same extraction applied to a deliberately widened window must disagree
    n, d, window = 40, 16, 5
    q = np.zeros((n, 1, d), dtype=np.float32)
    k = np.ones((n, 1, d), dtype=np.float32)
    v = one_hot_positions(n, 1, d)
    good = full_attend(q, k, v, window, 1.0)
    wrong = brute_masked_attention(q, k, v, window + 1, 1.0)
    assert not np.allclose(good[window:], wrong[window:], atol=1e-3)
    np.testing.assert_allclose(good, brute_masked_attention(q, k, v, window, 1.0), atol=1e-12)


def test_missing_history_is_rejected():
    q = np.zeros((1, 1, 4), np.float32)
    k = np.zeros((3, 1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attend(q, np.array([5]), k, k, 3, 4, 1.0)  # needs positions 2..5, has 3..5


# ----------------------------------------------------------------------------- rolling buffer

def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return rows


def ring_positions(window, chunks):
    """Write positions 0..sum(chunks)-1 in the given chunk sizes; return slot->position after each chunk."""
    ring = np.full((1, 1, window, 1), -1, dtype=np.int32)
    states, pos = [], 0
    for c in chunks:
        rows = np.arange(pos, pos + c, dtype=np.int32).reshape(c, 1, 1)
        oracle.ring_write(ring, rows, [0, c], [pos], [0])
        pos += c
        states.append((pos - 1, ring[0, 0, :, 0].copy()))
    return states


@pytest.mark.parametrize("window,name", [(3, "ring_w3.txt"), (4, "ring_w4.txt")])
def test_ring_matches_golden_tables(window, name):
    table = {row[0]: row[1:] for row in read_golden(name)}
    assert len(table) == 12
    for chunks in ([1] * 12, [window] * (12 // window), [5, 7], [12], [2, 9, 1]):
        for e, slots in ring_positions(window, chunks):
            assert list(slots) == table[e], (chunks, e)


def test_ring_batch_with_permuted_rows_matches_golden_table():
    """One batched write of three ragged sequences into permuted cache rows
    (cache_idx = 2, 0, 1), one of them longer than W: every slot of every row
    and head against a table derived by hand from the slot rule (Mistral 7B
    (Chinese translation), section 2, paragraph "Rolling Buffer Cache")."""
    table = {row[0]: row[1:] for row in read_golden("ring_batch_w4.txt")}
    window, hkv, d = 4, 2, 3
    n_tok = 10
    # packed input row t, head g carries (t, g, 7): a misplaced row, head or byte shows
    rows = np.zeros((n_tok, hkv, d), np.int32)
    for t in range(n_tok):
        for g in range(hkv):
            rows[t, g] = (t, g, 7)
    ring = np.full((3, hkv, window, d), -1, np.int32)
    oracle.ring_write(ring, rows, [0, 3, 9, 10], [2, 0, 9], [2, 0, 1])
    for r in range(3):
        for g in range(hkv):
            for slot in range(window):
                t = table[r][slot]
                expect = [-1, -1, -1] if t < 0 else [t, g, 7]
                assert list(ring[r, g, slot]) == expect, (r, g, slot)
    # the same batch without cache_idx writes sequence b into row b
    ring2 = np.full((3, hkv, window, d), -1, np.int32)
    oracle.ring_write(ring2, rows, [0, 3, 9, 10], [2, 0, 9], None)
    for b, r in enumerate([2, 0, 1]):
        assert np.array_equal(ring2[b], ring[r])


def test_chunked_prefill_through_ring_equals_unchunked():
    rng = np.random.default_rng(11)
    n, hkv, group, d = 50, 2, 2, 8
    hq = hkv * group
    q, k, v = rnd(rng, (n, hq, d)), rnd(rng, (n, hkv, d)), rnd(rng, (n, hkv, d))
    scale = 0.37
    for window in (3, 4, 7, 16):
        ref = full_attend(q, k, v, window, scale)
        for chunk in (1, window - 1 if window > 1 else 1, window, window + 2, 13):
            ring_k = np.full((1, hkv, window, d), np.nan, dtype=np.float32)
            ring_v = np.full((1, hkv, window, d), np.nan, dtype=np.float32)
            out = np.empty_like(ref)
            for s in range(0, n, chunk):
                c = min(chunk, n - s)
                lo = max(0, s - window + 1)
                hist = list(range(lo, s))
                # keys of earlier chunks are read back from the ring (slot j mod W)
                hk = np.stack([ring_k[0, :, j % window, :] for j in hist]) if hist else np.zeros((0, hkv, d), np.float32)
                hv = np.stack([ring_v[0, :, j % window, :] for j in hist]) if hist else np.zeros((0, hkv, d), np.float32)
                kk = np.concatenate([hk, k[s:s + c]])
                vv = np.concatenate([hv, v[s:s + c]])
                out[s:s + c] = oracle.attend(q[s:s + c], np.arange(s, s + c), kk, vv, lo, window, scale)
                # attend first, then write the chunk into the ring
                oracle.ring_write(ring_k, k[s:s + c], [0, c], [s], [0])
                oracle.ring_write(ring_v, v[s:s + c], [0, c], [s], [0])
            np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_fig3_third_chunk_mask():
    table = {row[0]: row[1:] for row in read_golden("fig3_chunk3.txt")}
    n, window, chunk, d = 12, 4, 4, 16
    q = np.zeros((n, 1, d), np.float32)
    k = np.ones((n, 1, d), np.float32)
    v = np.zeros((n, 1, d), np.float32)
    v[np.arange(n), 0, np.arange(n)] = 1.0  # n <= d: plain one-hot of the position
    ring_k = np.full((1, 1, window, d), np.nan, np.float32)
    ring_v = np.full((1, 1, window, d), np.nan, np.float32)
    for s in range(0, n, chunk):
        lo = max(0, s - window + 1)
        hk = np.stack([ring_k[0, :, j % window] for j in range(lo, s)]) if s else np.zeros((0, 1, d), np.float32)
        hv = np.stack([ring_v[0, :, j % window] for j in range(lo, s)]) if s else np.zeros((0, 1, d), np.float32)
        out = oracle.attend(q[s:s + chunk], np.arange(s, s + chunk), np.concatenate([hk, k[s:s + chunk]]),
                            np.concatenate([hv, v[s:s + chunk]]), lo, window, 1.0)
        oracle.ring_write(ring_k, k[s:s + chunk], [0, chunk], [s], [0])
        oracle.ring_write(ring_v, v[s:s + chunk], [0, chunk], [s], [0])
    # third chunk: positions 8..11
    for r, i in enumerate(range(8, 12)):
        expect = table[i]
        got = out[r, 0] * len(expect)
        np.testing.assert_allclose(got[n:], 0.0, atol=1e-12)
        attended = [j for j in range(n) if abs(got[j] - 1.0) < 1e-12]
        assert attended == expect
        assert all(abs(got[j]) < 1e-12 for j in range(n) if j not in expect)
        assert not any(j <= 4 for j in attended)


def test_receptive_field_grows_by_window_minus_one_per_layer():
    """Figure 1: stacking k SWA layers lets position i see inputs i-k(W-1) .. i."""
    rng = np.random.default_rng(3)
    n, dm, window = 28, 8, 3
    # small query/key projections keep the softmax smooth, so that every path of
    # influence stays far above float32 resolution
    layers = [(0.1 * rng.standard_normal((dm, dm)), 0.1 * rng.standard_normal((dm, dm)),
               rng.standard_normal((dm, dm)) / math.sqrt(dm)) for _ in range(4)]

    def run(x):
        outs = []
        for wq, wk, wv in layers:
            qh = (x @ wq).astype(np.float32)[:, None, :]
            kh = (x @ wk).astype(np.float32)[:, None, :]
            vh = (x @ wv).astype(np.float32)[:, None, :]
            x = x + oracle.attend(qh, np.arange(n), kh, vh, 0, window, 1.0)[:, 0, :]
            outs.append(x)
        return outs

    x0 = rng.standard_normal((n, dm))
    base = run(x0)
    for j in (0, 5, 13):
        x1 = x0.copy()
        x1[j] += 0.5
        pert = run(x1)
        for depth, (a, b) in enumerate(zip(base, pert), start=1):
            changed = {i for i in range(n) if np.abs(a[i] - b[i]).max() > 1e-6}
            expect = {i for i in range(n) if 0 <= i - j <= depth * (window - 1)}
            assert changed == expect, (j, depth)


def test_cache_memory_stops_at_window():
    """32k positions through a W = 4096 ring: the ring keeps the last 4096 positions
    and uses 1/8 of the memory a full 32k cache needs."""
    window, n = 4096, 32768
    ring = np.full((1, 1, window, 1), -1, dtype=np.int32)
    rows = np.arange(n, dtype=np.int32).reshape(n, 1, 1)
    for s in range(0, n, 4096):
        oracle.ring_write(ring, rows[s:s + 4096], [0, 4096], [s], [0])
    held = np.sort(ring[0, 0, :, 0])
    assert np.array_equal(held, np.arange(n - window, n))
    full_bytes = rows.nbytes
    assert full_bytes // ring.nbytes == 8
    # theoretical attention span of the last layer for 32 layers (the paper's ~131K)
    assert 32 * window == 131072
    assert 32 * (window - 1) == 131040


def test_thread_count_does_not_change_results():
    """The oracle computes each (query, head) in one thread, in a fixed order: its
    results are bitwise the same at any thread count (the CPU baseline is timed at
    several)."""
    rng = np.random.default_rng(21)
    q, k, v = rnd(rng, (40, 4, 16)), rnd(rng, (40, 2, 16)), rnd(rng, (40, 2, 16))
    oracle.set_num_threads(1)
    a = oracle.attend(q, np.arange(40), k, v, 0, 9, 0.3)
    oracle.set_num_threads(max(2, os.cpu_count() or 2))
    b = oracle.attend(q, np.arange(40), k, v, 0, 9, 0.3)
    assert np.array_equal(a, b)
