"""Helpers for the GPU parity tests: upload/download of raw inputs, cache set-up
through the library's own cache write, and oracle references for a workload."""
from __future__ import annotations

import numpy as np

import oracle
import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import Workload, bf16_bits_from_f32, to_f32

BF16_NAN = 0x7FC0
TOL = {"bf16": 2e-2, "f32": 1e-4}   # max-abs error bars for attention outputs
REL_RMS_BF16 = 1e-2                  # regression guard on top of the max-abs bar


def torch():
    import torch as t
    return t


def dev(raw: np.ndarray, dtype: str):
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(t.bfloat16).to("cuda")
    return t.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to("cuda")


def host_raw(x, dtype: str) -> np.ndarray:
    t = torch()
    if dtype == "bf16":
        return x.detach().view(t.int16).cpu().numpy().view(np.uint16)
    return x.detach().cpu().numpy()


def host_f32(x, dtype: str) -> np.ndarray:
    return to_f32(host_raw(x, dtype), dtype)


def empty(shape, dtype: str):
    t = torch()
    return t.empty(shape, dtype=t.bfloat16 if dtype == "bf16" else t.float32, device="cuda")


def poisoned_cache(n_cache, hkv, window, d, dtype):
    """Cache tensors whose every slot starts as NaN: a stray read shows up as NaN."""
    t = torch()
    if dtype == "bf16":
        k = t.full((n_cache, hkv, window, d), BF16_NAN, dtype=t.int16, device="cuda").view(t.bfloat16)
        v = t.full((n_cache, hkv, window, d), BF16_NAN, dtype=t.int16, device="cuda").view(t.bfloat16)
    else:
        k = t.full((n_cache, hkv, window, d), float("nan"), dtype=t.float32, device="cuda")
        v = t.full((n_cache, hkv, window, d), float("nan"), dtype=t.float32, device="cuda")
    return swa.Cache(k, v)


def write_history(cache: swa.Cache, wl: Workload):
    """Write every sequence's history (positions hist_lo .. start-1) with swa_cache_write."""
    lens = [s.start_pos - s.hist_lo for s in wl.seqs]
    if sum(lens) == 0:
        return
    batch = swa.Batch(lens, [s.hist_lo for s in wl.seqs], wl.cache_idx)
    swa.swa_cache_write(cache, batch, dev(wl.hist_packed("k"), wl.dtype), dev(wl.hist_packed("v"), wl.dtype))


def new_batch(wl: Workload, mirrors=True) -> swa.Batch:
    return swa.Batch([s.n_new for s in wl.seqs], [s.start_pos for s in wl.seqs], wl.cache_idx, mirrors=mirrors)


def run_prefill(wl: Workload, cache: swa.Cache, batch=None):
    q, kn, vn = dev(wl.q, wl.dtype), dev(wl.k_new, wl.dtype), dev(wl.v_new, wl.dtype)
    out = empty((wl.total_tokens, wl.n_q_heads, wl.head_dim), wl.dtype)
    out.fill_(float("nan"))
    swa.swa_prefill_chunk(cache, batch or new_batch(wl), q, wl.n_q_heads, kn, vn, wl.scale, out)
    return out


def run_decode(wl: Workload, cache: swa.Cache, write_first=True):
    batch = new_batch(wl)
    if write_first:
        swa.swa_cache_write(cache, batch, dev(wl.k_new, wl.dtype), dev(wl.v_new, wl.dtype))
    q = dev(wl.q, wl.dtype)
    out = empty((wl.num_seqs, wl.n_q_heads, wl.head_dim), wl.dtype)
    out.fill_(float("nan"))
    ws_bytes = swa.swa_decode_workspace_size(cache, wl.num_seqs, wl.n_q_heads)
    ws = torch().empty(max(ws_bytes, 16), dtype=torch().uint8, device="cuda")
    swa.swa_decode(cache, batch, q, wl.n_q_heads, wl.scale, out, ws, ws_bytes)
    return out


def oracle_seq(wl: Workload, b: int, rows=None) -> np.ndarray:
    """Oracle output for sequence b (new-token rows `rows`, default all): float64 [n, Hq, D]."""
    s = wl.seqs[b]
    sl = wl.seq_tokens(b)
    q = to_f32(wl.q[sl], wl.dtype)
    kk = np.concatenate([to_f32(wl.hist_k[b], wl.dtype), to_f32(wl.k_new[sl], wl.dtype)])
    vv = np.concatenate([to_f32(wl.hist_v[b], wl.dtype), to_f32(wl.v_new[sl], wl.dtype)])
    rows = np.arange(s.n_new) if rows is None else np.asarray(rows)
    return oracle.attend(q[rows], s.start_pos + rows, kk, vv, s.hist_lo, wl.window, wl.scale)


def oracle_all(wl: Workload) -> np.ndarray:
    parts = [oracle_seq(wl, b) for b in range(wl.num_seqs)]
    return np.concatenate(parts) if parts else np.zeros((0, wl.n_q_heads, wl.head_dim))


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref)
    mx = float(err.max()) if err.size else 0.0
    assert mx <= TOL[dtype], f"{what}: max abs err {mx:.3e} > {TOL[dtype]}"
    if dtype == "bf16" and err.size:
        rel = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
        assert rel <= REL_RMS_BF16, f"{what}: rel-RMS {rel:.3e} > {REL_RMS_BF16}"
    return mx


def one_hot_v(n_pos, hkv, d, dtype, base=0):
    """Value row of position j with h = d / 2: one-hot(j mod h) in dims 0..h-1 and
    one-hot((j // h) mod h) in dims h..d-1 (h = 64 at head_dim 128)."""
    h = d // 2
    v = np.zeros((n_pos, hkv, d), np.float32)
    for r in range(n_pos):
        j = base + r
        v[r, :, j % h] = 1.0
        v[r, :, h + (j // h) % h] = 1.0
    return bf16_bits_from_f32(v) if dtype == "bf16" else v


def expected_hist(i, window, d=128):
    """Histogram of the one-hot codes (see one_hot_v) of the positions in
    J(i) = [max(0, i-W+1), i], and |J(i)|."""
    h = d // 2
    band = np.arange(max(0, i - window + 1), i + 1)
    lo = np.bincount(band % h, minlength=h)
    hi = np.bincount((band // h) % h, minlength=h)
    return np.concatenate([lo, hi]).astype(np.float64), len(band)
