"""Seeded synthetic workloads for sliding-window GQA attention.

This module only draws inputs: normal(0, 1) activations rounded to the input
dtype, sequence lengths, start positions and cache-row assignments.  It holds
none of the attention arithmetic and none of the cache-slot arithmetic, so the
GPU path and the CPU oracle can both be fed from it without sharing any of the
method.

The shapes follow Mistral 7B as described in the paper (grouped-query
attention with 32 query heads over 8 key/value heads, head_dim 128, sliding
window W = 4096; Mistral 7B (Chinese translation), sections 1 and 2).  The
paper publishes no attention inputs, so every tensor here is synthetic.

Raw tensors are returned in their storage form: ``uint16`` bit patterns for
bf16 and ``float32`` for f32.  :func:`to_f32` widens either one exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DTYPES = ("bf16", "f32")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns with round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f32(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_from_bf16_bits(raw)
    if dtype == "f32":
        return np.ascontiguousarray(raw, dtype=np.float32)
    raise ValueError(dtype)


def randn(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) drawn in float32, stored in ``dtype`` (bf16 via RNE)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


@dataclass
class Seq:
    """One sequence of a batch: ``n_new`` new tokens at absolute positions
    ``start_pos .. start_pos + n_new - 1``; ``hist_lo`` is the first earlier
    position whose keys/values are part of the workload (the history that is
    in the cache before the call)."""
    start_pos: int
    n_new: int
    hist_lo: int
    cache_row: int


@dataclass
class Workload:
    name: str
    window: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    scale: float
    seqs: List[Seq]
    n_cache: int
    # raw tensors (storage dtype): new tokens packed by sequence, token-major
    q: Optional[np.ndarray] = None        # [T, Hq, D]
    k_new: Optional[np.ndarray] = None    # [T, Hkv, D]
    v_new: Optional[np.ndarray] = None
    hist_k: List[np.ndarray] = field(default_factory=list)  # per seq [start-hist_lo, Hkv, D]
    hist_v: List[np.ndarray] = field(default_factory=list)

    @property
    def num_seqs(self) -> int:
        return len(self.seqs)

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([s.n_new for s in self.seqs])]).astype(np.int32)

    @property
    def start_pos(self) -> np.ndarray:
        return np.array([s.start_pos for s in self.seqs], dtype=np.int32)

    @property
    def cache_idx(self) -> np.ndarray:
        return np.array([s.cache_row for s in self.seqs], dtype=np.int32)

    @property
    def hist_start_pos(self) -> np.ndarray:
        return np.array([s.hist_lo for s in self.seqs], dtype=np.int32)

    @property
    def hist_cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([s.start_pos - s.hist_lo for s in self.seqs])]).astype(np.int32)

    @property
    def total_tokens(self) -> int:
        return int(sum(s.n_new for s in self.seqs))

    @property
    def max_new_tokens(self) -> int:
        return int(max([s.n_new for s in self.seqs] + [0]))

    def hist_packed(self, which: str) -> np.ndarray:
        parts = self.hist_k if which == "k" else self.hist_v
        shape = (0, self.n_kv_heads, self.head_dim)
        dt = np.uint16 if self.dtype == "bf16" else np.float32
        parts = [p for p in parts if p.shape[0] > 0]
        return np.concatenate(parts, axis=0) if parts else np.zeros(shape, dtype=dt)

    def seq_tokens(self, b: int) -> slice:
        cu = self.cu_seqlens
        return slice(int(cu[b]), int(cu[b + 1]))


def make_workload(name: str, seed: int, seqs_spec, *, window: int, n_q_heads: int,
                  n_kv_heads: int, head_dim: int, dtype: str, scale: Optional[float] = None,
                  history: bool = True, cache_rows=None, n_cache: Optional[int] = None) -> Workload:
    """Draw a workload.  ``seqs_spec`` is a list of (start_pos, n_new).

    The history of a sequence covers positions [max(0, start_pos - window + 1), start_pos),
    i.e. what a query at ``start_pos`` may read from the cache.  Draw order per sequence:
    history K, history V, new K, new V, new Q.
    """
    rng = np.random.default_rng(seed)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    n = len(seqs_spec)
    if cache_rows is None:
        cache_rows = list(range(n))
    seqs = []
    for b, (sp, c) in enumerate(seqs_spec):
        lo = max(0, sp - window + 1) if history else sp
        seqs.append(Seq(int(sp), int(c), int(lo), int(cache_rows[b])))
    wl = Workload(name, window, n_q_heads, n_kv_heads, head_dim, dtype, float(scale), seqs,
                  int(n_cache if n_cache is not None else (max(cache_rows) + 1 if n else 1)))
    qs, ks, vs = [], [], []
    for s in seqs:
        nh = s.start_pos - s.hist_lo
        wl.hist_k.append(randn(rng, (nh, n_kv_heads, head_dim), dtype))
        wl.hist_v.append(randn(rng, (nh, n_kv_heads, head_dim), dtype))
        ks.append(randn(rng, (s.n_new, n_kv_heads, head_dim), dtype))
        vs.append(randn(rng, (s.n_new, n_kv_heads, head_dim), dtype))
        qs.append(randn(rng, (s.n_new, n_q_heads, head_dim), dtype))
    dt = np.uint16 if dtype == "bf16" else np.float32
    cat = lambda xs, h: (np.concatenate(xs, axis=0) if xs else np.zeros((0, h, head_dim), dtype=dt))
    wl.q, wl.k_new, wl.v_new = cat(qs, n_q_heads), cat(ks, n_kv_heads), cat(vs, n_kv_heads)
    return wl


# --------------------------------------------------------------------------------------
# The five workloads of the benchmark suite (all synthetic, normal(0, 1) inputs).
# --------------------------------------------------------------------------------------

def tiny_prefill(seed: int = 1001) -> Workload:
    """Batch 1, seq 64, 4 query / 2 KV heads, head_dim 16, W = 8, f32, scale 1/sqrt(16)."""
    return make_workload("tiny-swa-gqa-f32", seed, [(0, 64)], window=8, n_q_heads=4,
                         n_kv_heads=2, head_dim=16, dtype="f32", scale=0.25)


def mistral_prefill(seed: int = 1002, window: int = 4096, n: int = 16384) -> Workload:
    """Batch 1, one prefill call over ``n`` tokens, 32 q / 8 kv heads, head_dim 128, bf16."""
    return make_workload(f"mistral-prefill-{n}-w{window}", seed, [(0, n)], window=window,
                         n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16")


def chunked_sequences(seed: int = 1003, batch: int = 4, n: int = 32768, window: int = 4096,
                      n_q_heads: int = 32, n_kv_heads: int = 8, head_dim: int = 128,
                      dtype: str = "bf16"):
    """Whole sequences for chunked prefill: q [B, N, Hq, D], k/v [B, N, Hkv, D] (raw)."""
    rng = np.random.default_rng(seed)
    k = randn(rng, (batch, n, n_kv_heads, head_dim), dtype)
    v = randn(rng, (batch, n, n_kv_heads, head_dim), dtype)
    q = randn(rng, (batch, n, n_q_heads, head_dim), dtype)
    return q, k, v


def batched_decode(seed: int = 1004, batch: int = 64, window: int = 4096,
                   pos_lo: int = 4096, pos_hi: int = 32768) -> Workload:
    """64 sequences, current positions uniform in [pos_lo, pos_hi), full W-slot history."""
    rng = np.random.default_rng(seed)
    pos = rng.integers(pos_lo, pos_hi, size=batch)
    return make_workload(f"decode-b{batch}-w{window}", seed + 1, [(int(p), 1) for p in pos],
                         window=window, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16")


def ragged_mixed(seed: int = 1005, variant: bool = False, window: int = 4096, n_seqs: int = 48,
                 n_prefill: int = 16, chunk: int = 4096, lmin: int = 512, lmax: int = 32768):
    """48 sequences, context lengths log-uniform in [512, 32768] (or all 8192 for the variant).

    The first ``n_prefill`` are in prefill with chunk ``chunk`` (the last min(chunk, L)
    positions of the context are new), the rest decode their last position.  Cache rows
    are a seeded permutation.  Returns (prefill Workload, decode Workload), sharing one
    cache of ``n_seqs`` rows.
    """
    rng = np.random.default_rng(seed)
    if variant:
        lens = np.full(n_seqs, 8192, dtype=np.int64)
    else:
        lens = np.rint(np.exp(rng.uniform(math.log(lmin), math.log(lmax), size=n_seqs))).astype(np.int64)
    rows = rng.permutation(n_seqs)
    pre = [(int(L - min(chunk, L)), int(min(chunk, L))) for L in lens[:n_prefill]]
    dec = [(int(L - 1), 1) for L in lens[n_prefill:]]
    tag = "variant" if variant else "loguniform"
    wp = make_workload(f"mixed-{tag}-prefill", seed + 1, pre, window=window, n_q_heads=32,
                       n_kv_heads=8, head_dim=128, dtype="bf16",
                       cache_rows=[int(r) for r in rows[:n_prefill]], n_cache=n_seqs)
    wd = make_workload(f"mixed-{tag}-decode", seed + 2, dec, window=window, n_q_heads=32,
                       n_kv_heads=8, head_dim=128, dtype="bf16",
                       cache_rows=[int(r) for r in rows[n_prefill:]], n_cache=n_seqs)
    return wp, wd
