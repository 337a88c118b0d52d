"""Dense brute-force sliding-window GQA attention (numpy, float64).

TEST INFRASTRUCTURE ONLY: a second, independent statement of the definition,
used to pin the C oracle on tiny inputs.  It builds the explicit N x N mask

    M[i, j] = (j <= i) and (i - j < W)

(Mistral 7B (Chinese translation), section 2, paragraph "Sliding Window
Attention" and the Figure 1 caption: a window of W tokens ending at the
query itself), sets masked scores to -inf, takes a dense row softmax and multiplies
by V.  Query head h reads key/value head h // G (grouped-query attention,
section 1).
"""
from __future__ import annotations

import numpy as np


def band_mask(n: int, window: int) -> np.ndarray:
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & ((i - j) < window)


def brute_masked_attention(q, k, v, window: int, scale: float) -> np.ndarray:
    """q [N, Hq, D], k/v [N, Hkv, D] for positions 0..N-1 -> out [N, Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, _ = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    mask = band_mask(n, window)
    out = np.empty_like(q)
    for h in range(hq):
        kh = k[:, h // group, :]
        vh = v[:, h // group, :]
        s = scale * (q[:, h, :] @ kh.T)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out
