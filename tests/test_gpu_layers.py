"""Stacked sliding-window layers on the GPU: a multi-layer rolling cache and the
receptive field of k layers.

Mistral 7B (Chinese translation), section 2:
  * paragraph "Sliding Window Attention" and the Figure 1 caption: a query
    attends to W positions ending at itself, so each layer moves information
    forward by at most W-1 positions and after k layers position i depends on
    positions i - k(W-1) .. i only;
  * paragraph "Rolling Buffer Cache": every layer keeps its own W-slot ring.
    Here the rings of all layers live in one [L][n_cache][Hkv][W][D] tensor and
    each layer's swa_cache points at its slice;
  * paragraph "Pre-fill and Chunking": the prompt goes through all layers chunk
    by chunk, each chunk attending to the layer's ring and to itself.

The layers around attention are synthetic stand-ins (fixed random projections
and a residual connection, fp32 torch matmuls); attention and the cache writes
run in the library.  Pins: exact properties (which outputs may change, what
each ring slice holds), every layer's attention against the oracle on the very
inputs the GPU saw, the whole fp32 stack against the same stack on the CPU with
the oracle's attention, and a 32-layer ring at 32K tokens (the paper's 8x less
cache memory, paragraph "Rolling Buffer Cache").
"""
import math

import numpy as np
import pytest

import oracle
import sliding_window_gqa_swa_amd as swa
from helpers import check_close, host_f32, torch

pytestmark = pytest.mark.gpu


def make_weights(n_layers, hq, hkv, d, seed):
    t = torch()
    g = t.Generator(device="cpu").manual_seed(seed)
    e = hq * d

    def w(a, b):
        return (t.randn(a, b, generator=g) / math.sqrt(a)).cuda()

    return [(w(e, hq * d), w(e, hkv * d), w(e, hkv * d), w(hq * d, e)) for _ in range(n_layers)]


def run_stack(x0, weights, window, chunk, dtype, hq, hkv, d):
    """Chunk-major pass of x0 [n][hq*d] through the layers.  Returns the final
    activations, the multi-layer cache tensors and every layer's K/V rows."""
    t = torch()
    n = x0.shape[0]
    n_layers = len(weights)
    tdt = t.bfloat16 if dtype == "bf16" else t.float32
    kk = t.full((n_layers, 1, hkv, window, d), float("nan"), dtype=tdt, device="cuda")
    vv = t.full((n_layers, 1, hkv, window, d), float("nan"), dtype=tdt, device="cuda")
    caches = [swa.Cache(kk[layer], vv[layer]) for layer in range(n_layers)]
    k_rows = [t.empty((n, hkv, d), dtype=tdt, device="cuda") for _ in range(n_layers)]
    v_rows = [t.empty((n, hkv, d), dtype=tdt, device="cuda") for _ in range(n_layers)]
    q_rows = [t.empty((n, hq, d), dtype=tdt, device="cuda") for _ in range(n_layers)]
    a_rows = [t.empty((n, hq, d), dtype=tdt, device="cuda") for _ in range(n_layers)]
    out = t.empty_like(x0)
    scale = 1.0 / math.sqrt(d)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        batch = swa.Batch([c], [s], [0])
        x = x0[s:s + c]
        for layer, (wq, wk, wv, wo) in enumerate(weights):
            q = (x @ wq).to(tdt).reshape(c, hq, d).contiguous()
            k = (x @ wk).to(tdt).reshape(c, hkv, d).contiguous()
            v = (x @ wv).to(tdt).reshape(c, hkv, d).contiguous()
            a = t.empty((c, hq, d), dtype=tdt, device="cuda")
            swa.swa_prefill_chunk(caches[layer], batch, q, hq, k, v, scale, a)
            swa.swa_cache_write(caches[layer], batch, k, v)
            k_rows[layer][s:s + c] = k
            v_rows[layer][s:s + c] = v
            q_rows[layer][s:s + c] = q
            a_rows[layer][s:s + c] = a
            x = x + a.float().reshape(c, hq * d) @ wo
        out[s:s + c] = x
    t.cuda.synchronize()
    return out, kk, vv, k_rows, v_rows, q_rows, a_rows


CASES = [("f32", 16, 4, 6), ("bf16", 128, 8, 16)]


@pytest.mark.parametrize("dtype,d,window,chunk", CASES)
def test_receptive_field_of_stacked_layers(dtype, d, window, chunk):
    t = torch()
    n_layers, hq, hkv, n = 3, 2, 1, 64
    weights = make_weights(n_layers, hq, hkv, d, seed=7)
    g = t.Generator(device="cpu").manual_seed(8)
    x0 = t.randn(n, hq * d, generator=g).cuda()
    base = run_stack(x0, weights, window, chunk, dtype, hq, hkv, d)[0]
    reach = n_layers * (window - 1)
    for j in (0, 17, n - 1):
        x1 = x0.clone()
        x1[j] += 1.0
        pert = run_stack(x1, weights, window, chunk, dtype, hq, hkv, d)[0]
        changed = (pert != base).any(dim=1).cpu().numpy()
        inside = np.array([j <= i <= j + reach for i in range(n)])
        # outside the receptive field nothing may move, not even by one ulp
        assert not changed[~inside].any(), (j, np.nonzero(changed & ~inside))
        if dtype == "f32":
            # fp32 resolves the whole field, up to its far edge j + k(W-1)
            assert changed[inside].all(), (j, np.nonzero(inside & ~changed))
        else:
            # bf16: at least the first layer's direct reach j .. j+W-1 is visible
            first = np.array([j <= i <= j + window - 1 for i in range(n)])
            assert changed[first].all(), (j, np.nonzero(first & ~changed))


@pytest.mark.parametrize("dtype,d,window,chunk", CASES)
def test_multilayer_cache_slices_hold_each_layers_last_window(dtype, d, window, chunk):
    t = torch()
    n_layers, hq, hkv, n = 3, 2, 1, 53
    weights = make_weights(n_layers, hq, hkv, d, seed=9)
    x0 = t.randn(n, hq * d, generator=t.Generator(device="cpu").manual_seed(10)).cuda()
    _, kk, vv, k_rows, v_rows, _, _ = run_stack(x0, weights, window, chunk, dtype, hq, hkv, d)
    # one allocation for all layers: L x (Hkv x W x D) elements, W slots per layer whatever n is
    assert kk.numel() == n_layers * hkv * window * d
    for layer in range(n_layers):
        for p in range(n - window, n):
            assert t.equal(kk[layer, 0, :, p % window].view(t.int16 if dtype == "bf16" else t.int32),
                           k_rows[layer][p].view(t.int16 if dtype == "bf16" else t.int32)), (layer, p)
            assert t.equal(vv[layer, 0, :, p % window].view(t.int16 if dtype == "bf16" else t.int32),
                           v_rows[layer][p].view(t.int16 if dtype == "bf16" else t.int32)), (layer, p)
    # the layers' K rows differ (independent projections), so a slice mix-up would show
    assert not t.equal(k_rows[0], k_rows[1])


@pytest.mark.parametrize("dtype,d,window,chunk", CASES)
def test_every_layer_matches_the_oracle(dtype, d, window, chunk):
    """Each layer's attention, computed chunk by chunk through that layer's slice of
    the multi-layer ring, equals the oracle's unchunked attention on the same q, k, v
    (the exact values the GPU saw), within the dtype's tolerance."""
    t = torch()
    n_layers, hq, hkv, n = 3, 2, 1, 64
    weights = make_weights(n_layers, hq, hkv, d, seed=11)
    x0 = t.randn(n, hq * d, generator=t.Generator(device="cpu").manual_seed(12)).cuda()
    _, _, _, k_rows, v_rows, q_rows, a_rows = run_stack(x0, weights, window, chunk, dtype, hq, hkv, d)
    for layer in range(n_layers):
        q, k, v = (host_f32(x[layer], dtype) for x in (q_rows, k_rows, v_rows))
        ref = oracle.attend(q, np.arange(n), k, v, 0, window, 1.0 / math.sqrt(d))
        check_close(host_f32(a_rows[layer], dtype), ref, dtype, f"layer {layer}")


def test_fp32_stack_matches_cpu_stack_with_oracle_attention():
    """The whole 3-layer fp32 stack (chunk-major through the rings) against the same
    stack on the CPU, layer-major and unchunked: the same fp32 projections and
    residuals, attention by the oracle (fp64, rounded to fp32 as the GPU stores it)."""
    t = torch()
    dtype, d, window, chunk = "f32", 16, 4, 6
    n_layers, hq, hkv, n = 3, 2, 1, 64
    weights = make_weights(n_layers, hq, hkv, d, seed=13)
    x0 = t.randn(n, hq * d, generator=t.Generator(device="cpu").manual_seed(14)).cuda()
    out = run_stack(x0, weights, window, chunk, dtype, hq, hkv, d)[0].cpu().numpy()
    x = x0.cpu().numpy().astype(np.float32)
    for wq, wk, wv, wo in weights:
        wq, wk, wv, wo = (w.cpu().numpy() for w in (wq, wk, wv, wo))
        q = (x @ wq).astype(np.float32).reshape(n, hq, d)
        k = (x @ wk).astype(np.float32).reshape(n, hkv, d)
        v = (x @ wv).astype(np.float32).reshape(n, hkv, d)
        a = oracle.attend(q, np.arange(n), k, v, 0, window, 1.0 / math.sqrt(d)).astype(np.float32)
        x = x + a.reshape(n, hq * d) @ wo
    err = float(np.abs(out - x).max())
    assert err <= 1e-4, err


def test_32_layer_ring_at_32k_tokens():
    """32 layers x 32768 tokens through 4096-slot rings (32 q / 8 kv heads, head_dim 128,
    bf16): every layer's slice of the [32][1][8][4096][128] tensors ends up holding
    exactly that layer's last 4096 positions, bit for bit, and the rings take 1/8 of
    the bytes a full 32K cache of the same layers would."""
    t = torch()
    L, N, C, W, hkv, d = 32, 32768, 4096, 4096, 8, 128
    kk = t.empty((L, 1, hkv, W, d), dtype=t.bfloat16, device="cuda")
    vv = t.empty((L, 1, hkv, W, d), dtype=t.bfloat16, device="cuda")
    full_bytes = 2 * L * N * hkv * d * 2
    assert full_bytes == 8 * (kk.numel() + vv.numel()) * 2

    def pattern(layer, s, which):
        # distinct 16-bit word per (layer, position, head, d, K or V)
        pos = t.arange(s, s + C, device="cuda", dtype=t.int64).view(C, 1, 1)
        g = t.arange(hkv, device="cuda", dtype=t.int64).view(1, hkv, 1)
        e = t.arange(d, device="cuda", dtype=t.int64).view(1, 1, d)
        w = (((layer * 2 + which) * 1000003 + pos * 977 + g * 131 + e) * 2654435761) >> 7
        return (w & 0x7F7F).to(t.int16).view(t.bfloat16).contiguous()

    for layer in range(L):
        c = swa.Cache(kk[layer], vv[layer])
        for s in range(0, N, C):
            swa.swa_cache_write(c, swa.Batch([C], [s], [0]), pattern(layer, s, 0), pattern(layer, s, 1))
    t.cuda.synchronize()
    slots = t.arange(N - C, N, device="cuda") % W
    for layer in range(L):
        for which, ring in ((0, kk), (1, vv)):
            expect = pattern(layer, N - C, which)                    # positions N-C .. N-1
            got = ring[layer, 0][:, slots, :].permute(1, 0, 2)        # [C][hkv][d] in position order
            assert t.equal(got.contiguous().view(t.int16), expect.view(t.int16)), (layer, which)
