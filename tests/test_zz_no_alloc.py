"""swa_decode_step_noalloc: the fused decode step with its split partials in the
library's own device array instead of a caller workspace.

It must give exactly what swa_decode_step gives (output and cache, bit for bit)
and match the fp64 oracle, on consecutive calls that share the array: the
second call is smaller than the first, so it runs over partials the first call
left behind.  Mistral 7B (Chinese translation), section 2, paragraphs "Rolling
Buffer Cache" and "Pre-fill and Chunking".
"""
import numpy as np
import pytest

import sliding_window_gqa_swa_amd as swa
from sliding_window_gqa_swa_amd.workloads import make_workload
from helpers import check_close, dev, host_f32, oracle_all, poisoned_cache, torch, write_history

pytestmark = pytest.mark.gpu


def run_both(n, group, seed):
    t = torch()
    hkv = 32 // group
    pos = np.random.default_rng(seed).integers(0, 20000, size=n)
    wl = make_workload("noalloc", seed, [(int(p), 1) for p in pos], window=4096, n_q_heads=32, n_kv_heads=hkv,
                       head_dim=128, dtype="bf16", cache_rows=list(reversed(range(n))))
    cache = poisoned_cache(n, hkv, 4096, 128, "bf16")
    write_history(cache, wl)
    c_ref = swa.Cache(cache.k.clone(), cache.v.clone())
    c_na = swa.Cache(cache.k.clone(), cache.v.clone())
    batch = swa.Batch([1] * n, [int(p) for p in pos], wl.cache_idx)
    q, kn, vn = dev(wl.q, "bf16"), dev(wl.k_new, "bf16"), dev(wl.v_new, "bf16")
    nb = swa.swa_decode_workspace_size(cache, n, 32)
    ws = t.empty(max(nb, 16), dtype=t.uint8, device="cuda")
    o_ref = t.full((n, 32, 128), float("nan"), dtype=t.bfloat16, device="cuda")
    o_na = t.full_like(o_ref, float("nan"))
    swa.swa_decode_step(c_ref, batch, q, 32, kn, vn, wl.scale, o_ref, ws, nb)
    swa.swa_decode_step_noalloc(c_na, batch, q, 32, kn, vn, wl.scale, o_na)
    t.cuda.synchronize()
    for a, b, what in ((o_ref, o_na, "output"), (c_ref.k, c_na.k, "cache K"), (c_ref.v, c_na.v, "cache V")):
        assert t.equal(a.view(t.int16), b.view(t.int16)), (what, n, group)
    check_close(host_f32(o_na, "bf16"), oracle_all(wl), "bf16", f"noalloc step n={n} G={group}")
    return nb


@pytest.mark.parametrize("group", [4, 1, 8])
def test_noalloc_step_equals_step_on_consecutive_calls(group):
    # both calls split their windows (workspace > 0); the second is smaller
    assert run_both(12, group, 101) > 0
    assert run_both(3, group, 102) > 0


def test_noalloc_step_without_split():
    # 64 sequences x 8 KV heads: one workgroup per ring, the array is not used
    assert run_both(64, 4, 103) == 0
    assert run_both(5, 4, 104) > 0
