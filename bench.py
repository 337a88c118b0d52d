#!/usr/bin/env python3
"""Benchmark of the sliding-window GQA hot path on one MI355X.

One step = one pass over every stage of the path, on synthetic seeded inputs
already resident in HBM:
  1. swa_prefill_chunk : Mistral-shaped prefill, 1 x 16384 tokens, 32 q / 8 kv
                         heads, head_dim 128, W = 4096, bf16 (fp32 accumulate);
  2. swa_cache_write   : that chunk into its 4096-slot rolling buffer;
  3. swa_cache_write   : one new token for each of 64 decoding sequences;
  4. swa_decode        : those 64 sequences (positions in [4096, 32768), full
                         4096-slot rings, 1 GiB of K/V).
The headline value is the prefill's band TFLOP/s (algorithmic FLOPs: 4 * D *
Hq * sum_i |J(i)|); the decode's K/V GB/s is reported beside it.  Each stage
is timed with HIP events on the stream it runs on.  Before the warm-up steps,
untimed steps run for 0.2 s: from idle, the part needs a few tens of
milliseconds of load to reach the clock it holds under it, and every timing of
the suite is preceded by 0.1 s of the same, and each suite timing is the
median of three windows of back-to-back launches.

The suite (default on) times the other workloads: causal attention and the
prefill without its band tile skip at 16K tokens, the chunk's cache write
against a plain device copy of the same bytes (both right after the prefill),
4 x 32768 tokens chunked through the ring (and a chunk-size sweep), the ragged
mixed batch, decode at G = 1, per-token decode steps, and a 32-layer ring.  The CPU baseline is the
fp64 oracle on the host cores: the whole 16K prefill, plus stated samples of
the other workloads.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--no-cpu-baseline] [--no-suite]
    python bench.py --only chunked|mixed|decode_g1|write_vs_copy   # one suite workload (for profilers)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SWA-GQA prefill band-TFLOP/s + decode KV GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
SPEC_CLOCK_GHZ = 2.4        # the clock the MFMA peak is quoted at
PREFILL_KERNEL = "prefill_bf16_kernel"
PMC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_mistral16k_w4096_pmc.json")
PREFILL_SRC = os.path.join(ROOT, "sliding_window_gqa_swa_amd", "csrc", "prefill_bf16.hip")
W = 4096
HQ, HKV, D = 32, 8, 128


def band_pairs(start: int, n: int, window: int) -> int:
    """Sum over query positions i in [start, start+n) of |J(i)| = min(i + 1, W)."""
    total = 0
    for i in range(start, start + n):
        total += min(i + 1, window)
    return total


def src_digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def pmc_record():
    """The committed counter summary of the prefill kernel, or None when it is
    missing or the kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_src_sha") != src_digest(PREFILL_SRC):
        return None
    return rec


def pmc_source() -> str:
    return (f"read from {os.path.relpath(PMC_FILE, ROOT)} (rocprofv3 counters of an earlier run; used only while "
            f"the prefill source sha256[:16] {src_digest(PREFILL_SRC)} matches the one recorded there)")


def pmc_traffic():
    """HBM bytes per prefill launch (calibrated FETCH_SIZE + WRITE_SIZE), or None."""
    rec = pmc_record()
    return None if rec is None else float(rec["traffic_bytes_per_launch"])


def sclk_estimate(t_launch_ms: float, tflops: float):
    """Shader clock implied by the prefill's cycle count per launch (GRBM_GUI_ACTIVE
    per XCD, constant from launch to launch) and its measured duration, with the
    fraction of the MFMA peak at that clock; None without the counter summary."""
    rec = pmc_record()
    if rec is None or "cycles_per_xcd_per_launch" not in rec:
        return None
    ghz = float(rec["cycles_per_xcd_per_launch"]) / (t_launch_ms * 1e6)
    peak_at_clk = PEAK_BF16_TFLOPS * ghz / SPEC_CLOCK_GHZ
    return {"ghz": round(ghz, 3), "spec_ghz": SPEC_CLOCK_GHZ, "mfma_peak_at_sclk_tflops": round(peak_at_clk, 1),
            "frac_of_peak_at_sclk": round(tflops / peak_at_clk, 4),
            "source": "GRBM_GUI_ACTIVE cycles per launch / 8 XCDs / this run's measured launch duration; the "
                      "cycle count is " + pmc_source()}


# ----------------------------------------------------------------------------- CPU baseline (the oracle)

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_timed(fn, threads: int, min_s: float = 0.0):
    """Seconds per call of fn (an oracle call) at `threads` OpenMP threads.  Calls
    shorter than min_s are repeated and averaged."""
    import oracle
    oracle.set_num_threads(threads)
    used = oracle.num_threads()
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    oracle.set_num_threads(host_threads())
    return dt / n, used


def cpu_baseline_prefill(wl):
    """The fp64 oracle on every query row of the 16K prefill (W = 4096)."""
    import numpy as np
    import oracle
    from sliding_window_gqa_swa_amd.workloads import to_f32
    n = wl.seqs[0].n_new
    rows = np.arange(n)
    q, k, v = to_f32(wl.q, wl.dtype), to_f32(wl.k_new, wl.dtype), to_f32(wl.v_new, wl.dtype)
    dt, used = oracle_timed(lambda: oracle.attend(q, rows, k, v, 0, wl.window, wl.scale), host_threads())
    flops = 4.0 * wl.head_dim * wl.n_q_heads * band_pairs(0, n, wl.window)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"all {n} query rows x {wl.n_q_heads} heads of the 16384-token prefill (W={wl.window}), "
                      f"fp64, {flops / 1e9:.1f} GFLOP in {dt:.2f} s"}


def cpu_leg_tiny():
    """Tiny fp32 configuration (1 x 64 tokens, 4 q / 2 kv heads, head_dim 16, W = 8): whole workload."""
    import numpy as np
    import oracle
    from sliding_window_gqa_swa_amd.workloads import tiny_prefill, to_f32
    wl = tiny_prefill(1001)
    q, k, v = to_f32(wl.q, "f32"), to_f32(wl.k_new, "f32"), to_f32(wl.v_new, "f32")
    pos = np.arange(64)
    flops = 4.0 * 16 * 4 * band_pairs(0, 64, 8)
    rec = {"workload": "tiny fp32: 1 x 64 tokens, 4 q / 2 kv heads, head_dim 16, W = 8 (whole)", "flops": flops}
    for th in (host_threads(), 1):
        dt, used = oracle_timed(lambda: oracle.attend(q, pos, k, v, 0, 8, 0.25), th, min_s=0.5)
        rec[f"threads_{used}"] = {"s_per_call": dt, "gflops": round(flops / dt / 1e9, 3)}
    return rec


def cpu_leg_decode(wd):
    """64-sequence decode (full 4096-slot windows): every sequence and head, all threads and one thread."""
    import numpy as np
    import oracle
    from sliding_window_gqa_swa_amd.workloads import to_f32
    args = []
    for b, s in enumerate(wd.seqs):
        kk = np.concatenate([to_f32(wd.hist_k[b], "bf16"), to_f32(wd.k_new[b:b + 1], "bf16")])
        vv = np.concatenate([to_f32(wd.hist_v[b], "bf16"), to_f32(wd.v_new[b:b + 1], "bf16")])
        args.append((to_f32(wd.q[b:b + 1], "bf16"), np.array([s.start_pos]), kk, vv, s.hist_lo))

    def run():
        for q, pos, kk, vv, lo in args:
            oracle.attend(q, pos, kk, vv, lo, W, wd.scale)

    kv_bytes = sum(2 * HKV * D * 2 * min(s.start_pos + 1, W) for s in wd.seqs)
    rec = {"workload": f"{wd.num_seqs}-sequence decode, full {W}-slot windows (whole)", "kv_bytes": kv_bytes}
    for th in (host_threads(), 1):
        dt, used = oracle_timed(run, th)
        rec[f"threads_{used}"] = {"s": round(dt, 3), "kv_gbps": round(kv_bytes / dt / 1e9, 3)}
    return rec


def cpu_leg_chunked(q, k, v, b=0, chunk_start=32768 - 4096, chunk=4096):
    """Chunked 4 x 32768 workload, sample: the last chunk of sequence 0 (every row and head)."""
    import numpy as np
    import oracle
    from sliding_window_gqa_swa_amd.workloads import to_f32
    rows = np.arange(chunk_start, chunk_start + chunk)
    lo = chunk_start - W + 1
    qs = to_f32(q[b, chunk_start:chunk_start + chunk], "bf16")
    ks, vs = to_f32(k[b, lo:chunk_start + chunk], "bf16"), to_f32(v[b, lo:chunk_start + chunk], "bf16")
    dt, used = oracle_timed(lambda: oracle.attend(qs, rows, ks, vs, lo, W, 1 / 128 ** 0.5), host_threads())
    flops = 4.0 * D * HQ * band_pairs(chunk_start, chunk, W)
    return {"sample": f"sequence {b}, positions {chunk_start}..{chunk_start + chunk - 1} (the last chunk), all heads",
            "cores": used, "gflop": round(flops / 1e9, 1), "s": round(dt, 2), "tflops": round(flops / dt / 1e12, 4)}


def cpu_leg_mixed(wp, wd, rows_per_seq=256):
    """Ragged mixed batch, sample: every decode sequence, and the last `rows_per_seq`
    query rows of every prefill sequence."""
    import numpy as np
    import oracle
    from sliding_window_gqa_swa_amd.workloads import to_f32

    def seq_args(wl, b, rows):
        s = wl.seqs[b]
        sl = wl.seq_tokens(b)
        kk = np.concatenate([to_f32(wl.hist_k[b], "bf16"), to_f32(wl.k_new[sl], "bf16")])
        vv = np.concatenate([to_f32(wl.hist_v[b], "bf16"), to_f32(wl.v_new[sl], "bf16")])
        return to_f32(wl.q[sl][rows], "bf16"), s.start_pos + rows, kk, vv, s.hist_lo

    args, flops = [], 0.0
    for wl, per in ((wp, rows_per_seq), (wd, 1)):
        for b, s in enumerate(wl.seqs):
            rows = np.arange(max(0, s.n_new - per), s.n_new)
            args.append(seq_args(wl, b, rows))
            flops += 4.0 * D * HQ * sum(min(int(s.start_pos + r) + 1, W) for r in rows)

    def run():
        for q, pos, kk, vv, lo in args:
            oracle.attend(q, pos, kk, vv, lo, W, wp.scale)

    dt, used = oracle_timed(run, host_threads())
    return {"sample": f"all {wd.num_seqs} decode sequences and the last {rows_per_seq} query rows of each of the "
                      f"{wp.num_seqs} prefill sequences, all heads", "cores": used, "gflop": round(flops / 1e9, 2),
            "s": round(dt, 2), "tflops": round(flops / dt / 1e12, 4)}


# ----------------------------------------------------------------------------- timing helpers

SETTLE_S = 0.2  # untimed load before every measurement (the clock ramp from idle takes ~40 ms)
SETTLE_S_SUITE = 0.1


def settle(fn, seconds: float) -> int:
    """Run `fn` repeatedly for `seconds` of wall time, untimed, and return the launch count.

    From idle, the part takes a few tens of milliseconds of load to reach the clock it holds
    under that load. The 16K prefill takes ~0.87 ms per launch over its first 20 launches and
    0.79 ms from about the 50th on (one box, back-to-back launches). A synchronisation every
    8 launches keeps the host from queueing far ahead of the GPU, so the wall time tracks the
    GPU's busy time."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


def time_ms(fn, reps: int, windows: int = 3) -> float:
    """Milliseconds per launch of `fn`, HIP events on the current stream (after `settle`):
    the mean over `reps` back-to-back launches, taken in `windows` separate windows, and the
    median of those means (a lone stall of the host or the part, tens of milliseconds, then
    spoils one window instead of the figure)."""
    import torch
    settle(fn, SETTLE_S_SUITE)
    means = []
    for _ in range(windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / reps)
    return sorted(means)[len(means) // 2]


def time_ms_cold(fn, reps: int, flush) -> float:
    """Mean milliseconds of `fn`, each launch timed alone after `flush` has
    overwritten the 256 MB Infinity Cache (so no input is served from it)."""
    import torch
    settle(lambda: (flush(), fn()), SETTLE_S_SUITE)
    total = 0.0
    for _ in range(reps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    return total / reps


def uploader(dev):
    import numpy as np
    import torch

    def up(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(dev)
    return up


def bf16_cache(n, hkv, window, dev, fill=0.0):
    import torch
    import sliding_window_gqa_swa_amd as swa
    return swa.Cache(torch.full((n, hkv, window, D), fill, dtype=torch.bfloat16, device=dev),
                     torch.full((n, hkv, window, D), fill, dtype=torch.bfloat16, device=dev))


def write_history(cache, wl, up):
    import sliding_window_gqa_swa_amd as swa
    hb = swa.Batch([s.start_pos - s.hist_lo for s in wl.seqs], [s.hist_lo for s in wl.seqs], wl.cache_idx)
    swa.swa_cache_write(cache, hb, up(wl.hist_packed("k")), up(wl.hist_packed("v")))


# ----------------------------------------------------------------------------- suite

def suite_causal_and_no_skip(pq, pk, pv, pout, scale, t_swa_ms, reps):
    """The paper's 2x at 16K / W = 4096 against standard attention: the same kernel
    with W >= N (causal attention), and the W = 4096 prefill with its band tile skip
    turned off (every key tile of the causal triangle visited, out-of-band keys masked)."""
    import torch
    import sliding_window_gqa_swa_amd as swa
    dev = pq.device
    n = pq.shape[0]
    b1 = swa.Batch([n], [0], [0])
    cc = bf16_cache(1, HKV, n, dev)
    t_causal = time_ms(lambda: swa.swa_prefill_chunk(cc, b1, pq, HQ, pk, pv, scale, pout), reps)
    del cc
    c4 = bf16_cache(1, HKV, W, dev)
    t_noskip = time_ms(lambda: swa.swa_prefill_chunk_no_tile_skip(c4, b1, pq, HQ, pk, pv, scale, pout), reps)
    causal_flops = 4.0 * D * HQ * band_pairs(0, n, n)
    band_flops = 4.0 * D * HQ * band_pairs(0, n, W)
    torch.cuda.synchronize()
    return {
        "causal_prefill_16k": {"ms": round(t_causal, 4), "tflops": round(causal_flops / t_causal / 1e9, 1)},
        "no_tile_skip_prefill_16k_w4096": {
            "ms": round(t_noskip, 4), "band_tflops": round(band_flops / t_noskip / 1e9, 1),
            "causal_triangle_tflops": round(causal_flops / t_noskip / 1e9, 1),
            "note": "W = 4096 result, every key tile of the causal triangle visited and masked outside the band"},
        "swa_vs_causal_speedup_16k": round(t_causal / t_swa_ms, 3),
        "swa_vs_no_tile_skip_speedup_16k": round(t_noskip / t_swa_ms, 3),
        "causal_over_band_pairs_16k": round(band_pairs(0, n, n) / band_pairs(0, n, W), 3),
    }


def suite_write_vs_copy(pcache, pbatch, pq, pk, pv, pout, scale, reps):
    """The chunk's cache write against a plain device copy of the same bytes, each timed
    alone right after the 16K prefill (the position it has in the step, where the prefill's
    134 MB of output has just displaced the chunk's K/V from the Infinity Cache).  The write
    moves the last min(C, W) tokens of K and of V; the copy, one contiguous device-to-device
    copy in one launch, moves as many bytes from the end of the chunk's K (which the prefill
    has just read too): the same bytes read and written, with no slot arithmetic."""
    import torch
    import sliding_window_gqa_swa_amd as swa
    n = pk.shape[0]
    rows = min(n, W, n // 2)
    src = pk[n - 2 * rows:]
    dst = torch.empty_like(src)
    nbytes = 2 * src.numel() * src.element_size()
    assert nbytes == 2 * 2 * min(n, W) * pk[0].numel() * pk.element_size()

    def pre():
        swa.swa_prefill_chunk(pcache, pbatch, pq, HQ, pk, pv, scale, pout)

    def copy():
        dst.copy_(src)

    out = {}
    for name, fn in (("cache_write", lambda: swa.swa_cache_write(pcache, pbatch, pk, pv)), ("device_copy", copy)):
        settle(lambda: (pre(), fn()), SETTLE_S_SUITE)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            pre()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
        out[name] = {"us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    out["bytes"] = nbytes
    out["write_over_copy_rate"] = round(out["device_copy"]["us"] / out["cache_write"]["us"], 3)
    return {"chunk_write_vs_device_copy_after_prefill": out}


def suite_chunked(up, scale, reps, cpu: bool):
    """4 x 32768 tokens through the ring in chunks of 4096 (W = 4096), a chunk-size
    sweep, and the chunk cache write with a cold Infinity Cache."""
    import numpy as np
    import torch
    import sliding_window_gqa_swa_amd as swa
    from sliding_window_gqa_swa_amd.workloads import chunked_sequences
    dev = torch.device("cuda:0")
    B, N, C = 4, 32768, 4096
    q, k, v = chunked_sequences(1003, batch=B, n=N, window=W)
    qd, kd, vd = up(q), up(k), up(v)
    cache = bf16_cache(B, HKV, W, dev)
    oc = torch.empty((B * C, HQ, D), dtype=torch.bfloat16, device=dev)
    chunks = []
    for s in range(0, N, C):
        batch = swa.Batch([C] * B, [s] * B, list(range(B)))
        qc = qd[:, s:s + C].reshape(B * C, HQ, D).contiguous()
        kc = kd[:, s:s + C].reshape(B * C, HKV, D).contiguous()
        vc = vd[:, s:s + C].reshape(B * C, HKV, D).contiguous()
        t_p = time_ms(lambda: swa.swa_prefill_chunk(cache, batch, qc, HQ, kc, vc, scale, oc), reps)
        t_w = time_ms(lambda: swa.swa_cache_write(cache, batch, kc, vc), reps)
        chunks.append((t_p, t_w, 4.0 * D * HQ * B * band_pairs(s, C, W)))
    sweep = {}
    for cs in (W // 4, W // 2, W, 2 * W):
        cache.k.zero_()
        cache.v.zero_()
        t_tot, w_tot = 0.0, 0.0
        ob = torch.empty((B * cs, HQ, D), dtype=torch.bfloat16, device=dev)
        for s in range(0, N, cs):
            batch = swa.Batch([cs] * B, [s] * B, list(range(B)))
            qc = qd[:, s:s + cs].reshape(B * cs, HQ, D).contiguous()
            kc = kd[:, s:s + cs].reshape(B * cs, HKV, D).contiguous()
            vc = vd[:, s:s + cs].reshape(B * cs, HKV, D).contiguous()
            t_tot += time_ms(lambda: swa.swa_prefill_chunk(cache, batch, qc, HQ, kc, vc, scale, ob), reps)
            w_tot += time_ms(lambda: swa.swa_cache_write(cache, batch, kc, vc), reps)
        fl = 4.0 * D * HQ * B * band_pairs(0, N, W)
        act = B * cs * (HQ + HKV + HKV + HQ) * D * 2  # q, k_new, v_new, out of one call
        sweep[f"C={cs}"] = {"prefill_ms": round(t_tot, 3), "prefill_tflops": round(fl / t_tot / 1e9, 1),
                            "cache_write_ms": round(w_tot, 3), "calls": N // cs,
                            "activation_mib_per_call": round(act / 2**20, 1)}
        del ob
    big = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    batch = swa.Batch([C] * B, [N - C] * B, list(range(B)))
    kc = kd[:, N - C:].reshape(B * C, HKV, D).contiguous()
    vc = vd[:, N - C:].reshape(B * C, HKV, D).contiguous()
    t_w_cold = time_ms_cold(lambda: swa.swa_cache_write(cache, batch, kc, vc), reps, lambda: big.fill_(1))
    del big, kc, vc, qd, kd, vd, cache
    tot_ms = sum(c[0] for c in chunks)
    wbytes = 2 * 2 * B * C * HKV * D * 2
    res = {"chunked_4x32k_w4096": {
        "prefill_ms_per_chunk": [round(c[0], 4) for c in chunks],
        "prefill_tflops_chunks_1_7": round(sum(c[2] for c in chunks[1:]) / sum(c[0] for c in chunks[1:]) / 1e9, 1),
        "prefill_tflops_all": round(sum(c[2] for c in chunks) / tot_ms / 1e9, 1),
        "cache_write_ms_per_chunk": round(float(np.mean([c[1] for c in chunks])), 4),
        "cache_write_gbps": round(wbytes / float(np.mean([c[1] for c in chunks])) / 1e6, 1),
        "cache_write_cold_ms": round(t_w_cold, 4),
        "cache_write_cold_gbps": round(wbytes / t_w_cold / 1e6, 1)},
        "chunk_sweep_4x32k_w4096": sweep}
    if cpu:
        leg = cpu_leg_chunked(q, k, v)
        leg["gpu_tflops_chunks_1_7"] = res["chunked_4x32k_w4096"]["prefill_tflops_chunks_1_7"]
        res["chunked_4x32k_w4096"]["cpu_oracle"] = leg
    return res


def suite_mixed(up, scale, reps, cpu: bool):
    """Ragged mixed batch: 16 prefill + 32 decode sequences sharing one 48-row cache,
    and the context-8192 variant.  Each launch is set against its roofline bound
    (algorithmic FLOPs or bytes at the MFMA / HBM peak)."""
    import torch
    import sliding_window_gqa_swa_amd as swa
    from sliding_window_gqa_swa_amd.workloads import ragged_mixed
    dev = torch.device("cuda:0")
    res = {}
    for variant in (False, True):
        wp, wd = ragged_mixed(1005, variant=variant)
        cache = bf16_cache(48, HKV, W, dev)
        for wl in (wp, wd):
            write_history(cache, wl, up)
        pb = swa.Batch([s.n_new for s in wp.seqs], [s.start_pos for s in wp.seqs], wp.cache_idx)
        mq, mk, mv = up(wp.q), up(wp.k_new), up(wp.v_new)
        mo = torch.empty((wp.total_tokens, HQ, D), dtype=torch.bfloat16, device=dev)
        db = swa.Batch([1] * wd.num_seqs, [s.start_pos for s in wd.seqs], wd.cache_idx)
        dq, dk, dv = up(wd.q), up(wd.k_new), up(wd.v_new)
        do = torch.empty((wd.num_seqs, HQ, D), dtype=torch.bfloat16, device=dev)
        wsb = swa.swa_decode_workspace_size(cache, wd.num_seqs, HQ)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        t_p = time_ms(lambda: swa.swa_prefill_chunk(cache, pb, mq, HQ, mk, mv, scale, mo), reps)
        t_dw = time_ms(lambda: swa.swa_cache_write(cache, db, dk, dv), reps)
        t_d = time_ms(lambda: swa.swa_decode(cache, db, dq, HQ, scale, do, ws, wsb), reps)
        t_step = time_ms(lambda: swa.swa_decode_step(cache, db, dq, HQ, dk, dv, scale, do, ws, wsb), reps)
        pfl = 4.0 * D * HQ * sum(band_pairs(s.start_pos, s.n_new, W) for s in wp.seqs)
        kvb = sum(2 * HKV * D * 2 * min(s.start_pos + 1, W) for s in wd.seqs)
        wbytes = 2 * 2 * wd.num_seqs * HKV * D * 2
        b_p, b_d, b_w = pfl / (PEAK_BF16_TFLOPS * 1e9), kvb / (PEAK_HBM_GBPS * 1e6), wbytes / (PEAK_HBM_GBPS * 1e6)
        rec = {"prefill_ms": round(t_p, 4), "prefill_tflops": round(pfl / t_p / 1e9, 1),
               "decode_us": round(t_d * 1e3, 1), "decode_gbps": round(kvb / t_d / 1e6, 1),
               "decode_write_us": round(t_dw * 1e3, 1), "fused_decode_step_us": round(t_step * 1e3, 1),
               "bound_ms": {"prefill": round(b_p, 4), "decode": round(b_d, 4), "decode_write": round(b_w, 5)},
               "end_to_end_ms": round(t_p + t_d + t_dw, 4),
               "end_to_end_frac_of_bound": round((b_p + b_d + b_w) / (t_p + t_d + t_dw), 3),
               "end_to_end_fused_ms": round(t_p + t_step, 4),
               "end_to_end_fused_frac_of_bound": round((b_p + b_d + b_w) / (t_p + t_step), 3)}
        if cpu and not variant:
            rec["cpu_oracle"] = cpu_leg_mixed(wp, wd)
        res["mixed_" + ("ctx8192" if variant else "loguniform")] = rec
        del cache
    return res


def suite_decode_g1(scale, reps, n_seqs=32):
    """Decode at G = 1 (32 query heads over 32 KV heads: the VALU kernel), full
    4096-slot rings, caches filled on the device from a seeded generator."""
    import numpy as np
    import torch
    import sliding_window_gqa_swa_amd as swa
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1006)
    hkv = 32
    cache = swa.Cache(torch.randn((n_seqs, hkv, W, D), generator=g, device=dev).to(torch.bfloat16),
                      torch.randn((n_seqs, hkv, W, D), generator=g, device=dev).to(torch.bfloat16))
    pos = np.random.default_rng(1006).integers(W, 8 * W, size=n_seqs)
    db = swa.Batch([1] * n_seqs, [int(p) for p in pos], list(range(n_seqs)))
    q = torch.randn((n_seqs, HQ, D), generator=g, device=dev).to(torch.bfloat16)
    o = torch.empty((n_seqs, HQ, D), dtype=torch.bfloat16, device=dev)
    wsb = swa.swa_decode_workspace_size(cache, n_seqs, HQ)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    t = time_ms(lambda: swa.swa_decode(cache, db, q, HQ, scale, o, ws, wsb), reps)
    kvb = n_seqs * 2 * hkv * D * 2 * W
    del cache
    return {"decode_g1_32seq_w4096": {"us": round(t * 1e3, 1), "gbps": round(kvb / t / 1e6, 1),
                                      "kv_bytes": kvb, "workspace_bytes": wsb}}


def suite_multilayer_ring(up, reps):
    """A 32-layer rolling cache for one 32768-token sequence: the rings of all layers are
    one [32][1][8][4096][128] tensor; every layer writes its 8 chunks of 4096 tokens.
    Device bytes are compared with a full 32K cache of the same layers (not allocated)."""
    import torch
    import sliding_window_gqa_swa_amd as swa
    dev = torch.device("cuda:0")
    L, N, C = 32, 32768, 4096
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(dev)
    kk = torch.empty((L, 1, HKV, W, D), dtype=torch.bfloat16, device=dev)
    vv = torch.empty((L, 1, HKV, W, D), dtype=torch.bfloat16, device=dev)
    ring_bytes = torch.cuda.memory_allocated(dev) - before
    full_bytes = 2 * L * N * HKV * D * 2
    caches = [swa.Cache(kk[layer], vv[layer]) for layer in range(L)]
    g = torch.Generator(device=dev).manual_seed(1007)
    kn = torch.randn((C, HKV, D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((C, HKV, D), generator=g, device=dev).to(torch.bfloat16)
    batches = [swa.Batch([C], [s], [0]) for s in range(0, N, C)]

    def all_writes():
        for c in caches:
            for b in batches:
                swa.swa_cache_write(c, b, kn, vn)

    t = time_ms(all_writes, max(1, reps // 5))
    del kk, vv, caches
    return {"multilayer_ring_32x32k": {
        "layers": L, "tokens": N, "ring_bytes": ring_bytes, "full_cache_bytes": full_bytes,
        "full_over_ring": round(full_bytes / ring_bytes, 3),
        "cache_writes_ms_all_layers_and_chunks": round(t, 3)}}


def decode_step_latency(dcache, positions, rows, dq, dk, dv, scale, reps: int, steps_per_graph: int = 16):
    """Per-token step time for small and full batches (the 64-sequence rings of
    the main step, full windows), and for 1 and 8 sequences at position 500
    (a context shorter than the window).  `eager_*`: back-to-back calls from
    Python, host launch cost included.  `graph_*`: `steps_per_graph`
    consecutive steps captured in one HIP graph, replay time / steps_per_graph
    -- the device-side step time.  Each form is cache write + decode as two
    calls, or the fused swa_decode_step."""
    import torch
    import sliding_window_gqa_swa_amd as swa
    dev = dq.device
    res = {}
    for n, short in ((1, False), (8, False), (64, False), (1, True), (8, True)):
        batch = swa.Batch([1] * n, [500] * n if short else positions[:n], rows[:n])
        q, k, v = dq[:n], dk[:n], dv[:n]
        out = torch.empty((n, HQ, D), dtype=torch.bfloat16, device=dev)
        nb = swa.swa_decode_workspace_size(dcache, n, HQ)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)

        def separate():
            swa.swa_cache_write(dcache, batch, k, v)
            swa.swa_decode(dcache, batch, q, HQ, scale, out, ws, nb)

        def fused():
            swa.swa_decode_step(dcache, batch, q, HQ, k, v, scale, out, ws, nb)

        rec = {}
        for name, fn in (("write_then_decode", separate), ("fused_step", fused)):
            rec["eager_" + name + "_us"] = round(time_ms(fn, reps) * 1e3, 1)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(steps_per_graph):
                    fn()
            rec["graph_" + name + "_us"] = round(time_ms(graph.replay, max(2, reps // steps_per_graph)) * 1e3
                                                 / steps_per_graph, 1)
            del graph
        res[f"batch_{n}" + ("_pos500" if short else "")] = rec
    return res


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-suite", action="store_true", help="skip the other workloads")
    ap.add_argument("--only", choices=["chunked", "mixed", "decode_g1", "write_vs_copy"],
                    help="run one suite workload alone and print its record (for profilers)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path would shard by sequence or KV head (decode) and by query range with a\n"
              "W-1 position halo (prefill), but no multi-GPU code is built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sliding_window_gqa_swa_amd as swa
    from sliding_window_gqa_swa_amd.workloads import batched_decode, mistral_prefill

    swa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    up = uploader(dev)
    scale = 1.0 / D ** 0.5

    def write_vs_copy():
        wp = mistral_prefill(1002, window=W, n=16384)
        n = wp.seqs[0].n_new
        pq, pk, pv = up(wp.q), up(wp.k_new), up(wp.v_new)
        pout = torch.empty((n, HQ, D), dtype=torch.bfloat16, device=dev)
        return suite_write_vs_copy(bf16_cache(1, HKV, W, dev), swa.Batch([n], [0], [0]), pq, pk, pv, pout,
                                   wp.scale, 50)

    if args.only:
        fn = {"chunked": lambda: suite_chunked(up, scale, 5, False),
              "mixed": lambda: suite_mixed(up, scale, 5, False),
              "decode_g1": lambda: suite_decode_g1(scale, 20),
              "write_vs_copy": write_vs_copy}[args.only]
        print(json.dumps({"only": args.only, **fn()}))
        return

    # ---- prefill workload (Mistral shape, 16K tokens, W = 4096)
    wp = mistral_prefill(1002, window=W, n=16384)
    n = wp.seqs[0].n_new
    pq, pk, pv = up(wp.q), up(wp.k_new), up(wp.v_new)
    pout = torch.empty((n, HQ, D), dtype=torch.bfloat16, device=dev)
    pcache = bf16_cache(1, HKV, W, dev)
    pbatch = swa.Batch([n], [0], [0])
    band_flops = 4.0 * D * HQ * band_pairs(0, n, W)
    pwrite_bytes = 2 * 2 * min(n, W) * HKV * D * 2

    # ---- decode workload (64 sequences, full rings)
    wd = batched_decode(1004)
    B = wd.num_seqs
    dcache = swa.Cache(torch.empty((B, HKV, W, D), dtype=torch.bfloat16, device=dev),
                       torch.empty((B, HKV, W, D), dtype=torch.bfloat16, device=dev))
    write_history(dcache, wd, up)
    dbatch = swa.Batch([1] * B, [s.start_pos for s in wd.seqs], wd.cache_idx)
    dq, dk, dv = up(wd.q), up(wd.k_new), up(wd.v_new)
    dout = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev)
    ws_bytes = swa.swa_decode_workspace_size(dcache, B, HQ)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    kv_bytes = sum(2 * HKV * D * 2 * min(s.start_pos + 1, W) for s in wd.seqs)
    dwrite_bytes = 2 * 2 * B * HKV * D * 2
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        swa.swa_prefill_chunk(pcache, pbatch, pq, HQ, pk, pv, wp.scale, pout)
        rec(1)
        swa.swa_cache_write(pcache, pbatch, pk, pv)
        rec(2)
        swa.swa_cache_write(dcache, dbatch, dk, dv)
        rec(3)
        swa.swa_decode(dcache, dbatch, dq, HQ, wd.scale, dout, ws, ws_bytes)
        rec(4)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    # untimed steps until the clock has settled, then the warm-up steps, then the timed ones
    settle_steps = settle(step, SETTLE_S)
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    part = np.zeros(4)
    for ev in events:
        for i in range(4):
            part[i] += ev[i].elapsed_time(ev[i + 1])
    part /= args.steps  # ms per launch
    t_pre, t_pw, t_dw, t_dec = part
    tflops = band_flops / (t_pre * 1e-3) / 1e12
    dec_gbps = kv_bytes / (t_dec * 1e-3) / 1e9

    traffic = pmc_traffic()
    sclk = sclk_estimate(t_pre, tflops)
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": SETTLE_S, "steps": settle_steps,
                   "why": "untimed steps before the warm-up: from idle the clock takes a few tens of ms of load to settle"},
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations rounded to bf16 (no weights, no dataset)",
        "config": {"workload": "mistral-shape SWA-GQA prefill 1x16384 W=4096 + chunk cache write "
                               "+ 64-sequence decode (W=4096 rings)",
                   "global_batch": 1, "seq_len": n, "window": W, "n_q_heads": HQ, "n_kv_heads": HKV,
                   "head_dim": D, "decode_batch": B, "parallelism": "single GPU"},
        "decode_kv_gbps": round(dec_gbps, 1),
        "parts_ms": {"prefill": round(t_pre, 4), "cache_write_chunk": round(t_pw, 4),
                     "cache_write_decode": round(t_dw, 4), "decode": round(t_dec, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": pmc_source() if traffic is not None else
                     "null: the prefill source changed since the committed counters were taken",
                     "kernel": PREFILL_KERNEL, "algorithmic_flops_per_launch": band_flops},
        "sclk": sclk,
        "decode_roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS,
                            "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                            "algorithmic_bytes_per_launch": kv_bytes},
        "cache_write_gbps": {"chunk": round(pwrite_bytes / (t_pw * 1e-3) / 1e9, 1),
                             "decode": round(dwrite_bytes / (t_dw * 1e-3) / 1e9, 1)},
        "pages_context": {"swa_vs_standard_speedup_at_16k_w4096": 2.0, "cache_memory_reduction_at_32k": 8.0,
                          "hardware": "not stated"},
    }
    cpu = not args.no_cpu_baseline
    if not args.no_suite:
        s = suite_causal_and_no_skip(pq, pk, pv, pout, wp.scale, t_pre, reps=10)
        s.update(suite_write_vs_copy(pcache, pbatch, pq, pk, pv, pout, wp.scale, reps=50))
        s.update(suite_chunked(up, scale, 10, cpu))
        s.update(suite_mixed(up, scale, 10, cpu))
        s.update(suite_decode_g1(scale, 20))
        s["decode_step_latency"] = decode_step_latency(
            dcache, [x.start_pos for x in wd.seqs], list(wd.cache_idx), dq, dk, dv, wd.scale, reps=50)
        del dcache, pcache
        s.update(suite_multilayer_ring(up, 10))
        result["suite"] = s
    if cpu:
        result["cpu_baseline"] = cpu_baseline_prefill(wp)
        result["cpu_baseline"]["gpu_over_cpu"] = round(tflops / result["cpu_baseline"]["value"], 1)
        result["cpu_baseline_other_configs"] = {"tiny_fp32": cpu_leg_tiny(), "decode_64seq": cpu_leg_decode(wd)}
        result["cpu_baseline_other_configs"]["decode_64seq"]["gpu_kv_gbps"] = round(dec_gbps, 1)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
