"""CPU checks of the algorithmic work bench.py divides by: the band's
(query, key) pair count, the prefill FLOPs it reports, the decode's K/V bytes
and the committed counter record it reads traffic and the clock from.

Band of query i (Mistral 7B (Chinese translation), section 2, paragraph
"Sliding Window Attention"): keys j with i - W < j <= i and j >= 0.
"""
import json
import os

import numpy as np

import bench


def brute_pairs(start, n, window):
    i = np.arange(start, start + n)[:, None]
    j = np.arange(0, start + n)[None, :]
    return int(((j <= i) & (j > i - window)).sum())


def test_band_pairs_equals_brute_force_count():
    for start, n, window in [(0, 1, 1), (0, 64, 8), (0, 200, 64), (100, 77, 64), (5000, 300, 4096),
                             (0, 300, 4096), (4095, 3, 4096), (30, 40, 1)]:
        assert bench.band_pairs(start, n, window) == brute_pairs(start, n, window), (start, n, window)


def test_band_pairs_closed_form_at_the_bench_shape():
    # n >= W from position 0: a triangle of W rows, then W keys for each later row
    n, w = 16384, 4096
    assert bench.band_pairs(0, n, w) == w * (w + 1) // 2 + (n - w) * w == 58_722_304
    # causal attention (W >= n) counts the whole triangle
    assert bench.band_pairs(0, n, n) == n * (n + 1) // 2


def test_prefill_flops_of_the_headline():
    # 2 FLOPs per multiply-add, two products (Q K^T and P V) of D each, per head and band pair
    flops = 4.0 * bench.D * bench.HQ * bench.band_pairs(0, 16384, bench.W)
    assert flops == 962_106_228_736.0
    assert bench.HQ == 32 and bench.HKV == 8 and bench.D == 128 and bench.W == 4096


def test_committed_counter_record_is_consistent():
    rec = json.load(open(bench.PMC_FILE))
    cal = rec["copy_calibration"]
    assert abs(cal["fetch_factor"] - cal["bytes_each_way_kib"] / cal["fetch_kib"]) < 1e-9
    assert abs(cal["write_factor"] - cal["bytes_each_way_kib"] / cal["write_kib"]) < 1e-9
    traffic = 1024 * (rec["fetch_kib_per_dispatch"] * cal["fetch_factor"] +
                      rec["write_kib_per_dispatch"] * cal["write_factor"])
    assert abs(traffic - rec["traffic_bytes_per_launch"]) < 1.0
    alg = rec["algorithmic_bytes_per_launch"]
    # Q, K, V read and O written once: (32 + 8 + 8) heads read and 32 written, 16384 rows of 256 B
    assert alg["read_q_k_v"] == 16384 * (32 + 8 + 8) * 128 * 2
    assert alg["write_out"] == 16384 * 32 * 128 * 2
    assert rec["cycles_per_xcd_per_launch"] == rec["gui_active_cycles_per_launch"] / 8
    # the record belongs to the prefill source in the tree (bench.py reports it only then)
    assert bench.pmc_record() is not None, "profiles/ counter record was taken on another prefill source"
    assert bench.pmc_traffic() == rec["traffic_bytes_per_launch"]


def test_sclk_estimate_from_cycles_and_time():
    rec = bench.pmc_record()
    t_ms = 0.75
    s = bench.sclk_estimate(t_ms, 1282.8)
    assert abs(s["ghz"] - round(rec["cycles_per_xcd_per_launch"] / (t_ms * 1e6), 3)) < 1e-9
    assert abs(s["mfma_peak_at_sclk_tflops"] - round(2500.0 * s["ghz"] / 2.4, 1)) < 0.2
