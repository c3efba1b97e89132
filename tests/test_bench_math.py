"""CPU tier: the measurement arithmetic bench.py reports -- algorithmic flops,
compulsory bytes, and the attainable rate min(MFMA peak, intensity x HBM
rate) -- against hand counts and the Zipf batch's totals."""
import numpy as np
import pytest

import bench
import workloads


def test_algorithmic_flops_hand_counts():
    lengths = np.array([3, 1, 2])
    # 4 * (9 + 1 + 4) * H * D; causal halves it; first-token: one query per
    # sequence sees all its keys (non-causal) or one key (causal)
    assert bench.algorithmic_flops(lengths, 2, 16, False) == 4 * 14 * 2 * 16
    assert bench.algorithmic_flops(lengths, 2, 16, True) == 4 * 14 * 2 * 16 / 2
    assert bench.algorithmic_flops(lengths, 2, 16, False, first_token=True) == 4 * 6 * 2 * 16
    assert bench.algorithmic_flops(lengths, 2, 16, True, first_token=True) == 4 * 3 * 2 * 16


def test_compulsory_bytes_hand_count():
    # q and out: 5 rows; k and v: 7 rows; H = 2, D = 8, 2-byte elements; lse 4 bytes per (row, head)
    assert bench.compulsory_bytes(5, 7, 2, 8, 2) == (2 * 5 + 2 * 7) * 2 * 8 * 2 + 4 * 5 * 2


def test_zipf_batch_totals():
    wl = workloads.make_workload(workloads.WORKLOAD_NAMES["zipf"])
    flops = bench.workload_flops(wl, wl.heads)
    assert round(flops / 1e9, 3) == 1271.756
    nbytes = bench.compulsory_bytes(wl.total_tokens, wl.total_tokens, wl.heads, wl.head_dim, 2)
    assert round(nbytes / 1e9, 4) == 1.0779


def test_cross_flops_use_both_lengths():
    wl = workloads.make_workload(workloads.WORKLOAD_NAMES["cross"])
    lq = wl.query_lengths().astype(np.float64)
    lk = wl.lengths.astype(np.float64)
    assert bench.workload_flops(wl, wl.heads) == pytest.approx(4 * float(np.sum(lq * lk)) * wl.heads * wl.head_dim)


def test_attainable_on_both_sides_of_the_ridge():
    peaks = {"mfma_tflops": 2000.0, "copy_gbs": 5000.0}
    # intensity 1,000 flop/B: above the ridge (2,500 / 8 = 312.5), so the MFMA peak bounds it
    a = bench.attainable(1e12, 1e9, 1000.0, 2500.0, peaks)
    assert a["ai_flop_per_byte"] == 1000.0 and a["datasheet_tflops"] == 2500.0 and a["frac"] == 0.4
    assert a["measured_tflops"] == 2000.0 and a["frac_measured"] == 0.5
    # intensity 100 flop/B: below the ridge, bandwidth-bound: 100 x 8 TB/s = 800 TFLOP/s
    b = bench.attainable(1e11, 1e9, 400.0, 2500.0, peaks)
    assert b["datasheet_tflops"] == 800.0 and b["frac"] == 0.5
    assert b["measured_tflops"] == 500.0 and b["frac_measured"] == 0.8
    assert "measured_tflops" not in bench.attainable(1e11, 1e9, 400.0, 2500.0, None)


def test_bench_refuses_more_than_one_gpu():
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
