"""Host-side checks of bench.py (no GPU): the one-GPU guard, the visible-pair count behind
the attention flops, the roofline arithmetic and the committed counter summaries."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("L", [1, 7, 64, 131])
@pytest.mark.parametrize("mask,window", [(0, 0), (1, 0), (2, 1), (2, 5), (2, 64), (2, 1000)])
def test_allowed_pairs_counts_the_visible_pairs(L, mask, window):
    i = np.arange(L)[:, None]
    k = np.arange(L)[None, :]
    if mask == 0:
        vis = np.ones((L, L), bool)
    elif mask == 1:
        vis = k <= i
    else:
        vis = (k <= i) & (k > i - window)
    assert bench.allowed_pairs(L, mask, window) == int(vis.sum())


def test_roofline_fields():
    r = bench.roof("mfma", 2.5e12, 2.0)   # 2.5 TFLOP in 2 ms
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1250.0) and r["frac"] == pytest.approx(0.5)
    h = bench.roof("hbm", 8e9, 2.0)       # 8 GB in 2 ms
    assert h["bound"] == "hbm" and h["unit"] == "GB/s"
    assert h["achieved"] == pytest.approx(4000.0) and h["frac"] == pytest.approx(0.5)


def test_counter_summaries_parse():
    for w in ["iha_window_p2_b4_n4096", "iha_window_p4_b2_n8192_wide"]:
        for step in ["prep", "gemm", "attention", "collapse"]:
            t = bench.counter_traffic(w, step)
            assert t is None or (isinstance(t, int) and t > 0)
    assert bench.counter_traffic("no_such_workload", "gemm") is None
