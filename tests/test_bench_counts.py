"""CPU checks of the benchmark's work counts against brute force on small
shapes: the exact visible (query, key) pairs behind the FLOP and exp2
counts, and the accumulate mode's dQ partial-add bytes."""
import numpy as np
import pytest

import bench
import workloads as W


def _visible(lq, lk, causal, window):
    i = np.arange(lq)[:, None] + (lk - lq)
    j = np.arange(lk)[None, :]
    left, right = window if window is not None else (-1, -1)
    if causal:
        right = 0 if right < 0 else min(right, 0)
    vis = np.ones((lq, lk), bool)
    if right >= 0:
        vis &= j <= i + right
    if left >= 0:
        vis &= j >= i - left
    return vis


CASES = [(300, 300, True, None), (130, 700, True, None), (700, 130, True, None),
         (256, 256, False, None), (500, 500, True, (100, 0)), (260, 400, False, (40, 30)),
         (64, 64, True, (0, 0))]


@pytest.mark.parametrize("lq,lk,causal,window", CASES)
def test_exact_pairs_are_the_visible_pairs(lq, lk, causal, window):
    assert bench.exact_pairs(lq, lk, causal, window) == _visible(lq, lk, causal, window).sum()


@pytest.mark.parametrize("lq,lk,causal,window", CASES)
def test_dq_add_bytes_by_brute_force(lq, lk, causal, window):
    """A 128-key tile adds a 64-row query tile's partial (valid rows x
    head_dim fp32) iff some pair of the two tiles is visible."""
    vis = _visible(lq, lk, causal, window)
    rows = 0
    for n0 in range(0, lk, 128):
        for q0 in range(0, lq, 64):
            if vis[q0:q0 + 64, n0:n0 + 128].any():
                rows += min(64, lq - q0)
    wl = W.custom("t", 1, 3, 1, lq, lk, 96, causal, seed=1, window=window)
    assert bench.dq_add_bytes(wl, [lq], [lk]) == rows * 3 * 96 * 4


def test_tile_kernel_hbm_rates_follow_the_committed_profile(monkeypatch):
    """The default line's per-kernel HBM GB/s: counter bytes of the committed
    profile over the kernel times at the headline, none elsewhere, and none
    for a kernel whose sources changed since the profile."""
    kms = {"main": 0.5, "dq": 0.4}
    assert bench.tile_kernel_GBs(kms, False) == {}
    monkeypatch.setattr(bench, "committed_traffic", lambda: 5.0e8)
    monkeypatch.setattr(bench, "committed_dq_traffic", lambda: 4.0e8)
    assert bench.tile_kernel_GBs(kms, True) == {"main": 1000.0, "dq": 1000.0}
    monkeypatch.setattr(bench, "committed_dq_traffic", lambda: None)
    assert bench.tile_kernel_GBs(kms, True) == {"main": 1000.0}


def test_metric_labels_name_each_workload():
    """The headline keeps the metric label it is quoted on; the other
    workloads' lines name their own shape."""
    assert bench.metric_name(bench.METRIC, W.WORKLOADS[3]) == bench.METRIC
    labels = {c: bench.metric_name(bench.METRIC, W.WORKLOADS[c]) for c in (1, 2, 4, 5)}
    assert labels[1].endswith("S=128 D=64 non-causal MHA")
    assert labels[2].endswith("S=1024 D=64 causal MHA")
    assert labels[4].endswith("Sq=2048 Sk=8192 D=128 causal GQA")
    assert "16 seqs" in labels[5] and labels[5].endswith("D=96 causal MHA")
