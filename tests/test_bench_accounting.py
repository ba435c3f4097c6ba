"""Useful-FLOP accounting of bench.py against the oracle's mask (CPU only)."""
import numpy as np
import pytest

import bench
import oracle
import workloads


@pytest.mark.parametrize("lq,lk,causal,window", [
    (50, 50, False, 0), (50, 50, True, 0), (30, 70, True, 0), (70, 30, True, 0),
    (300, 300, True, 17), (40, 200, True, 64), (1, 1, True, 1)])
def test_visible_pairs_match_oracle_mask(lq, lk, causal, window):
    got = bench.visible_pairs_per_row(lq, lk, causal, window)
    assert np.array_equal(got, oracle.visible_counts(lq, lk, causal, window))


def test_workload_useful_flops():
    w = workloads.GQA_CAUSAL_BF16
    pairs = bench.useful_pairs(w)
    assert pairs == 989_633_984
    assert bench.useful_flops(w) == pytest.approx(5.067e11, rel=1e-3)
    assert bench.useful_pairs(workloads.SWA_BF16) == 58_722_304 * 4 * 32
    assert bench.useful_pairs(workloads.TINY_F32) == 2 * (17 ** 2 + 64 ** 2 + 129 ** 2)
    assert bench.useful_flops(workloads.MLA_BF16) == bench.useful_pairs(workloads.MLA_BF16) * 640


def test_bias_pairs_count_only_finite_entries():
    w = workloads.dense_f16(64, False, bias=True).with_(seqlens_q=(3000, 1500),
                                                        seqlens_kv=(3000, 1500))
    bias = workloads.prefix_lm_bias(w.seqlens_q, 1024)
    expect = sum(int(np.maximum(1024, np.arange(L) + 1).clip(max=L).sum()) for L in w.seqlens_q)
    assert bench.useful_pairs(w, bias) == expect * w.hq


def test_multi_gpu_request_exits_with_message():
    import subprocess, sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_window_override_is_refused_for_windowless_workloads():
    """--window only applies to a sliding-window workload; elsewhere bench.py
    exits with status 2 before it does any work."""
    import subprocess, sys, os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--workload", "gqa_causal_bf16",
                        "--window", "64"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--window" in r.stderr


def test_window_override_changes_the_accounting():
    w = workloads.SWA_BF16.with_(window=1024)
    assert bench.useful_pairs(w) < bench.useful_pairs(workloads.SWA_BF16)
    # each 16384-token causal sequence with W keys per row: W*(W+1)/2 + (L-W)*W per head
    L, W = 16384, 1024
    assert bench.useful_pairs(w) == 4 * 32 * (W * (W + 1) // 2 + (L - W) * W)
