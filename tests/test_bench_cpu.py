"""Host logic of bench.py and the workload generators (no GPU): the FLOP counts behind the
metric, the window's pair count against the oracle's mask, the traffic-figure bookkeeping, and
the one-GPU contract."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_flop_count():
    """10 B H Sq Sk D, halved for the causal mask: the metric's own formula."""
    w = workloads.get(workloads.HEADLINE)
    assert (w.B, w.H, w.H_kv, w.Sq, w.Sk, w.D, w.causal, w.dtype) == (2, 32, 8, 4096, 4096, 128, True, "bf16")
    assert w.bwd_flops() == 10 * 2 * 32 * 4096 * 4096 * 128 / 2
    assert bench.allowed_pairs(w) == 2 * 32 * 4096 * 4096 / 2


@pytest.mark.parametrize("causal,window,Sq,Sk", [(True, 5, 37, 37), (False, 5, 30, 44),
                                                 (True, 16, 70, 20), (False, 3, 50, 9)])
def test_window_pair_count_matches_the_oracle_mask(causal, window, Sq, Sk):
    w = workloads.Workload("t", "bf16", 2, 3, 1, Sq, Sk, 64, causal, seed=0, window=window)
    n = int(oracle.allowed_mask(np.arange(Sq), Sk, causal, window).sum())
    assert w.allowed_pairs() == 2 * 3 * n


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    for f in ("bwd16.hip", "common.h", "launch.h"):
        shutil.copy(os.path.join(bench.CSRC, f), tmp_path / f)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    d0 = bench.source_digest("bwd_dkdv")
    with open(tmp_path / "bwd16.hip", "a") as fh:
        fh.write("\n// a comment\n\n")
    assert bench.source_digest("bwd_dkdv") == d0
    with open(tmp_path / "bwd16.hip", "a") as fh:
        fh.write("static int unused_symbol;\n")
    assert bench.source_digest("bwd_dkdv") != d0


def test_recorded_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    name = workloads.HEADLINE
    path = tmp_path / f"bwd_dkdv_{name}_hbm_traffic.md"
    path.write_text(f"source_digest: {bench.source_digest('bwd_dkdv')}\nhbm_bytes_per_launch: 1.5e8\n")
    assert bench.recorded_traffic("bwd_dkdv", name) == 1.5e8
    path.write_text("source_digest: 0000000000000000\nhbm_bytes_per_launch: 1.5e8\n")
    assert bench.recorded_traffic("bwd_dkdv", name) is None
    assert bench.recorded_traffic("bwd_dq", name) is None  # no file


def test_inputs_are_seeded_and_rounded():
    torch = pytest.importorskip("torch")
    w = workloads.Workload("t", "bf16", 1, 2, 1, 9, 7, 64, True, seed=123, do_std=0.1)
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    assert [tuple(x.shape) for x in a] == [(1, 2, 9, 64), (1, 1, 7, 64), (1, 1, 7, 64), (1, 2, 9, 64)]
    assert all(x.dtype == torch.bfloat16 and x.is_contiguous() for x in a)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert float(a[3].float().std()) < 0.2 < float(a[0].float().std())  # dO scaled by do_std


def test_call_stats():
    s = bench.call_stats([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s == {"calls": 5, "median": 3.0, "min": 1.0, "p90": 4.6}
    s = bench.call_stats([float(i) for i in range(1, 21)])  # 1..20
    assert s["median"] == 10.5 and s["min"] == 1.0 and abs(s["p90"] - 18.1) < 1e-9
