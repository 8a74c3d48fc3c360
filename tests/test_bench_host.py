"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the
algorithmic work the roofline divides by, and the gate that retires HBM
traffic counters once a kernel source changes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("S,G,k,B", [(1, 1, 1, 1), (5, 2, 1, 1), (7, 3, 2, 2), (64, 8, 1, 3)])
def test_attention_flop_counts_visible_pairs(S, G, k, B):
    """4*d FLOP per visible (row, key) pair (two d-long products), counted by
    enumerating the causal pairs of every row set: G*k selected rows and the
    shared row per token."""
    cfg = synth.WORKLOADS["main_s2k"].replace(B=B, S=S, G=G, N=G * 2, k=k)
    pairs = 0
    for _b in range(B):
        for _rowset in range(G * k + 1):
            for s in range(S):
                pairs += sum(1 for key in range(S) if key <= s)
    assert bench.prefill_path_flops(cfg)["attention"] == 4 * cfg.d * pairs


def test_long_context_work_and_decode_bytes():
    # the 128k-token prefill's attention work and the 16 x 65536-key decode's KV bytes
    assert bench.prefill_path_flops(synth.WORKLOADS["long_s128k"])["attention"] == 19791360294912
    assert bench.decode_kv_bytes(synth.WORKLOADS["decode_kv64k"]) == 4 * 2 ** 30


def test_traffic_counters_retire_when_the_source_changes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    sha = bench.source_sha("prefill.hip")
    (tmp_path / "ok.txt").write_text(f"x\ntraffic_bytes_per_launch=12345 source_sha={sha}\n")
    (tmp_path / "stale.txt").write_text("x\ntraffic_bytes_per_launch=12345 source_sha=0000000000000000\n")
    assert bench.measured_traffic("prefill.hip", "ok.txt") == 12345
    assert bench.measured_traffic("prefill.hip", "stale.txt") is None
    assert bench.measured_traffic("prefill.hip", "missing.txt") is None
    # the hash covers the shared headers too, so it differs between kernel files
    assert bench.source_sha("prefill.hip") != bench.source_sha("decode.hip")
