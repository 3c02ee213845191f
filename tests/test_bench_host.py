"""Host logic of bench.py (no GPU): the algorithmic byte counts behind every
GB/s figure, on the workloads' own tables, against the sizes stated for
them; the traffic value that follows the step kernel's source hash; and the
refusal to run on more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_step_bytes():
    """decode workload (seed 1002): 124,503 tokens in 7,815 pages; the
    dequant moves 653,423,260 bytes, the 64-row append 336,384"""
    old, new_len, indices, indptr, last, bt = W.decode_append_tables(np.random.default_rng(1002), 64, 4096, 20000, 16)
    assert int(new_len.sum()) == 124503 and int(((new_len + 15) // 16).sum()) == 7815
    assert bench.dequant_bytes(new_len, 16, 8, 128, 4) == 653423260
    # per row and head: 2 B x 128 in, 64 + 8 out, for K and V; 8 B of indices per row
    assert bench.append_bytes(64, 8, 128) == 64 * (2 * 8 * (256 + 64 + 8) + 8) == 336384


def test_materialize_and_attention_bytes():
    """materialize workload (seed 1004): 12,070 active pages, 618,161,868
    bytes; decode attention over the decode cache with 32 query heads:
    144,507,548 bytes"""
    lens, P, maxp, bt, indptr = W.materialize_tables(np.random.default_rng(1004), 32, 128, 32768, 16)
    assert int(((lens + 15) // 16).sum()) == 12070
    assert bench.materialize_bytes(lens, 16, 8, 128, 32) == 618161868
    old, new_len, *_ = W.decode_append_tables(np.random.default_rng(1002), 64, 4096, 20000, 16)
    assert bench.attention_bytes(new_len, 16, 8, 128, 32) == 144507548


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    summary = tmp_path / "counters.md"
    summary.write_text(f"traffic_bytes_per_launch = 123\nsource_sha256 = {bench.dequant_source_hash()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.recorded_traffic() == 123
    summary.write_text("traffic_bytes_per_launch = 123\nsource_sha256 = " + "0" * 64 + "\n")
    assert bench.recorded_traffic() is None                  # sources changed since the counters
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic() is None


def test_committed_traffic_matches_the_sources():
    """the committed counter summary was taken on the step kernel's current
    sources, so the benchmark reports its traffic"""
    assert bench.recorded_traffic() is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
