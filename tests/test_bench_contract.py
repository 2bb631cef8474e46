"""Host-side parts of the benchmark's contract (no GPU): the default workload
and timing settings, the link between the candidate GEMM's source and the
committed HBM-traffic summary that the bench line's `traffic` comes from, and
the refusal of more than one GPU."""

import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402


def test_defaults_name_the_largest_layer_and_the_timing_protocol(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert args.gpus == 1
    assert args.config == "70b-mlp"
    assert args.hbm_reps >= 10          # median of at least ten cache-evicted repetitions
    assert bench.FLUSH_BYTES >= 4 * 256 * 2 ** 20   # evicts the 256 MB last-level cache


def test_traffic_figure_belongs_to_the_current_gemm_source():
    """The committed summary carries the hash of gemm_sse.hip it was measured
    on; the bench reports its bytes only while the source still hashes to it."""
    got = bench.measured_traffic("70b-mlp:0")
    assert got is not None, "profiles/hbm_traffic_70b-mlp.md no longer matches gemm_sse.hip"
    assert 0.5e9 < got < 1e10
    assert bench.measured_traffic("no-such-layer:0") is None


def test_traffic_is_dropped_when_the_source_changes(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("70b-mlp:0") is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
