"""bench.py without a GPU: the one-GPU guard, and the committed HBM-counter
summaries matching the current kernel sources (the bench reports
roofline.traffic only from a summary taken from these sources)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


@pytest.mark.parametrize("kernel", ["ffn_gate_up_sel", "ffn_down_combine"])
def test_counter_summaries_match_the_sources(kernel):
    path = os.path.join(bench.PROFILES, f"{kernel}_decode1_counters.txt")
    assert os.path.exists(path), path
    t = bench.read_traffic(kernel, "decode1")
    assert t is not None, f"{path} was taken from other sources than the current ones; retake the counters"
    algo = {"ffn_gate_up_sel": 53534720, "ffn_down_combine": 26804224}[kernel]
    assert 0.99 * algo < t < 1.10 * algo


def test_source_hash_follows_the_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash("ffn_gate_up_sel")
    assert h == bench.kernel_source_hash("ffn_gate_up_sel") and len(h) == 16
    assert h != bench.kernel_source_hash("gather_cold")
    # a summary with another hash is not used
    (tmp_path / "ffn_gate_up_sel_decode1_counters.txt").write_text(
        "source_hash: 0000000000000000\ntraffic_bytes_per_launch: 1\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic("ffn_gate_up_sel", "decode1") is None
