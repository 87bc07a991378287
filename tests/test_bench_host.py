"""bench.py without a GPU: the one-GPU guard, and the committed HBM-counter
summaries (the bench reports roofline.traffic only from a summary taken from
the current kernel sources)."""
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
def test_counter_summaries_are_used_only_for_their_sources(kernel):
    """A summary is used only while its source hash matches the kernel's
    current sources; then its traffic is within 10% of the algorithmic bytes.
    Taken from other sources, the bench reports traffic as null."""
    path = os.path.join(bench.PROFILES, f"{kernel}_decode1_counters.txt")
    assert os.path.exists(path), path
    kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
    t = bench.read_traffic(kernel, "decode1")
    if kv["source_hash"].strip() != bench.kernel_source_hash(kernel):
        assert t is None
        return
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
