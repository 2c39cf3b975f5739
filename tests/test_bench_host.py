"""Host logic of bench.py (no GPU): the HBM traffic it reports comes only from a counter
summary taken on the kernel's current sources with the same launches per step."""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _setup(tmp_path, src_text):
    csrc = tmp_path / "dynamic_sparse_attention_rank_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text(src_text)
    sha = hashlib.sha256(src_text.encode()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_counters_w.txt").write_text(
        "# summary\n\nkernel: kern\nlaunches_per_step: 12\nsources: k.hip\n"
        f"sources_sha256: {sha}\nfetch_bytes_per_launch: 1000\nwrite_bytes_per_launch: 24\n")
    return csrc


def test_counter_traffic_needs_same_sources_and_launches(tmp_path, monkeypatch):
    csrc = _setup(tmp_path, "kernel source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("kern", "w", 12) == 1024.0
    assert bench.counter_traffic("kern", "w", 8) is None          # another split of the work
    assert bench.counter_traffic("other", "w", 12) is None        # no entry for the kernel
    assert bench.counter_traffic("kern", "missing", 12) is None   # no summary for the workload
    (csrc / "k.hip").write_text("kernel source, changed\n")
    assert bench.counter_traffic("kern", "w", 12) is None         # sources changed since
