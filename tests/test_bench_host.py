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
    (prof / "counters_w.txt").write_text(
        "# summary\n\nkernel: kern\nlaunches_per_step: 12\nsources: k.hip\n"
        f"sources_sha256: {sha}\nfetch_bytes_per_launch: 1000\nwrite_bytes_per_launch: 24\n"
        "l2_hit_pct: 71.5\n")
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


def test_counter_summary_carries_the_other_counters(tmp_path, monkeypatch):
    _setup(tmp_path, "kernel source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    v = bench.counter_summary("kern", "w", 12)
    assert float(v["l2_hit_pct"]) == 71.5


def test_rooflines_of_the_mid_workload():
    """The selection's roofline at S=64K (Q_lr, K_lr read once, idx written once: 845.6 MB at
    8 TB/s = 0.106 ms) and the attention FLOPs per edge (4 G d forward, 10 G d backward)."""
    from synth import CONFIGS
    cfg = CONFIGS["mid"]
    ks = [6554] * 24
    tk = bench.topk_roofline(cfg, ks)
    assert tk["bound"] == "hbm" and abs(tk["bytes"] - 845.6e6) < 0.1e6
    assert abs(tk["ms"] - 0.1057) < 1e-3
    f_fwd, f_bwd, fd_fwd, _ = bench.flops(cfg, ks)
    E = bench.n_edges(cfg, ks)
    assert E == 1024 * 6554 * 24
    assert f_fwd == 4 * 64 * 128 * E and f_bwd == 10 * 64 * 128 * E
    assert abs(fd_fwd / f_fwd - 65536 / 6554) < 1e-9
