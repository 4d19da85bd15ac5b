"""Host-side parts of bench.py: the one-GPU guard, the CPU oracle baseline and the
traffic figure's tie to the GEMM source (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_cpu_baseline_repeats_whole_passes():
    import bench
    from workloads import generate, get_config, small_variant
    cfg = small_variant(get_config("tiny_f32"), 32)
    inp = generate(cfg, "cpu")
    rec = bench.cpu_baseline(cfg, inp, 32, min_seconds=0.3)
    assert rec["kind"] == "oracle"
    assert rec["passes"] >= 1 and rec["seconds"] >= 0.3
    assert rec["value"] == pytest.approx(32 * rec["passes"] / rec["seconds"])
    assert f"{rec['passes']} pass" in rec["sample"]
    for key in ("cores", "host_cpus", "blas", "cpu_model", "unit"):
        assert key in rec


def test_traffic_figure_follows_the_gemm_source(monkeypatch):
    """The committed counter figure is reported only for the GEMM source it was taken on."""
    import bench
    entries = json.load(open(bench.TRAFFIC_FILE))
    assert entries
    for name, e in entries.items():
        assert e["traffic_bytes"] > 0 and e["algorithmic_bytes"] > 0
        monkeypatch.setattr(bench, "source_sha", lambda sha=e["gemm_source_sha"]: sha)
        assert bench.load_traffic(name) == e["traffic_bytes"]
        monkeypatch.setattr(bench, "source_sha", lambda: "0" * 16)
        assert bench.load_traffic(name) is None
    assert bench.load_traffic("no_such_workload") is None
