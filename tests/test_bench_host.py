"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the counter
summary lookup (null traffic when the summary was taken on other kernel
sources), and the time-budgeted CPU baseline."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = bench.kernel_sources_sha256()
    (prof / "mla_split_kernel.wl.traffic.txt").write_text(
        f"# header\nkernel_sources_sha256: {good}\ntraffic_bytes_per_launch: 1234\n"
        "combine_read_bytes_per_launch: 10\ncombine_write_bytes_per_launch: 5\n")
    (prof / "mla_split_kernel.old.traffic.txt").write_text(
        "kernel_sources_sha256: 0000\ntraffic_bytes_per_launch: 99\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hash itself is computed from the real sources
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: good)
    assert bench.measured_traffic("wl") == 1234
    assert bench.measured_traffic("wl", whole_call=True) == 1249
    assert bench.measured_traffic("old") is None
    assert bench.measured_traffic("missing") is None


def test_cpu_baseline_reports_a_bounded_sample():
    from mla_synth import generate, ragged
    inp = generate("tiny")
    r = bench.cpu_baseline(inp, 0.05)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1 and r["seconds"] < 5
    rg = ragged(inp, q_lens=[1, 0])
    assert bench.cpu_baseline(inp, 0.05, rg)["value"] > 0
