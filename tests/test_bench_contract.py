"""The benchmark's command-line contract on the CPU: one GPU only, and the
counted-traffic guard (no GPU is touched by these tests)."""
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
import pytest  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    for argv in (["--gpus", "2"], ["--gpus", "8", "--steps", "1"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def test_world_size_above_one_exits():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_reported_only_for_counted_sources(monkeypatch):
    # with the device code the counters were taken on, every counted workload
    # reports bytes; any other key, or changed sources, report None
    if bench.kernel_sources_hash() != bench.TRAFFIC_SRC:
        assert all(bench.traffic_for(k) is None for k in bench.TRAFFIC)
        pytest.skip("device code changed since the counters were taken (traffic reads null)")
    for key in bench.TRAFFIC:
        assert bench.traffic_for(key) > 0
    assert bench.traffic_for(("decode-batch", 4)) is None
    assert bench.traffic_for(None) is None
    monkeypatch.setattr(bench, "TRAFFIC_SRC", "0" * 16)
    assert all(bench.traffic_for(k) is None for k in bench.TRAFFIC)
