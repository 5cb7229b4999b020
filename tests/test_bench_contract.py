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
    # reports bytes and names its source; any other key, or changed sources,
    # report None with the reason
    if bench.kernel_sources_hash() != bench.TRAFFIC_SRC:
        for k in bench.TRAFFIC:
            b, why = bench.traffic_for(k)
            assert b is None and why.startswith("stale")
        pytest.skip("device code changed since the counters were taken (traffic reads null)")
    for key in bench.TRAFFIC:
        b, src = bench.traffic_for(key)
        assert b > 0 and src == bench.TRAFFIC_DOC
    assert bench.traffic_for(("decode-batch", 4))[0] is None
    assert bench.traffic_for(None)[0] is None
    monkeypatch.setattr(bench, "TRAFFIC_SRC", "0" * 16)
    assert all(bench.traffic_for(k)[0] is None for k in bench.TRAFFIC)


def test_host_info_threads_follow_affinity_and_omp(monkeypatch):
    aff = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    info, threads = bench.host_info()
    assert threads == aff and info["affinity_cpus"] == aff and info["nproc"] == os.cpu_count()
    assert info["OMP_NUM_THREADS"] is None
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    info, threads = bench.host_info()
    assert threads == 1 and info["OMP_NUM_THREADS"] == "1"
