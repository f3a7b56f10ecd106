"""Host-side checks of bench.py's contract (no GPU): one GPU only, and the recorded HBM
traffic is reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_keyed_to_the_kernel_sources(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        recs = json.load(f)
    assert recs
    for key, rec in recs.items():
        # the record's parts add up; it is reported exactly when it was taken on these sources
        assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
        current = rec["source_sha256"] == bench.source_digest(bench.KERNEL_SOURCES[key])
        assert bench.load_traffic(key) == (rec["bytes_per_launch"] if current else None)
    # a changed source (or a missing record) reports no traffic
    sources = {}
    for key, paths in bench.KERNEL_SOURCES.items():
        src = tmp_path / (key + ".hip")
        src.write_bytes(open(paths[0], "rb").read() + b"\n")
        sources[key] = [str(src)] + paths[1:]
    monkeypatch.setattr(bench, "KERNEL_SOURCES", sources)
    for key in recs:
        assert bench.load_traffic(key) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic("gemm_exact") is None


def test_settle_runs_whole_blocks_for_the_wall_time():
    """The untimed settle phase: nothing at 0 ms, whole blocks with a synchronization after
    each until the wall time has passed."""
    class FakeCuda:
        syncs = 0

        @classmethod
        def synchronize(cls):
            cls.syncs += 1

    class FakeTorch:
        cuda = FakeCuda

    calls = []
    assert bench.settle(FakeTorch, lambda: calls.append(1), 0.0) == 0 and not calls
    n = bench.settle(FakeTorch, lambda: calls.append(1), 5.0, block=7)
    assert n == len(calls) and n > 0 and n % 7 == 0 and FakeCuda.syncs == n // 7
