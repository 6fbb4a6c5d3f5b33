"""bench.py's host-side contract, without a GPU: one GPU only, and counter-derived traffic
reported only while the committed counter summary was taken on the current kernel sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_use():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                      # no JSON line


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_recorded_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()     # deterministic
    f = tmp_path / "counters.md"
    f.write_text("# summary\n\n"
                 f"`traffic_bytes_per_launch dsa::k_a 1234 {h}`\n"
                 f"`traffic_bytes_per_launch dsa::k_b 99 {'0' * 64}`\n")
    monkeypatch.setattr(bench, "counter_file", lambda workload: str(f))
    assert bench.recorded_traffic("dsa::k_a", "w") == 1234          # taken on these sources
    assert bench.recorded_traffic("dsa::k_b", "w") is None          # stale: other sources
    assert bench.recorded_traffic("dsa::k_c", "w") is None          # not recorded
    monkeypatch.setattr(bench, "counter_file", lambda workload: str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("dsa::k_a", "w") is None


def test_committed_counter_summary_parses():
    """The committed summary of the decode step names the traffic of its kernels in the
    machine-readable form the bench reads."""
    path = bench.counter_file("decode_b4_mtp1_L65536")
    assert os.path.exists(path)
    rows = [l.strip().strip("`").split() for l in open(path)]
    rows = [r for r in rows if r and r[0] == "traffic_bytes_per_launch"]
    assert {r[1] for r in rows} >= {"dsa::indexer_stream_kernel", "dsa::sfa_kernel"}
    for r in rows:
        assert len(r) == 4 and int(r[2]) > 0 and len(r[3]) == 64
