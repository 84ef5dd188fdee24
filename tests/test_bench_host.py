"""Host-side checks of bench.py (no GPU): the one-GPU contract and the rule that a
profiled traffic figure is reported only while the kernel's sources are the ones the
counters were taken with."""
import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_profiled_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    import bench
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "state_space_model_ssm_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_bytes(b"kernel source, first version")
    (csrc / "common.hpp").write_bytes(b"shared header")
    sha = hashlib.sha256(b"kernel source, first version" + b"shared header").hexdigest()[:16]
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel": "k", "bytes_per_launch": 1234, "fetch": 1000, "write": 234, "src_sha": sha,
           "sources": ["k.hip", "common.hpp"]}
    (prof / "k_workload.md").write_text("# k\n\nsome table\n\ntraffic-json: " + json.dumps(rec) + "\n")
    assert bench.profiled_traffic("k") == 1234
    assert bench.profiled_traffic("another_kernel") is None
    (csrc / "common.hpp").write_bytes(b"shared header, edited")
    assert bench.profiled_traffic("k") is None  # a source changed since the counters
    (csrc / "common.hpp").unlink()
    assert bench.profiled_traffic("k") is None  # a source is gone
