"""bench.py's host logic on the CPU: the one-GPU refusal and the counted-traffic
record (returned only for its workload and while the kernel sources match the
digest taken with the counters)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "only one GPU is measured" in r.stderr
    assert r.stdout == ""


def _record(tmp_path, srcs, workload="w1", nbytes=123456):
    h = __import__("hashlib").sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    rec = {"workload": workload, "bytes_per_launch": nbytes, "source_sha256": h.hexdigest()}
    p = tmp_path / "profile.md"
    p.write_text("# summary\n\ntraffic: " + json.dumps(rec) + "\n")
    return str(p)


def test_counted_traffic_follows_workload_and_source_digest(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(src)])
    monkeypatch.setattr(bench, "PROFILE", _record(tmp_path, [str(src)]))
    assert bench.counted_traffic("w1") == 123456
    assert bench.counted_traffic("w2") is None          # another workload
    src.write_text("// kernel v2\n")                     # the kernel changed since the counters
    assert bench.counted_traffic("w1") is None
    monkeypatch.setattr(bench, "PROFILE", str(tmp_path / "missing.md"))
    assert bench.counted_traffic("w1") is None


def test_committed_traffic_record_is_near_the_algorithmic_bytes():
    # when the committed record matches the sources, it counts the weights,
    # activations and logits about once (the kernel streams W2 exactly once)
    got = bench.counted_traffic("vicuna7b_b1")
    if got is None:
        pytest.skip("kernel sources changed since the counters were taken")
    alg = 4 * 32000 * 4096 * 2 + 4 * 4096 * 2 + 4 * 32000 * 4
    assert 1.0 <= got / alg < 1.02
