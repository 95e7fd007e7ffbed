"""Host-side behaviour of bench.py that needs no GPU."""
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
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_is_used_only_while_its_source_hash_matches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda k: str(tmp_path / f"{k}.txt"))
    k = "bwd_grad_kernel"
    assert bench.recorded_traffic(k) is None          # no record
    good = bench.kernel_source_hash(k)
    (tmp_path / f"{k}.txt").write_text(f"# comment: 1\nsource_sha256: {good}\ntraffic_bytes_per_launch: 12345\n")
    assert bench.recorded_traffic(k) == 12345.0
    (tmp_path / f"{k}.txt").write_text("source_sha256: 00\ntraffic_bytes_per_launch: 12345\n")
    assert bench.recorded_traffic(k) is None          # kernel source changed since the counters


def test_committed_traffic_records_name_their_kernel_and_commands():
    for k in bench.KERNELS:
        path = os.path.join(ROOT, "profiles", f"{k}_gpt2_long_traffic.txt")
        assert os.path.exists(path), path
        text = open(path).read()
        assert f"kernel: {k}" in text
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
        kv = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith("#"))
        assert float(kv["traffic_bytes_per_launch"]) > float(kv["compulsory_bytes_per_launch"]) > 0
