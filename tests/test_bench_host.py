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


def test_hbm_model_reproduces_the_committed_traffic_records():
    """bench.hbm_model_bytes gives the compulsory and tiled-model counts that the
    committed counter records state for the long-context workload, and the
    tiled model grows linearly in N at a fixed token count (Theorem 2 with
    fixed block rows) while the compulsory count stays constant."""
    import bench
    m = bench.hbm_model_bytes(1, 12, 8192, 64, 2, True)
    for kernel, key in (("fwd_kernel", "fwd"), ("bwd_grad_kernel", "grad")):
        kv = {}
        with open(bench.traffic_file(kernel)) as f:
            for line in f:
                if ":" in line and not line.lstrip().startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        assert int(kv["compulsory_bytes_per_launch"]) == m[f"{key}_compulsory"]
        assert int(kv["tiled_model_bytes_per_launch"]) == m[f"{key}_tiled_model"]
    a = bench.hbm_model_bytes(8, 12, 2048, 64, 2, True)
    b = bench.hbm_model_bytes(4, 12, 4096, 64, 2, True)
    assert a["fwd_compulsory"] == b["fwd_compulsory"]
    reread_a = a["fwd_tiled_model"] - a["fwd_compulsory"]
    reread_b = b["fwd_tiled_model"] - b["fwd_compulsory"]
    # block pairs beyond the first read, per head (nb^2/2 - nb with nb = N/128),
    # times heads: 112 * 96 at N = 2048, 480 * 48 at N = 4096
    assert reread_a * 480 * 48 == reread_b * 112 * 96


def test_warm_up_runs_exactly_w_steps_when_given_else_until_time_and_ten_steps(monkeypatch):
    calls = {"step": 0, "sync": 0}

    def step():
        calls["step"] += 1

    def sync():
        calls["sync"] += 1

    assert bench.warm_up(step, 3, sync) == 3 and calls["step"] == 3
    assert bench.warm_up(step, 0, sync) == 0 and calls["step"] == 3
    # Default: whole groups of ten, synchronised, until both 10 steps and WARM_SECONDS have passed.
    monkeypatch.setattr(bench, "WARM_SECONDS", 0.0)
    calls["step"] = 0
    assert bench.warm_up(step, None, sync) == 10 and calls["step"] == 10
    clock = iter([0.0, 0.1, 0.2, 0.35, 0.6])
    monkeypatch.setattr(bench, "WARM_SECONDS", 0.3)
    monkeypatch.setattr(bench.time, "time", lambda: next(clock))
    calls["step"] = 0
    n = bench.warm_up(step, None, sync)
    assert n == calls["step"] == 30  # t = 0.1, 0.2 after the first two groups, 0.35 >= 0.3 after the third
