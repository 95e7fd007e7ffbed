"""The XCD placement arithmetic (csrc/fa_place.h) on the host: every workgroup
of a launch maps to a distinct (head, block level) inside the launch, for
every head count 1..80 and level count 1..72, with and without the CU-pairing
reversal.  The kernels index their buffers with these values, so this is the
bounds check of the launch geometry."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_placement_is_a_bijection_onto_each_launch(tmp_path):
    exe = tmp_path / "check_placement"
    src = os.path.join(ROOT, "tests", "native", "check_placement.cpp")
    inc = os.path.join(ROOT, "io_aware_exact_07_amd", "csrc")
    r = subprocess.run([HIPCC, "-std=c++17", "-O1", "-I", inc, src, "-o", str(exe)], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:"), r.stdout
    assert "12 heads x 64 levels: on=1" in r.stdout
