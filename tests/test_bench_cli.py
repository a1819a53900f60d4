"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message (the library runs on one GPU), and the measured-profile
lookups return nothing for a workload with no summary."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profile_lookups_without_a_summary():
    assert bench.measured_traffic("no_such_workload", "k_fwd_small<4>") is None
    assert bench.measured_mfma_util("no_such_workload") is None


def test_profile_lookup_rejects_another_kernel():
    # the decode summary is for the one-wave kernel only
    assert bench.measured_traffic("decode", "k_fwd_mfma") is None
