"""Host-side checks of bench.py's contract (no GPU needed): more than one GPU
is refused with a message before anything touches a device, and the HBM
traffic figure is reported only for a workload whose counters were recorded
against the current GEMM sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "single GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_null_without_a_record():
    assert bench.gate_up_traffic("no_such_workload") is None


def test_traffic_records_name_known_workloads():
    for name, (digest, nbytes) in bench.GATE_UP_TRAFFIC.items():
        assert name.startswith("kimi")
        assert len(digest) == 16 and int(digest, 16) >= 0
        assert nbytes > 0
