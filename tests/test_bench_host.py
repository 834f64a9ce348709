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


def test_cpu_baseline_parity_statistic():
    """The bench's parity report (cpu_baseline with the GPU rows passed in):
    zero for the oracle's own rows, above the bar for rows with one element
    moved by 10 % of the RMS, and only rows of tokens with local slots count."""
    import numpy as np
    import oracle
    import workloads as W
    wl = W.tiny()
    r = oracle.forward(wl)
    got = np.full((wl.T, wl.H), 0x7FC1, np.uint16)      # rows of unrouted tokens: a NaN pattern
    got[r["tokens"][r["written"]]] = r["out"][r["written"]]
    res = bench.cpu_baseline(wl, 1 << 30, got=got)
    p = res["parity"]
    assert p["pass"] and p["max_abs_over_rms"] == 0.0 and p["bits_differ"] == 0
    assert p["tokens"] == int(r["written"].sum()) and p["finite"]
    vals = (got.astype(np.uint32) << 16).view(np.float32)
    rms = float(np.sqrt(np.mean(vals[r["tokens"][r["written"]]].astype(np.float64) ** 2)))
    t = int(r["tokens"][r["written"]][0])
    bad = got.copy()
    bad[t, 3] = (np.array([vals[t, 3] + 0.1 * rms], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    p = bench.cpu_baseline(wl, 1 << 30, got=bad)["parity"]
    assert not p["pass"] and p["max_abs_over_rms"] > 0.05 and p["bits_differ"] == 1
