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
    assert p["strict_pass"] and p["max_abs_over_rms"] == 0.0 and p["bits_differ"] == 0
    assert p["tokens"] == int(r["written"].sum()) and p["finite"]
    vals = (got.astype(np.uint32) << 16).view(np.float32)
    rms = float(np.sqrt(np.mean(vals[r["tokens"][r["written"]]].astype(np.float64) ** 2)))
    t = int(r["tokens"][r["written"]][0])
    bad = got.copy()
    bad[t, 3] = (np.array([vals[t, 3] + 0.1 * rms], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    p = bench.cpu_baseline(wl, 1 << 30, got=bad)["parity"]
    assert not p["strict_pass"] and p["max_abs_over_rms"] > 0.05 and p["bits_differ"] == 1


def test_cpu_baseline_parity_separates_y_from_the_merge():
    """With the GPU's y passed in: y against the oracle's y, and the oracle's
    merge of that y against the GPU's rows.  A y moved by a few bf16 steps,
    merged exactly, is reported as coming from y only; an output element
    moved by itself is not."""
    import numpy as np
    import oracle
    import workloads as W
    wl = W.tiny()
    r = oracle.forward(wl)
    R = int(r["R"])
    y_dev = np.zeros((R, wl.H), np.uint16)
    y_dev[r["slots"]] = r["y"]
    got = np.full((wl.T, wl.H), 0x7FC1, np.uint16)
    got[r["tokens"][r["written"]]] = r["out"][r["written"]]
    p = bench.cpu_baseline(wl, 1 << 30, got=got, got_y=y_dev)["parity"]
    assert p["y_max_abs_over_rms"] == 0.0 and p["y_bits_differ"] == 0 and p["y_strict_pass"]
    assert p["merge_of_device_y_bits_differ"] == 0 and p["above_bar_from_y_only"]
    # y of one slot moved by 40 bf16 steps in every column, merged by the oracle's merge
    s = int(r["slots"][0])
    y2 = y_dev.copy()
    y2[s] = (y2[s].astype(np.int64) + 40 * np.where(y2[s] & 0x8000, -1, 1)).astype(np.uint16)
    ident = np.arange(R, dtype=np.int64)
    toks = r["tokens"]
    m_out, wr = oracle.combine_tokens(y2, ident, r["slot_of_assign"], r["topk_gate"], toks, wl.k)
    got2 = np.full_like(got, 0x7FC1)
    got2[toks[wr]] = m_out[wr]
    p = bench.cpu_baseline(wl, 1 << 30, got=got2, got_y=y2)["parity"]
    assert not p["y_strict_pass"] and p["above_bar"] > 0
    assert p["merge_of_device_y_bits_differ"] == 0 and p["above_bar_from_y_only"]
    # the same output with an exact y: the merge is what differs
    p = bench.cpu_baseline(wl, 1 << 30, got=got2, got_y=y_dev)["parity"]
    assert p["y_strict_pass"] and not p["above_bar_from_y_only"]
