"""Pins for the oracle's schedule, windows and minibatch rule.

Schedule (tahou.com MoK article, layout-planning paragraph; PyTorchKR wiki
summary, key point on the {src_rank, src_index} schedule made without a
sort): per-expert counts, exclusive offsets, and a stable placement of each
local assignment a = t*k + j in its expert's segment.  Pinned against
np.bincount / np.cumsum / a stable np.argsort, and exhaustively against the
positional definition on tiny inputs.

Windows and the two-wave minibatch rule (minibatch paragraph of the article;
wiki key point giving 2368 for the hidden 7168 / intermediate 2048 shape).
"""
import os
import itertools

import numpy as np
import pytest


def _check_schedule(orc, idx, base, n_local):
    T, k = idx.shape
    s = orc.build_schedule(idx, base, n_local)
    flat = idx.reshape(-1).astype(np.int64) - base
    local = (flat >= 0) & (flat < n_local)
    key = np.where(local, flat, n_local)
    counts = np.bincount(flat[local], minlength=n_local)
    assert np.array_equal(s["counts"], counts)
    assert np.array_equal(s["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    R = int(local.sum())
    assert s["R"] == R
    assert np.array_equal(s["assign_of_slot"], np.argsort(key, kind="stable")[:R])
    soa = s["slot_of_assign"]
    assert np.all(soa[~local] == -1)
    assert np.array_equal(soa[s["assign_of_slot"]], np.arange(R))   # bijection
    return s


@pytest.mark.parametrize("T,E,k,base,n_local", [(1000, 8, 2, 0, 8), (777, 384, 8, 40, 8),
                                               (300, 64, 4, 10, 20), (50, 4, 4, 0, 4),
                                               (129, 16, 1, 15, 1)])
def test_schedule_vs_numpy(orc, T, E, k, base, n_local):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_schedule(orc, idx, base, n_local)


def test_schedule_exhaustive_tiny(orc):
    """All routings with T <= 3, E <= 3, k <= 2 against the positional definition:
    slot(a) = offsets[e(a)] + #{a' < a : e(a') = e(a)}."""
    for E in (1, 2, 3):
        for k in range(1, min(E, 2) + 1):
            rows = list(itertools.permutations(range(E), k))
            for T in (1, 2, 3):
                for combo in itertools.product(rows, repeat=T):
                    idx = np.array(combo, np.int32).reshape(T, k)
                    for base, n_local in ((0, E), (1, max(E - 1, 1))):
                        s = orc.build_schedule(idx, base, n_local)
                        flat = idx.reshape(-1) - base
                        for a, e in enumerate(flat):
                            if 0 <= e < n_local:
                                before = sum(1 for b in range(a) if flat[b] == e)
                                assert s["slot_of_assign"][a] == s["offsets"][e] + before
                            else:
                                assert s["slot_of_assign"][a] == -1


def test_counts_sum_to_routed_rows(orc):
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(8)[:2] for _ in range(4096)]).astype(np.int32)
    s = orc.build_schedule(idx, 0, 8)
    assert s["counts"].sum() == 4096 * 2


def _windows_brute(offsets, M, nwin):
    R = offsets[-1]
    out = []
    for b in range(nwin):
        lo, hi = min(b * M, R), min((b + 1) * M, R)
        out.append([min(max(o, lo), hi) for o in offsets])
    return np.array(out, np.int32)


@pytest.mark.parametrize("M", [1, 7, 64, 512, 2560, 10000])
def test_windows(orc, M):
    offsets = np.array([0, 3715, 5332, 6326, 7030, 7463, 7769, 8004, 8192], np.int32)
    nwin = -(-8192 // M) + 1
    w = orc.windows(offsets, M, nwin)
    assert np.array_equal(w, _windows_brute(offsets.tolist(), M, nwin))
    # segments of consecutive windows tile [0, R) without overlap
    lens = w[:, 1:] - w[:, :-1]
    assert np.array_equal(lens.sum(0), np.diff(offsets))
    per_win = lens.sum(1)
    assert np.all(per_win[:-2] == M) and per_win[-1] == 0


def _golden_rows(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    with open(path) as f:
        return [[int(v) for v in ln.split()] for ln in f if ln.strip() and not ln.startswith("#")]


def test_minibatch_two_wave_rule(orc):
    # the one sizing figure the pages print (fixture cites it)
    for n_cus, tm, tn, n_out, want in _golden_rows("minibatch_two_wave.txt"):
        assert orc.choose_minibatch(n_cus, tm, tn, n_out) == want
    # closed form, rounded up to 64 rows, clipped to what is available
    assert orc.choose_minibatch(224, 256, 256, 4096) == 7168
    assert orc.choose_minibatch(256, 256, 256, 4096, 8192) == 8192
    assert orc.choose_minibatch(256, 256, 256, 4096, 5000) == 5000
    assert orc.choose_minibatch(10, 16, 16, 4096) == 64
