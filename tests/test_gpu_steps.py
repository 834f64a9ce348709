"""GPU parity of each step of the layer against the CPU oracle, through the C-ABI.

Bars: bit-exact for top-k ids, counts, offsets, slot_of_assign,
assign_of_slot, window segments and dispatched rows (bf16 copies and MXFP8
codes + scales).  Gates: |d| <= 2^-19 * gate (the fp32 error budget of
exp, sum and divide over k <= 32 terms).  Expert outputs and merged rows:
max|d| <= 2e-2 * RMS (bf16) or 6e-2 * RMS (MXFP8) of the oracle's values.
"""
import numpy as np
import pytest
import torch

import bars
import oracle
import workloads as W
from gpu_harness import (DeviceWorkload, assert_close_rms, check_layer_out, check_y_rows, colblk_rows,
                         colblk_scales, empty_u16,
                         gpu_schedule, to_dev, to_host)

pytestmark = pytest.mark.gpu

GATE_RTOL = 2.0 ** -19


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _check_gates(g_gpu, g_orc):
    g_orc = g_orc.astype(np.float64)
    assert np.all(np.abs(g_gpu.astype(np.float64) - g_orc) <= GATE_RTOL * np.maximum(g_orc, 1e-38))


@pytest.mark.parametrize("T,E,k,kind", [(1000, 8, 2, "normal"), (333, 384, 8, "normal"),
                                        (257, 64, 1, "normal"), (100, 4096, 32, "normal"),
                                        (500, 8, 8, "ties"), (300, 384, 8, "ties"),
                                        (64, 3, 3, "ties"), (77, 130, 5, "normal")])
def test_route(T, E, k, kind):
    rng = np.random.default_rng(T * 7 + E)
    if kind == "ties":
        logits = rng.integers(-1, 2, (T, E)).astype(np.float32)
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32) * 2
    idx_o, gate_o = oracle.route_topk(logits, k)
    import token_dispatch_grouped_top_amd as mok
    li = to_dev(logits)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    mok.mok_route_topk(li, T, E, k, idx, gate)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(idx), idx_o)
    _check_gates(to_host(gate), gate_o)


@pytest.mark.parametrize("T,E,k,base,n_local", [(1, 8, 2, 0, 8), (4096, 8, 2, 0, 8),
                                               (5000, 384, 8, 40, 8), (3000, 512, 4, 0, 256),
                                               (1111, 64, 3, 60, 4), (2049, 16, 16, 0, 16),
                                               (700, 300, 1, 299, 1)])
def test_schedule(T, E, k, base, n_local):
    rng = np.random.default_rng(T + n_local)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    s = gpu_schedule(to_dev(idx), T, k, base, n_local)
    torch.cuda.synchronize()
    ref = oracle.build_schedule(idx, base, n_local)
    assert np.array_equal(to_host(s["counts"]), ref["counts"])
    assert np.array_equal(to_host(s["offsets"]), ref["offsets"])
    assert np.array_equal(to_host(s["soa"])[:T * k], ref["slot_of_assign"])
    aos = to_host(s["aos"])
    assert np.array_equal(aos[:ref["R"]], ref["assign_of_slot"])
    assert np.all(aos[ref["R"]:] == -7)      # entries past R are left untouched


def test_schedule_pool_and_windows():
    wl = W.small_pool(21, n_partitions=9, part_rows=700, H=64, I=64, E=384, k=8, expert_base=40,
                      counts=[900, 3, 0, 450, 1, 800, 77, 12])
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    import token_dispatch_grouped_top_amd as mok
    for M in (1, 64, 100, 512, 2243, 5000):
        nwin = -(-wl.T * wl.k // M)
        nwin = min(nwin, 200)
        win = torch.empty((nwin, wl.n_local + 1), dtype=torch.int32, device="cuda")
        mok.mok_build_windows(s["offsets"], wl.n_local, M, nwin, win)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(win), oracle.windows(ref["offsets"], M, nwin)), M
    assert np.array_equal(to_host(s["soa"]), ref["slot_of_assign"])
    assert np.array_equal(to_host(s["aos"])[:ref["R"]], ref["assign_of_slot"])
    # schedule and windows in one call: the same arrays, bit for bit
    A = wl.T * wl.k
    ws = torch.empty(mok.mok_schedule_workspace_size(wl.T, wl.k, wl.n_local), dtype=torch.uint8,
                     device="cuda")
    for M in (64, 2243):
        nwin = min(-(-A // M), 200)
        counts = torch.full((wl.n_local,), -7, dtype=torch.int32, device="cuda")
        offs = torch.full((wl.n_local + 1,), -7, dtype=torch.int32, device="cuda")
        soa = torch.full((A,), -7, dtype=torch.int32, device="cuda")
        aos = torch.full((A,), -7, dtype=torch.int32, device="cuda")
        win = torch.full((nwin, wl.n_local + 1), -7, dtype=torch.int32, device="cuda")
        mok.mok_build_schedule_windows(dw.topk_idx, wl.T, wl.k, wl.expert_base, wl.n_local, counts,
                                       offs, soa, aos, M, nwin, win, ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(counts), np.diff(ref["offsets"]))
        assert np.array_equal(to_host(offs), ref["offsets"])
        assert np.array_equal(to_host(soa), ref["slot_of_assign"])
        assert np.array_equal(to_host(aos)[:ref["R"]], ref["assign_of_slot"])
        assert np.all(to_host(aos)[ref["R"]:] == -7)
        assert np.array_equal(to_host(win), oracle.windows(ref["offsets"], M, nwin)), M


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("S,Wn", [(256, 256), (255, 201)])
def test_gather_bit_exact(mx, S, Wn):
    """Windows of Wn slots through a ring of S rows.  (255, 201): windows
    start at odd slots and wrap around the ring, also between the two slots
    a wave gathers together."""
    import token_dispatch_grouped_top_amd as mok
    wl = W.small_pool(22, n_partitions=5, part_rows=300, H=448, I=64, E=64, k=4, expert_base=8,
                      counts=[200, 1, 0, 333, 90])
    wl.x[7, :32] = 0                        # an all-zero MX block
    wl.x[8, 5] = 0x8000                     # -0.0
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R, H = ref["R"], wl.H
    fmt = mok.MOK_ACT_MXFP8_E4M3 if mx else mok.MOK_ACT_BF16
    ring = torch.zeros((S, H), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    ring_sc = torch.zeros((S, H // 32), dtype=torch.uint8, device="cuda") if mx else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s0 in range(0, R, Wn):    # window by window through the ring
        mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, s0, s0 + Wn,
                                ring, ring_sc, S, fmt, status)
        torch.cuda.synchronize()
        slots = np.arange(s0, min(s0 + Wn, R))
        got = colblk_rows(ring, S)[slots % S]
        exp = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], slots, mx)
        if mx:
            assert np.array_equal(got, exp[0])
            assert np.array_equal(colblk_scales(ring_sc, S)[slots % S], exp[1])
        else:
            assert np.array_equal(got, exp)
    assert int(status.item()) == 0


def _ffn_case(mx, seed=23):
    # ragged everywhere: 3 x 256-row tiles with tails, an empty expert,
    # I = 320 (not a multiple of the 128-column gate/up tile), H = 576.
    return W.small_pool(seed, n_partitions=4, part_rows=250, H=576, I=320, E=32, k=4,
                        expert_base=3, counts=[300, 17, 0, 260, 1],
                        act_format=W.ACT_MXFP8 if mx else W.ACT_BF16)


@pytest.mark.parametrize("mx", [False, True])
def test_expert_ffn(mx):
    import token_dispatch_grouped_top_amd as mok
    wl = _ffn_case(mx)
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R, H, I = ref["R"], wl.H, wl.I
    fmt = wl.act_format
    ring = torch.zeros((R, H), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    ring_sc = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda") if mx else None
    mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, 0, R, ring,
                            ring_sc, R, fmt)
    act = torch.zeros((R, I), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    act_sc = torch.zeros((R, I // 32), dtype=torch.uint8, device="cuda") if mx else None
    y = empty_u16(R, H)
    mok.mok_expert_ffn(dw.desc(), ring, ring_sc, R, s["offsets"], 0, R, dw.w_gu, dw.w_d,
                       act, act_sc, R, y, R)
    torch.cuda.synchronize()
    slots = np.arange(R)
    xr = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], slots, mx)
    check_y_rows(to_host(y), wl, xr, oracle.expert_of_slots(ref["offsets"], slots), "y")


def test_combine():
    import token_dispatch_grouped_top_amd as mok
    wl = W.small_pool(24, n_partitions=3, part_rows=333, H=1024, I=64, E=16, k=6, expert_base=2,
                      counts=[100, 300, 0, 250, 1, 99])
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R = ref["R"]
    y_np = W.normal_bf16(np.random.SeedSequence(5), R * wl.H, 1.0).reshape(R, wl.H)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dw.outs[0]
    mok.mok_combine(to_dev(y_np), R, s["soa"], dw.topk_gate, wl.T, wl.k, wl.H, out, status)
    torch.cuda.synchronize()
    got = dw.out_rows(out)
    o_ref, written = oracle.combine_tokens(y_np, np.arange(R), ref["slot_of_assign"],
                                           wl.topk_gate, np.arange(wl.T), wl.k)
    assert np.all(got[~written] == 0x7FC1)
    # same y on both sides: the fp32 j-order sum may round apart from the fp64 one only
    # where the exact sum is within the fp32 error of a bf16 tie
    yv = bars.bf16_values(y_np)
    lo, hi = bars.out_band(yv, yv, np.arange(R), ref["slot_of_assign"], wl.topk_gate,
                           np.arange(wl.T), wl.k)
    bars.band_stats(got[written], o_ref[written], lo[written], hi[written], 2e-2, "combine")
    assert int(status.item()) == 0
    # the slot-driven merge writes the same rows, bit for bit
    out2 = dw.new_out()
    mok.mok_combine_slots(to_dev(y_np), R, s["aos"], s["offsets"], wl.n_local, R, s["soa"],
                          dw.topk_gate, wl.k, wl.H, out2, status)
    torch.cuda.synchronize()
    assert np.array_equal(dw.out_rows(out2), got)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("M", [64, 256, 1000])
def test_forward_small_pool(mx, M):
    wl = _ffn_case(mx, seed=25)
    dw = DeviceWorkload(wl)
    ws, d = dw.forward(minibatch=M)
    import token_dispatch_grouped_top_amd as mok
    assert mok.mok_device_status(ws) == 0
    got = dw.out_rows(dw.outs[0])
    r = oracle.forward(wl)
    check_layer_out(got, wl, r, f"out M={M}")


def test_forward_tiny():
    wl = W.tiny()
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward()
    import token_dispatch_grouped_top_amd as mok
    assert mok.mok_device_status(ws) == 0
    r = oracle.forward(wl)
    assert np.array_equal(to_host(dw.topk_idx), r["topk_idx"])
    _check_gates(to_host(dw.topk_gate), r["topk_gate"])
    got = dw.out_rows(dw.outs[0])
    assert r["written"].all()
    check_layer_out(got, wl, r, "out tiny")


def test_forward_minibatch_invariance_and_determinism():
    wl = _ffn_case(False, seed=26)
    dw = DeviceWorkload(wl)
    outs = []
    for M, S in ((64, 0), (100, 300), (256, 0), (577, 0), (2000, 0), (256, 0)):
        dw.reset_out(dw.outs[0])
        dw.forward(minibatch=M, ring_slots=S)
        outs.append(dw.out_rows(dw.outs[0]))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_forward_edge_cases():
    import token_dispatch_grouped_top_amd as mok
    # no local rows: nothing written
    wl = W.small_pool(27, n_partitions=2, part_rows=64, H=128, I=128, E=16, k=2, expert_base=0,
                      counts=[0, 0, 0])
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward()
    assert mok.mok_device_status(ws) == 0
    assert np.all(dw.out_rows(dw.outs[0]) == 0x7FC1)
    # capacity exceeded: status set, out untouched
    wl = W.small_pool(28, n_partitions=2, part_rows=64, H=128, I=128, E=16, k=2, expert_base=0,
                      counts=[40, 30])
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward(max_rows=50)
    assert mok.mok_device_status(ws) == mok.MOK_ERR_CAPACITY
    assert np.all(dw.out_rows(dw.outs[0]) == 0x7FC1)
    ws, _ = dw.forward(max_rows=70)
    assert mok.mok_device_status(ws) == 0
    r = oracle.forward(wl)
    got = dw.out_rows(dw.outs[0])
    check_layer_out(got, wl, r, "out capacity 70")
    # one expert takes every row
    wl = W.small_pool(29, n_partitions=1, part_rows=600, H=256, I=128, E=8, k=1, expert_base=0,
                      counts=[600, 0, 0, 0])
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward(minibatch=256)
    r = oracle.forward(wl)
    check_layer_out(dw.out_rows(dw.outs[0]), wl, r, "out one expert")


def test_forward_empty_input():
    import token_dispatch_grouped_top_amd as mok
    wl = W.small_pool(30, n_partitions=1, part_rows=8, H=128, I=128, E=8, k=2, expert_base=0,
                      counts=[1, 1])
    dw = DeviceWorkload(wl)
    d = dw.desc()
    wsb = mok.mok_forward_workspace_size(d, 0, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    mok.mok_moe_forward_routed(d, dw.topk_idx, dw.topk_gate, 0, dw.x, dw.w_gu, dw.w_d,
                               dw.outs[0], ws)
    mok.mok_moe_forward(d, None, 0, dw.x, dw.w_gu, dw.w_d, dw.outs[0], ws)
    assert mok.mok_device_status(ws) == 0
    assert np.all(dw.out_rows(dw.outs[0]) == 0x7FC1)
