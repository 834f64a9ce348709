"""GPU tests of the MXFP8 backward of the layer share (mok_combine_backward_mx,
mok_expert_gate_up_save_h_mx, mok_expert_ffn_backward_mx, mok_expert_wgrad_mx
and mok_dispatch_backward; the article reports the MXFP8 backward beside the
bf16 one) against oracle.backward_mx.

The GPU forward (MXFP8 gather, gate/up, down) produces the stored rows the
backward reads; the oracle recomputes everything from the workload, rounding
each buffer where the path stores it.  Bars (tests/bars.py, mx_backward_bands):
  - the ring and dy (codes and scales): bit-exact, the same decisions on the
    same values;
  - y, h, dx_s, dx and the weight gradients: inside their rounding bands
    (bit-exact outside the flagged elements);
  - act and dh: the device's dequantised values inside the quantisations of
    the interval its pre-quantisation value may take;
  - dgate: inside the interval of <dout, y> over y's bands.
  Tokens without a local slot are not written.
Shapes: a ragged pool (tiles with tails, an empty expert) and a wider one;
h recomputed (either gate/up weight layout) or kept by the forward.

With MXFP8 weights too (each GEMM's weights quantised along its own
contraction dimension, the forward's packed weights for the forward and the
recompute of h, the backward's transposed packs for the two dgrads), the
block-scaled MFMA's error leaves dh's codes a step from the oracle's in more
places: dh is checked against its band, and dx_s, dx and the weight gradients
against the bands of their own GEMM given the device's dh and act
(bars.mx_stage_bands), beside the strict bar against the oracle's values.
"""
import numpy as np
import pytest
import torch

import bars
import oracle
import workloads as W
from gpu_harness import (SENTINEL, DeviceWorkload, colblk_rows, colblk_scales, empty_u16, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _case(name):
    if name == "ragged_w8":              # MXFP8 weights too
        wl = _case("ragged")
        wl.weight_format = 1
        return wl
    if name == "ragged":
        return W.small_pool(84, n_partitions=4, part_rows=250, H=576, I=320, E=32, k=4,
                            expert_base=3, counts=[300, 17, 0, 260, 1], act_format=W.ACT_MXFP8)
    return W.small_pool(85, n_partitions=4, part_rows=256, H=1024, I=512, E=64, k=8,
                        expert_base=0, counts=[200, 150, 0, 90, 301, 5, 64, 100],
                        act_format=W.ACT_MXFP8)


def _u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8, device="cuda")


def _run(wl, packed: int, kept: bool):
    """The MXFP8 forward and backward through the C-ABI; host copies of every
    buffer the checks read."""
    import token_dispatch_grouped_top_amd as mok
    dw = DeviceWorkload(wl)
    H, I, k = wl.H, wl.I, wl.k
    s = dw.schedule(dw.topk_idx)
    R = int(oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)["R"])
    d = dw.desc()
    dp = dw.desc(weights_packed=packed)
    w_gu, w_d = dw.weights(dp)
    ring, ring_sc = _u8(R, H), _u8(R, H // 32)
    mok.mok_dispatch_gather(dw.x, H, k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, ring_sc,
                            R, mok.MOK_ACT_MXFP8_E4M3)
    act, act_sc = _u8(R, I), _u8(R, I // 32)
    y = empty_u16(R, H)
    h = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    if kept:
        mok.mok_expert_gate_up_save_h_mx(dp, ring, ring_sc, R, s["offsets"], 0, R, w_gu, act,
                                         act_sc, R, h)
        mok.mok_expert_down(dp, act, act_sc, R, s["offsets"], 0, R, w_d, y, R)
    else:
        mok.mok_expert_ffn(dp, ring, ring_sc, R, s["offsets"], 0, R, w_gu, w_d, act, act_sc, R,
                           y, R)
    dout_np = W.normal_bf16(np.random.SeedSequence(700 + R), wl.T * H, 1.0).reshape(wl.T, H)
    dout = mok.Tokens([to_dev(dout_np[p * wl.part_rows:(p + 1) * wl.part_rows])
                       for p in range(wl.n_partitions)], wl.part_rows)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dy, dy_sc = _u8(R, H), _u8(R, H // 32)
    dgate = torch.full((wl.T, k), float("nan"), dtype=torch.float32, device="cuda")
    mok.mok_combine_backward_mx(dout, y, R, s["aos"], s["offsets"], wl.n_local, R, dw.topk_gate,
                                k, H, dy, dy_sc, R, dgate, status)
    gu_t_b, d_t_b = mok.mok_packed_weights_bwd_size(d)
    gu_t = torch.empty(gu_t_b, dtype=torch.uint8, device="cuda")
    d_t = torch.empty(d_t_b, dtype=torch.uint8, device="cuda")
    mok.mok_pack_weights_bwd(d, dw.w_gu, dw.w_d, gu_t, d_t)
    dh, dh_sc = _u8(R, 2 * I), _u8(R, 2 * I // 32)
    dxs = empty_u16(R, H)
    mok.mok_expert_ffn_backward_mx(dp, None if kept else ring, None if kept else ring_sc, R, dy,
                                   dy_sc, s["offsets"], 0, R, None if kept else w_gu, gu_t, d_t,
                                   h, kept, dh, dh_sc, dxs, R)
    wws = torch.empty(mok.mok_wgrad_workspace_size(d, R), dtype=torch.uint8, device="cuda")
    dwgu = torch.full((wl.n_local, 2 * I, H), SENTINEL, dtype=torch.int16, device="cuda")
    dwd = torch.full((wl.n_local, H, I), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_wgrad_mx(d, ring, ring_sc, R, act, act_sc, R, dy, dy_sc, dh, dh_sc, R,
                            s["offsets"], dwgu, dwd, wws)
    dx = dw.new_out()
    mok.mok_dispatch_backward(dxs, R, s["aos"], s["offsets"], wl.n_local, R, s["soa"], k, H, dx,
                              status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return dout_np, dict(
        R=R, ring=colblk_rows(ring, R), ring_sc=colblk_scales(ring_sc, R), y=to_host(y),
        act=colblk_rows(act, R), act_sc=colblk_scales(act_sc, R),
        dy=colblk_rows(dy, R), dy_sc=colblk_scales(dy_sc, R), dgate=to_host(dgate),
        h=to_host(h), dh=colblk_rows(dh, R), dh_sc=colblk_scales(dh_sc, R), dxs=to_host(dxs),
        dx=dw.out_rows(dx), dwd=to_host(dwd), dwgu=to_host(dwgu))


def _check(wl, dout_np, g, what):
    r = oracle.backward_mx(wl, dout_np)
    R, k = r["R"], wl.k
    assert g["R"] == R
    b = bars.mx_backward_bands(wl, r, dout_np)
    # the forward's stored rows
    assert np.array_equal(g["ring"], r["x_codes"]) and np.array_equal(g["ring_sc"], r["x_scales"])
    w_mx = getattr(wl, "weight_format", 0) == 1
    tol = 6e-2 if w_mx else 2e-2
    act_vals = oracle.mx_values(g["act"], g["act_sc"])
    bars.interval_stats(act_vals, b["a_q0"], *b["a"], f"{what} act (MXFP8)")
    bars.band_stats(g["y"], r["y"], *b["y"], tol, f"{what} y")
    # merge backward: dy bit-exact, dgate in its interval, nothing for non-local picks
    assert np.array_equal(g["dy"], r["dy_codes"]), what
    assert np.array_equal(g["dy_sc"], r["dy_scales"]), what
    aos = r["assign_of_slot"][:R]
    g_lo, g_hi = b["dgate"]
    g_got = g["dgate"].reshape(-1)[aos].astype(np.float64)
    g_ref = r["dgate"].reshape(-1)[aos]
    assert np.all((g_ref >= g_lo) & (g_ref <= g_hi)), what
    assert np.all((g_got >= g_lo) & (g_got <= g_hi)), (what, "dgate")
    assert np.all(np.isnan(g["dgate"].reshape(-1)[~np.isin(np.arange(wl.T * k), aos)])), what
    # FFN backward
    bars.band_stats(g["h"], r["h"], *b["h"], tol, f"{what} h")
    dh_got = oracle.mx_values(g["dh"], g["dh_sc"])
    st = bars.interval_stats(dh_got, b["dh_q0"], *b["dh"], f"{what} dh (MXFP8)")
    wr = r["written"]
    assert np.all(g["dx"][~wr] == SENTINEL), what
    if not w_mx:
        assert st["differ"] <= max(8, st["n"] // 1000), (what, st)
        bars.band_stats(g["dxs"], r["dx_slots"], *b["dx_slots"], 2e-2, f"{what} dx_s")
        bars.band_stats(g["dx"][wr], r["dx"][wr], b["dx"][0][wr], b["dx"][1][wr], 2e-2, f"{what} dx")
        bars.band_stats(g["dwd"], r["dw_d"], *b["dw_d"], 2e-2, f"{what} dW_d")
        bars.band_stats(g["dwgu"], r["dw_gu"], *b["dw_gu"], 2e-2, f"{what} dW_gu")
        return
    # MXFP8 weights: act and dh are checked above against the oracle's bands;
    # the later stages given the device's own dh and act (bars.mx_stage_bands).
    # The strict statistic against the oracle's values is reported: one E4M3
    # step of a stored act or dh element (1/16 to 1/8 of it), inside its band,
    # moves a weight-gradient element of a small expert by more than 6e-2 RMS
    sb = bars.mx_stage_bands(wl, r, dh_got, act_vals)
    for key, gk in (("dx_slots", "dxs"), ("dw_d", "dwd"), ("dw_gu", "dwgu")):
        lo, hi, ce = sb[key]
        bars.band_stats(g[gk], bars.bf16_bits(ce), lo, hi, 6e-2,
                        f"{what} {key} (given the device's dh)")
        bars.strict_stats(g[gk], r[key], 6e-2, f"{what} {key} against the oracle", check=False)
    dxs_v = bars.bf16_values(g["dxs"])
    soa = r["slot_of_assign"]
    d_lo, d_hi = bars.out_band(dxs_v, dxs_v, np.arange(r["R"]), soa, np.ones(soa.size),
                               np.arange(wl.T), wl.k)
    dxc = np.zeros((wl.T, wl.H))
    np.add.at(dxc, r["token_of_slot"], dxs_v)
    ref_dx = bars.bf16_bits(bars.bf16_rne(dxc))
    bars.band_stats(g["dx"][wr], ref_dx[wr], d_lo[wr], d_hi[wr], 6e-2,
                    f"{what} dx (given the device's dx_s)")
    bars.strict_stats(g["dx"][wr], r["dx"][wr], 6e-2, f"{what} dx against the oracle",
                      check=False)


@pytest.mark.parametrize("name,packed", [("ragged", 0), ("ragged", 1), ("wide", 1), ("ragged_w8", 1)])
def test_mx_backward_matches_oracle(name, packed):
    wl = _case(name)
    dout_np, g = _run(wl, packed, kept=False)
    _check(wl, dout_np, g, f"MXFP8 backward {name} packed={packed}")


@pytest.mark.parametrize("name", ["ragged", "ragged_w8"])
def test_mx_backward_from_kept_h(name):
    """The forward keeps h (mok_expert_gate_up_save_h_mx, no workspace): its act
    and y, and the backward from that h, are bit-identical to the recompute
    path, and both match the oracle."""
    wl = _case(name)
    dout_np, kept = _run(wl, 1, kept=True)
    _, rec = _run(wl, 1, kept=False)
    for key in ("y", "h", "dy", "dy_sc", "dh", "dh_sc", "dxs", "dx", "dwd", "dwgu"):
        assert np.array_equal(kept[key], rec[key]), key
    _check(wl, dout_np, kept, f"MXFP8 backward {name}, kept h")
