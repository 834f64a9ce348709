"""GPU tests of the backward of the layer share (mok_combine_backward,
mok_expert_ffn_backward, mok_dispatch_backward; the pages report the
backward pass beside the forward).

The GPU forward (gather, gate/up, down) produces the stored rows the
backward reads; the oracle (oracle.backward) recomputes everything from the
workload in fp64.  Bars:
  - dy = w dout: within one bf16 ulp (the device rounds w dout from fp32);
  - dgate = <dout, y>: the device sums its own bf16 y, which is held to the
    forward's bar (2e-2 RMS(y) per element), so |dgate - ref| <=
    2e-2 * RMS(y) * sqrt(H) * ||dout[t]|| + 1e-3 * sum_h |dout y_ref|;
  - dx (per token, after the reverse dispatch): the device stores h = [g, u],
    dy and dh in bf16 on the way (relative error 2^-9 each), and dx sums 2I
    products of dh with W_gu, so its error is bounded per element by
    8 * 2^-9 * sum_j |W_gu[j][h]| |dh_j| (summed over the token's slots, from
    the oracle's fp64 dh) plus the layer's 2e-2 * RMS; tokens without a local
    slot are not written.
  - weight gradients dW_d = sum dy a^T and dW_gu = sum dh x^T (mok_expert_wgrad):
    per element 2e-2 * RMS + 8 * 2^-9 * sum_s |dy||a| (resp. |dh||x|), the
    rounding bound of their bf16 operands; an empty expert's gradients are 0.
Shapes: a ragged pool (tiles with tails, an empty expert) and a wider one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import (SENTINEL, DeviceWorkload, assert_close_rms, colblk_rows, empty_u16,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _case(name):
    if name == "ragged":
        return W.small_pool(81, n_partitions=4, part_rows=250, H=576, I=320, E=32, k=4,
                            expert_base=3, counts=[300, 17, 0, 260, 1])
    return W.small_pool(82, n_partitions=4, part_rows=256, H=1024, I=512, E=64, k=8,
                        expert_base=0, counts=[200, 150, 0, 90, 301, 5, 64, 100])


@pytest.mark.parametrize("name,packed", [("ragged", 0), ("ragged", 1), ("wide", 1)])
def test_backward_matches_oracle(name, packed):
    import token_dispatch_grouped_top_amd as mok
    wl = _case(name)
    dw = DeviceWorkload(wl)
    H, I, k = wl.H, wl.I, wl.k
    s = dw.schedule(dw.topk_idx)
    ref_sched = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R = ref_sched["R"]
    d = dw.desc()
    # forward: the rows the backward reads (ring = gathered x, y)
    ring = torch.zeros((R, H), dtype=torch.int16, device="cuda")
    mok.mok_dispatch_gather(dw.x, H, k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, None, R,
                            mok.MOK_ACT_BF16)
    act = torch.zeros((R, I), dtype=torch.int16, device="cuda")
    y = empty_u16(R, H)
    mok.mok_expert_ffn(d, ring, None, R, s["offsets"], 0, R, dw.w_gu, dw.w_d, act, None, R, y, R)
    # dout for every pool token
    dout_np = W.normal_bf16(np.random.SeedSequence(500 + R), wl.T * H, 1.0).reshape(wl.T, H)
    dout = mok.Tokens([to_dev(dout_np[p * wl.part_rows:(p + 1) * wl.part_rows])
                       for p in range(wl.n_partitions)], wl.part_rows)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dy = torch.zeros((R, H), dtype=torch.int16, device="cuda")
    dgate = torch.full((wl.T, k), float("nan"), dtype=torch.float32, device="cuda")
    mok.mok_combine_backward(dout, y, R, s["aos"], s["offsets"], wl.n_local, R, dw.topk_gate, k, H,
                             dy, R, dgate, status)
    gu_t_b, d_t_b = mok.mok_packed_weights_bwd_size(d)
    gu_t = torch.empty(gu_t_b, dtype=torch.uint8, device="cuda")
    d_t = torch.empty(d_t_b, dtype=torch.uint8, device="cuda")
    mok.mok_pack_weights_bwd(d, dw.w_gu, dw.w_d, gu_t, d_t)
    h = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    dh = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    dxs = empty_u16(R, H)
    db = dw.desc(weights_packed=packed)                 # h recomputed with either gate/up layout
    mok.mok_expert_ffn_backward(db, ring, R, dy, s["offsets"], 0, R, dw.weights(db)[0], gu_t, d_t, h,
                                dh, dxs, R)
    wsb = mok.mok_wgrad_workspace_size(d, R)
    wws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    dwgu = torch.full((wl.n_local, 2 * I, H), SENTINEL, dtype=torch.int16, device="cuda")
    dwd = torch.full((wl.n_local, H, I), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_wgrad(d, ring, R, act, R, dy, dh, R, s["offsets"], dwgu, dwd, wws)
    dx = dw.new_out()
    mok.mok_dispatch_backward(dxs, R, s["aos"], s["offsets"], wl.n_local, R, s["soa"], k, H, dx,
                              status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = oracle.backward(wl, dout_np)
    assert ref["R"] == R
    # dy: one bf16 ulp of w dout
    dy_got = oracle.bf16_value(colblk_rows(dy, R)).astype(np.float64)
    assert np.all(np.abs(dy_got - ref["dy"]) <= 2.0 ** -8 * np.abs(ref["dy"]) + 1e-30)
    # dgate: bounded by the forward's y error
    aos = ref_sched["assign_of_slot"][:R]
    t_of = aos // k
    g_got = to_host(dgate).reshape(-1)[aos]
    g_ref = ref["dgate"].reshape(-1)[aos]
    yv = oracle.bf16_value(ref["y"]).astype(np.float64)
    dv = oracle.bf16_value(dout_np).astype(np.float64)[t_of]
    rms_y = float(np.sqrt(np.mean(yv * yv)))
    bound = 2e-2 * rms_y * np.sqrt(H) * np.linalg.norm(dv, axis=1) + 1e-3 * np.sum(np.abs(dv * yv), 1)
    assert np.all(np.abs(g_got - g_ref) <= bound)
    nonlocal_mask = ~np.isin(np.arange(wl.T * k), aos)
    assert np.all(np.isnan(to_host(dgate).reshape(-1)[nonlocal_mask]))
    # dx per token
    got = dw.out_rows(dx)
    wr = ref["written"]
    assert np.all(got[~wr] == SENTINEL)
    wgu = np.abs(oracle.bf16_value(wl.w_gu).astype(np.float64))
    mag = np.zeros((wl.T, H))
    for e in np.unique(ref["expert_of_slot"]):
        r = np.nonzero(ref["expert_of_slot"] == e)[0]
        np.add.at(mag, ref["token_of_slot"][r], np.abs(ref["dh"][r]) @ wgu[e])
    dref = ref["dx"][wr]
    gv = oracle.bf16_value(got[wr]).astype(np.float64)
    assert np.all(np.isfinite(gv))
    rms = float(np.sqrt(np.mean(dref * dref)))
    bar = 2e-2 * rms + 8 * 2.0 ** -9 * mag[wr]
    assert np.all(np.abs(gv - dref) <= bar), float(np.max(np.abs(gv - dref) / bar))
    # weight gradients: per element, 2e-2 RMS plus the rounding bound of the bf16
    # operands over the expert's slots (8 * 2^-9 * sum_s |u_s| |v_s|)
    eos, xv = ref["expert_of_slot"], oracle.bf16_value(oracle.gather_rows(
        wl.x, k, aos, np.arange(R), False)).astype(np.float64)
    wguv = oracle.bf16_value(wl.w_gu).astype(np.float64)
    for name_, got_t, refw in (("dW_down", dwd, ref["dw_d"]), ("dW_gate_up", dwgu, ref["dw_gu"])):
        gw = oracle.bf16_value(to_host(got_t)).astype(np.float64)
        assert np.all(np.isfinite(gw)), name_
        rmsw = float(np.sqrt(np.mean(refw * refw)))
        for e in range(wl.n_local):
            r = np.nonzero(eos == e)[0]
            if name_ == "dW_down":
                hh = xv[r] @ wguv[e].T
                av = oracle.silu_and_grad(hh[:, :I])[0] * hh[:, I:]
                magw = np.abs(ref["dy"][r]).T @ np.abs(av)
            else:
                magw = np.abs(ref["dh"][r]).T @ np.abs(xv[r])
            barw = 2e-2 * rmsw + 8 * 2.0 ** -9 * magw
            assert np.all(np.abs(gw[e] - refw[e]) <= barw), (name_, e, float(np.max(np.abs(gw[e] - refw[e]) / barw)))


def test_wgrad_offsets_past_rows_stay_in_bounds():
    """Device offsets that claim more slots than rows (a broken caller) must
    not take the weight gradients outside their buffers: every expert then
    gets one 32-slot segment.  The call returns, writes every gradient
    element (finite, the sentinel gone) and leaves the guard bytes around
    the workspace untouched."""
    import token_dispatch_grouped_top_amd as mok
    H, I, n_local, rows = 256, 128, 4, 64
    d = mok.mok_layer_desc(hidden=H, inter=I, n_experts=8, top_k=2, expert_base=0,
                           n_local=n_local, act_format=mok.MOK_ACT_BF16, weight_format=0)
    g = torch.Generator().manual_seed(7)
    def rnd(*shape):
        return (torch.randn(*shape, generator=g) * 0.5).to(torch.bfloat16).view(torch.int16).cuda()
    ring, act, dy, dh = rnd(rows, H), rnd(rows, I), rnd(rows, H), rnd(rows, 2 * I)
    offsets = torch.tensor([0, 100, 5000, 5001, 90000], dtype=torch.int32, device="cuda")
    wsb = mok.mok_wgrad_workspace_size(d, rows)
    guard = 1 << 16
    buf = torch.full((wsb + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    wws = buf[guard:guard + wsb]
    dwgu = torch.full((n_local, 2 * I, H), SENTINEL, dtype=torch.int16, device="cuda")
    dwd = torch.full((n_local, H, I), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_wgrad(d, ring, rows, act, rows, dy, dh, rows, offsets, dwgu, dwd, wws)
    torch.cuda.synchronize()
    for t in (dwgu, dwd):
        v = t.view(torch.bfloat16).float()
        assert torch.isfinite(v).all()
    assert int((buf[:guard] != 0x5A).sum()) == 0 and int((buf[guard + wsb:] != 0x5A).sum()) == 0


@pytest.mark.parametrize("name,packed", [("ragged", 0), ("wide", 1)])
def test_saved_h_matches_recompute(name, packed):
    """mok_expert_gate_up_save_h stores act bit-identical to mok_expert_gate_up
    and h bit-identical to the backward's recompute; the backward fed that h
    (mok_expert_ffn_backward_saved) gives dh and dx bit-identical to the
    recomputing one."""
    import token_dispatch_grouped_top_amd as mok
    wl = _case(name)
    dw = DeviceWorkload(wl)
    H, I, k = wl.H, wl.I, wl.k
    s = dw.schedule(dw.topk_idx)
    R = int(to_host(s["offsets"])[-1])
    d = dw.desc(weights_packed=packed)
    w_gu, _ = dw.weights(d)
    ring = torch.zeros((R, H), dtype=torch.int16, device="cuda")
    mok.mok_dispatch_gather(dw.x, H, k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, None, R,
                            mok.MOK_ACT_BF16)
    act1 = torch.full((R, I), SENTINEL, dtype=torch.int16, device="cuda")
    act2 = torch.full((R, I), SENTINEL, dtype=torch.int16, device="cuda")
    hs = torch.full((R, 2 * I), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_gate_up(d, ring, None, R, s["offsets"], 0, R, w_gu, act1, None, R)
    mok.mok_expert_gate_up_save_h(d, ring, R, s["offsets"], 0, R, w_gu, act2, R, hs)
    gu_t_b, d_t_b = mok.mok_packed_weights_bwd_size(d)
    gu_t = torch.empty(gu_t_b, dtype=torch.uint8, device="cuda")
    d_t = torch.empty(d_t_b, dtype=torch.uint8, device="cuda")
    mok.mok_pack_weights_bwd(d, dw.w_gu, dw.w_d, gu_t, d_t)
    g = torch.Generator().manual_seed(900 + R)
    dy = (torch.randn(R, H, generator=g) * 0.5).to(torch.bfloat16).view(torch.int16).cuda()
    h1 = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    dh1 = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    dh2 = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    dx1, dx2 = empty_u16(R, H), empty_u16(R, H)
    mok.mok_expert_ffn_backward(d, ring, R, dy, s["offsets"], 0, R, w_gu, gu_t, d_t, h1, dh1, dx1, R)
    mok.mok_expert_ffn_backward_saved(d, dy, s["offsets"], 0, R, gu_t, d_t, hs, dh2, dx2, R)
    torch.cuda.synchronize()
    assert torch.equal(act1, act2)
    assert torch.equal(h1, hs)
    assert torch.equal(dh1, dh2)
    assert torch.equal(dx1, dx2)
