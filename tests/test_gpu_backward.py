"""GPU tests of the backward of the layer share (mok_combine_backward,
mok_expert_ffn_backward, mok_dispatch_backward; the pages report the
backward pass beside the forward).

The GPU forward (gather, gate/up, down) produces the stored rows the
backward reads; the oracle (oracle.backward) recomputes everything from the
workload in fp64.  Bars (tests/bars.py, derived from where the device rounds):
  - dy = w dout: its bf16 rounding, within 2^-8 of the value;
  - dgate = <dout, y>: the device sums its own bf16 y, which may differ from the
    oracle's only inside y's rounding bands; so dgate must lie in the interval
    of <dout, y> over those bands (plus the fp32 sum's error);
  - dx (per token, after the reverse dispatch) and the weight gradients
    dW_d = sum dy a^T, dW_gu = sum dh x^T: within 6 standard deviations of the
    bf16 roundings of dy, h = [g, u], dh, dx_s, a and the result, propagated
    to first order and summed root-sum-square per element.  (The CPU tests in
    tests/test_bars_host.py show these bars reject a 10 % error.)
  Tokens without a local slot are not written; an empty expert's gradients
  are 0.
Shapes: a ragged pool (tiles with tails, an empty expert) and a wider one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import bars
from gpu_harness import SENTINEL, DeviceWorkload, colblk_rows, empty_u16, to_dev, to_host

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
    _check_backward(wl, ref, dout_np, ref_sched, colblk_rows(dy, R), to_host(dgate),
                    dw.out_rows(dx), to_host(dwd), to_host(dwgu), f"{name} packed={packed}")


def _check_backward(wl, ref, dout_np, ref_sched, dy_bits, dgate_got, dx_rows, dwd_bits, dwgu_bits,
                    what):
    """The device's backward results against oracle.backward, by the bars of
    tests/bars.py: dy within one bf16 ulp of w dout; dgate inside the interval
    of <dout, y> over the forward's rounding bands of y; dx and the weight
    gradients within 6 sigma of the propagated bf16 roundings (root-sum-square,
    per element)."""
    H, I, k, R = wl.H, wl.I, wl.k, ref["R"]
    # dy: the bf16 rounding of w dout, within 2^-8 of its value
    dy_got = bars.bf16_values(dy_bits)
    assert np.all(np.abs(dy_got - ref["dy"]) <= 2.0 ** -8 * np.abs(ref["dy"]) + 1e-30), what
    # dgate: the interval of <dout, y> over the allowed y of every slot
    aos = ref_sched["assign_of_slot"][:R]
    t_of = aos // k
    eos = ref["expert_of_slot"]
    _, a_ex, y_ex = oracle.ffn_rows(ref["x_rows"], eos, wl.w_gu, wl.w_d, False, exact=True)
    y_lo, y_hi, _ = bars.layer_y_band(wl, ref["x_rows"], eos, a_ex, y_ex)
    dv = bars.bf16_values(dout_np)[t_of]
    g_lo, g_hi = bars.dgate_band(dv, y_lo, y_hi)
    g_got = dgate_got.reshape(-1)[aos].astype(np.float64)
    g_ref = ref["dgate"].reshape(-1)[aos]
    assert np.all((g_ref >= g_lo) & (g_ref <= g_hi)), what
    bad = (g_got < g_lo) | (g_got > g_hi)
    assert not bad.any(), (what, "dgate", int(bad.sum()))
    nonlocal_mask = ~np.isin(np.arange(wl.T * k), aos)
    assert np.all(np.isnan(dgate_got.reshape(-1)[nonlocal_mask])), what
    width = float(np.median((g_hi - g_lo) / (np.abs(g_ref) + 1e-30)))
    # dx per token
    wr = ref["written"]
    assert np.all(dx_rows[~wr] == SENTINEL), what
    xv = bars.bf16_values(ref["x_rows"])
    wgu = bars.bf16_values(wl.w_gu)
    wd = bars.bf16_values(wl.w_d)
    s_dh, s_dxs = bars.ffn_backward_sigma(xv, eos, wgu, wd, ref["dy"], ref["h"], ref["dh"])
    bar = bars.dx_bar(s_dxs, t_of, ref["dx"])
    gv = bars.bf16_values(dx_rows)
    assert np.all(np.isfinite(gv[wr])), what
    dd = np.abs(gv - ref["dx"])[wr]
    assert np.all(dd <= bar[wr]), (what, "dx", float(np.max(dd / bar[wr])))
    # weight gradients
    bd, bg = bars.wgrad_bars(eos, wl.n_local, xv, ref["a"], ref["dy"], ref["dh"], s_dh,
                             ref["dw_d"], ref["dw_gu"])
    worst = {}
    for name_, got_b, refw, barw in (("dW_down", dwd_bits, ref["dw_d"], bd),
                                     ("dW_gate_up", dwgu_bits, ref["dw_gu"], bg)):
        gw = bars.bf16_values(got_b)
        assert np.all(np.isfinite(gw)), (what, name_)
        q = np.abs(gw - refw) / barw
        assert np.all(q <= 1.0), (what, name_, float(q.max()))
        worst[name_] = float(q.max())
    print(f"[parity] backward {what}: dgate band width (median) {width:.2e} of |dgate|; dx at "
          f"{float(np.max(dd / bar[wr])):.2f} of its 6-sigma bar (median bar "
          f"{float(np.median(bar[wr] / (np.abs(ref['dx'][wr]) + 1e-30))):.2e} of |dx|); weight "
          f"gradients at {worst['dW_down']:.2f} / {worst['dW_gate_up']:.2f} of theirs", flush=True)


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


def test_saved_h_with_split_workspace():
    """mok_expert_gate_up_save_h with a K-split workspace in which the gate/up
    tiles really split (one busy expert: 2 tiles per XCD, cut into 8 pieces):
    act is bit-identical to mok_expert_gate_up with the same workspace; the
    kept h (summed from the pieces' fp32 partials) is the bf16 rounding of the
    oracle's fp64 h within 6 sigma of the fp32 accumulation; dh and dx_s of the
    backward from it are within the bars of the fp64 chain."""
    import token_dispatch_grouped_top_amd as mok
    counts, H, I = [300, 0, 0, 0, 0, 0, 0, 0], 2048, 1024
    wl = W.pool_workload("split_save_h", 61, 8, 1024, H, I, 64, 8, 5, counts, x_std=1.0,
                         w_std=0.02, route_share=64)
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    R = int(to_host(s["offsets"])[-1])
    d = dw.desc(weights_packed=1)
    w_gu, _ = dw.weights(d)
    ring = torch.zeros((R, H), dtype=torch.int16, device="cuda")
    mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, None, R,
                            mok.MOK_ACT_BF16)
    wsb = mok.mok_gemm_workspace_size()
    ws1 = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    act1 = torch.full((R, I), SENTINEL, dtype=torch.int16, device="cuda")
    act2 = torch.full((R, I), SENTINEL, dtype=torch.int16, device="cuda")
    hs = torch.full((R, 2 * I), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_gate_up(d, ring, None, R, s["offsets"], 0, R, w_gu, act1, None, R, ws1)
    mok.mok_expert_gate_up_save_h(d, ring, R, s["offsets"], 0, R, w_gu, act2, R, hs, ws2)
    torch.cuda.synchronize()
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    cnt_bytes = -(-n_cus * 4 // 256) * 256
    assert int(ws2[cnt_bytes:].count_nonzero()) > 0, "the gate/up tiles did not split"
    assert int(ws2[:cnt_bytes].count_nonzero()) == 0
    assert torch.equal(act1, act2)
    # h against the fp64 h of the oracle's rows
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    xr = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], np.arange(R), False)
    xv = bars.bf16_values(xr)
    wguv = bars.bf16_values(wl.w_gu)
    wdv = bars.bf16_values(wl.w_d)
    h64 = xv @ wguv[0].T
    rms, _ = bars._prefix_rms(wguv[0].astype(np.float32), xv, 256)
    band = bars.C_SIGMA * bars.U32 * np.sqrt(H / 16 / 3.0) * rms + 1e-38
    hg = bars.bf16_values(to_host(hs))
    assert np.all((hg >= bars.bf16_rne(h64 - band)) & (hg <= bars.bf16_rne(h64 + band)))
    # the backward from the kept h
    gu_t_b, d_t_b = mok.mok_packed_weights_bwd_size(d)
    gu_t = torch.empty(gu_t_b, dtype=torch.uint8, device="cuda")
    d_t = torch.empty(d_t_b, dtype=torch.uint8, device="cuda")
    mok.mok_pack_weights_bwd(d, dw.w_gu, dw.w_d, gu_t, d_t)
    dy_np = W.normal_bf16(np.random.SeedSequence(901), R * H, 0.5).reshape(R, H)
    # dy is column-blocked like the ring
    dyd = to_dev(_colblk(dy_np.view(np.uint8).reshape(R, 2 * H), R).view(np.uint16))
    dh = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda")
    dxs = empty_u16(R, H)
    mok.mok_expert_ffn_backward_saved(d, dyd, s["offsets"], 0, R, gu_t, d_t, hs, dh, dxs, R)
    torch.cuda.synchronize()
    dyv = bars.bf16_values(dy_np)
    eor = np.zeros(R, np.int64)
    dh64, dx64 = oracle.ffn_backward_values(xv, eor, wguv, wdv, dyv)
    s_dh, s_dxs = bars.ffn_backward_sigma(xv, eor, wguv, wdv, dyv, h64, dh64)
    dh_got = bars.bf16_values(colblk_rows(dh, R))
    assert np.all(np.abs(dh_got - dh64) <= bars.C_SIGMA * s_dh + 1e-30)
    dx_got = bars.bf16_values(to_host(dxs))
    assert np.all(np.abs(dx_got - dx64) <= bars.C_SIGMA * s_dxs + 1e-30)


def _colblk(rows_bytes: np.ndarray, rows: int) -> np.ndarray:
    """Column-blocked copy of row-major rows (64-byte block b of row r at byte
    (b * rows + r) * 64): the layout of the ring and of dy."""
    nb = rows_bytes.shape[1] // 64
    return np.ascontiguousarray(rows_bytes.reshape(rows, nb, 64).transpose(1, 0, 2)).reshape(-1)
