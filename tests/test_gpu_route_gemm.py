"""GPU tests of the router GEMM fused with the route (tahou.com MoK article,
routing paragraph: every token is scored against every expert, then the
router picks; mok_route_topk_gemm).

The device sums the bf16 products in fp32 in its own order; the oracle sums
them in fp64 (oracle.router_logits) and picks with oracle.route_topk.  Bars:
  - integer-valued inputs: every fp32 sum is exact, so picks are bit-exact
    against the oracle, ties (frequent here) included, and gates within the
    route's own bar;
  - Gaussian inputs: where the oracle's logits leave a margin larger than the
    fp32 error bound around every decision (the k-th against the (k+1)-th
    logit, and consecutive picks), the picks equal the oracle's; where only
    the k-th against the (k+1)-th is clear, the picked set does; elsewhere
    they are a valid top-k within that bound.  The bound for token t and
    expert e is n * 2^-24 * sum_h |x_th w_eh| with n = H / 16 + splits + 16
    fp32 additions on any path; the set must be clear for at least 90 % of
    the tokens (so the test has teeth).  Gates are held to the softmax of the oracle's logits over the
    device's picks.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _run(x, w, k):
    import token_dispatch_grouped_top_amd as mok
    T, H = x.shape
    E = w.shape[0]
    ws = torch.empty(max(mok.mok_route_gemm_workspace_size(T, E, H), 1), dtype=torch.uint8,
                     device="cuda")
    idx = torch.full((max(T, 1), k), -1, dtype=torch.int32, device="cuda")
    gate = torch.zeros((max(T, 1), k), dtype=torch.float32, device="cuda")
    mok.mok_route_topk_gemm(to_dev(x), to_dev(w), T, H, E, k, ws, idx, gate)
    torch.cuda.synchronize()
    return to_host(idx)[:T], to_host(gate)[:T]


@pytest.mark.parametrize("T,E,H,k", [(100, 40, 48, 3), (1000, 384, 7168, 8), (257, 8, 4096, 2),
                                     (33, 130, 272, 5)])
def test_route_gemm_integer_inputs_bit_exact(T, E, H, k):
    x = W.small_int_bf16(31 + T, (T, H), -2, 2)
    w = W.small_int_bf16(37 + E, (E, H), -2, 2)
    idx, gate = _run(x, w, k)
    logits = oracle.router_logits(x, w)
    assert np.abs(logits).max() < 2 ** 24                   # exact in fp32 too
    idx_o, gate_o = oracle.route_topk(logits.astype(np.float32), k)
    assert np.array_equal(idx, idx_o)
    assert np.all(np.abs(gate.astype(np.float64) - gate_o) <= 2.0 ** -19 * gate_o + 1e-30)


@pytest.mark.parametrize("T,E,H,k", [(1024, 384, 7168, 8), (4096, 8, 4096, 2), (256, 8, 256, 2)])
def test_route_gemm_gaussian(T, E, H, k):
    import token_dispatch_grouped_top_amd as mok
    x, w = W.router_inputs(41 + T + E, T, H, E)
    idx, gate = _run(x, w, k)
    L = oracle.router_logits(x, w)
    splits = mok.mok_route_gemm_workspace_size(T, E, H) // (4 * T * E)
    n_add = H // 16 + splits + 16
    absdot = np.abs(oracle.bf16_value(x).astype(np.float64)) @ \
        np.abs(oracle.bf16_value(w).astype(np.float64)).T
    delta = n_add * 2.0 ** -24 * absdot
    decided = 0
    for t in range(T):
        p = idx[t]
        assert len(set(p.tolist())) == k and p.min() >= 0 and p.max() < E
        lt, dt = L[t], delta[t]
        rest = np.setdiff1d(np.arange(E), p)
        # valid: every pick beats every non-pick, and picks are in order, within the bound
        if rest.size:
            assert (lt[p] + dt[p]).min() >= (lt[rest] - dt[rest]).max(), t
        assert np.all(lt[p[:-1]] + dt[p[:-1]] >= lt[p[1:]] - dt[p[1:]]), t
        # decided tokens: the oracle's picks, exactly
        po, _ = oracle.route_topk(lt[None, :].astype(np.float32), k)
        po = po[0]
        so = np.sort(lt)[::-1]
        order = np.argsort(-lt, kind="stable")
        margins = so[:min(k + 1, E) - 1] - so[1:min(k + 1, E)]
        need = dt[order[:min(k + 1, E) - 1]] + dt[order[1:min(k + 1, E)]]
        if np.all(margins > need):                      # every decision clear: same picks
            assert np.array_equal(p, po), t
        if k < E and margins[k - 1] > need[k - 1]:      # the set is clear: same set
            decided += 1
            assert set(p.tolist()) == set(po.tolist()), t
        g_ref = np.exp(lt[p] - lt[p[0]])
        g_ref /= g_ref.sum()
        tol = 2.0 * dt[p].max() * 2 + 1e-6
        assert np.all(np.abs(gate[t].astype(np.float64) - g_ref) <= tol * g_ref + 1e-7), t
    assert decided >= 0.9 * T or E <= k + 1 and decided >= 0.8 * T, (decided, T)


def test_route_gemm_empty_and_errors():
    import token_dispatch_grouped_top_amd as mok
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    idx = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    gate = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    w = torch.zeros((8, 64), dtype=torch.int16, device="cuda")
    mok.mok_route_topk_gemm(x, w, 0, 64, 8, 2, ws, idx, gate)      # T = 0: nothing
    with pytest.raises(mok.MokError) as e:
        mok.mok_route_topk_gemm(x, w, 4, 64, 8, 2, ws, idx, gate)  # workspace too small
    assert e.value.status == mok.MOK_ERR_WORKSPACE
    with pytest.raises(mok.MokError):
        mok.mok_route_topk_gemm(x, w, 4, 60, 8, 2, ws, idx, gate)  # H not a multiple of 16


def _router_layer(name, T, H, I, E, k, part_rows, seed, integer):
    """A layer whose routing comes from a router GEMM: tokens x [T][H] (in
    partitions of part_rows rows), router rows w_r [E][H]; the workload's
    logits are the oracle's router_logits of them (exact in fp32 for integer
    inputs)."""
    import dataclasses
    base = W.logits_workload(name, seed, T=T, H=H, I=I, E=E, k=k, x_std=1.0, w_std=0.02)
    if integer:
        x = W.small_int_bf16(seed + 1, (T, H), -2, 2)
        w_r = W.small_int_bf16(seed + 2, (E, H), -2, 2)
    else:
        x, w_r = W.router_inputs(seed + 3, T, H, E)
    logits = oracle.router_logits(x, w_r).astype(np.float32)
    wl = dataclasses.replace(base, x=x, logits=logits, n_partitions=T // part_rows,
                             part_rows=part_rows)
    return wl, w_r


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_layer_from_router_weights_integer_inputs(mode):
    """mok_moe_forward_router (router GEMM + pick + counts, schedule, gather, FFN,
    merge in one call) on integer-valued tokens and router rows: the routing is
    the oracle's exactly, so the merged rows meet the oracle's rounding bands."""
    import token_dispatch_grouped_top_amd as mok
    from gpu_harness import DeviceWorkload, check_layer_out
    wl, w_r = _router_layer("router_int", 768, 256, 320, 16, 2, 256, 51, True)
    assert np.abs(wl.logits).max() < 2 ** 24
    dw = DeviceWorkload(wl)
    d = dw.desc(mode=mode, minibatch=512, wait_timeout_us=500_000)
    ws = torch.empty(mok.mok_forward_router_workspace_size(d, wl.T), dtype=torch.uint8,
                     device="cuda")
    mok.mok_moe_forward_router(d, to_dev(w_r), wl.T, dw.x, dw.w_gu, dw.w_d, dw.outs[0], ws)
    assert mok.mok_device_status(ws) == 0
    r = oracle.forward(wl)
    check_layer_out(dw.out_rows(dw.outs[0]), wl, r, f"fused from router weights, mode {mode}")


def test_fused_layer_from_router_weights_matches_two_calls():
    """On Gaussian inputs with the Mixtral-shaped routing (T = 4096, E = 8,
    H = 4096, k = 2; I = 1024 to keep the test short):
    the fused router form writes the same bits as mok_route_topk_gemm followed
    by mok_moe_forward_routed (the same kernels decide the picks), and a
    smaller workspace is refused."""
    import token_dispatch_grouped_top_amd as mok
    from gpu_harness import DeviceWorkload
    wl, w_r = _router_layer("router_gauss", 4096, 4096, 1024, 8, 2, 1024, 52, False)
    dw = DeviceWorkload(wl, n_out=2)
    d = dw.desc(max_rows=wl.T * wl.k, weights_packed=1)
    w_gu, w_d = dw.weights(d)
    wr = to_dev(w_r)
    n = mok.mok_forward_router_workspace_size(d, wl.T)
    assert n > mok.mok_forward_workspace_size(d, wl.T, 1)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    with pytest.raises(mok.MokError) as e:
        mok.mok_moe_forward_router(d, wr, wl.T, dw.x, w_gu, w_d, dw.outs[0], ws, n - 1)
    assert e.value.status == mok.MOK_ERR_WORKSPACE
    mok.mok_moe_forward_router(d, wr, wl.T, dw.x, w_gu, w_d, dw.outs[0], ws)
    assert mok.mok_device_status(ws) == 0
    x_flat = to_dev(wl.x)
    rws = torch.empty(mok.mok_route_gemm_workspace_size(wl.T, wl.E, wl.H), dtype=torch.uint8,
                      device="cuda")
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    mok.mok_route_topk_gemm(x_flat, wr, wl.T, wl.H, wl.E, wl.k, rws, idx, gate)
    mok.mok_moe_forward_routed(d, idx, gate, wl.T, dw.x, w_gu, w_d, dw.outs[1], ws)
    assert mok.mok_device_status(ws) == 0
    for a, b in zip(dw.outs[0].parts, dw.outs[1].parts):
        assert torch.equal(a, b)
