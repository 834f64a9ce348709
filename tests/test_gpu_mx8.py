"""GPU tests of the grouped GEMMs with MXFP8 weights (both operands E4M3 with an
E8M0 scale per 32 along K, on gfx950's block-scaled FP8 MFMA).

The tahou.com MoK article fuses MXFP8 quantisation into the datapath; this
path carries the same format into the weights.  Parity:
  - the packed weights: bit-exact against the oracle's quantisation of each
    weight row (codes and scales, read back through the packed tile order);
  - the expert outputs y and merged rows: within 6e-2 * RMS of the oracle run
    with the same quantised weights (gpu_harness.assert_close_rms), for
    standalone calls (whole tiles and the K split), the stream-mode fused
    call over several windows of a ring, and the persistent mode;
  - the persistent mode is bit-identical to the stream mode with whole tiles
    (no_split_k = 1: the same tile code);
  - unpacked MXFP8 weights and bf16 activations with MXFP8 weights are
    refused.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceWorkload, assert_close_rms, check_layer_out, empty_u16, to_host

pytestmark = pytest.mark.gpu
BM = 256
WBLOCK = 256 * 64 + 256 * 2          # packed block per (expert, column tile, k-step)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _case(seed=71, counts=(300, 17, 0, 260, 1), H=576, I=320, n_partitions=4, part_rows=250):
    wl = W.small_pool(seed, n_partitions=n_partitions, part_rows=part_rows, H=H, I=I, E=32, k=4,
                      expert_base=3, counts=list(counts), act_format=W.ACT_MXFP8)
    wl.weight_format = 1
    return wl


def _weight_row(r, nt, swiglu, I, N):
    """Weight row held by row r of column tile nt (the packed tile order)."""
    if swiglu:
        wc, q = r >> 7, r & 127
        icol = min(nt * 128 + 64 * wc + (q & 63), I - 1)
        return icol if q < 64 else I + icol
    return min(nt * 256 + r, N - 1)


def _unpack_block(buf, blk, row):
    """Codes (64, in k order) and the 2 scales of tile row `row` in packed block `blk`."""
    base = blk * WBLOCK
    key = (row >> 2) & 3
    codes = np.concatenate([buf[base + row * 64 + ((c ^ key) << 4):][:16] for c in range(4)])
    scales = buf[base + 256 * 64 + 2 * row:][:2]
    return codes, scales


def test_packed_mxfp8_weights_bit_exact():
    import token_dispatch_grouped_top_amd as mok
    wl = _case()
    dw = DeviceWorkload(wl)
    d = dw.desc()
    pgu, pdn = dw.packed()
    gu_b, dn_b = mok.mok_packed_weights_size(d)
    n1, n2 = -(-wl.I // 128), -(-wl.H // 256)
    assert gu_b == wl.n_local * n1 * (wl.H // 64) * WBLOCK
    assert dn_b == wl.n_local * n2 * (wl.I // 64) * WBLOCK
    qgu, qdn = oracle.mx_quantize_rows(wl.w_gu), oracle.mx_quantize_rows(wl.w_d)
    gu, dn = to_host(pgu), to_host(pdn)
    rng = np.random.default_rng(5)
    for (buf, q, n_t, K, swiglu, N) in ((gu, qgu, n1, wl.H, True, wl.I), (dn, qdn, n2, wl.I, False, wl.H)):
        nk = K // 64
        for _ in range(60):
            e, nt, kt, r = (int(rng.integers(0, wl.n_local)), int(rng.integers(0, n_t)),
                            int(rng.integers(0, nk)), int(rng.integers(0, 256)))
            codes, scales = _unpack_block(buf, (e * n_t + nt) * nk + kt, r)
            wr = _weight_row(r, nt, swiglu, wl.I, N)
            assert np.array_equal(codes, q[0][e, wr, 64 * kt:64 * kt + 64]), (e, nt, kt, r)
            assert np.array_equal(scales, q[1][e, wr, 2 * kt:2 * kt + 2]), (e, nt, kt, r)


@pytest.mark.parametrize("split", [False, True])
def test_mxfp8_weight_gemms(split):
    import token_dispatch_grouped_top_amd as mok
    wl = _case()
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R, H, I = ref["R"], wl.H, wl.I
    ring = torch.zeros((R, H), dtype=torch.uint8, device="cuda")
    ring_sc = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda")
    mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, ring_sc,
                            R, wl.act_format)
    d = dw.desc()
    w_gu, w_d = dw.weights(d)
    ws = torch.zeros(mok.mok_gemm_workspace_size(), dtype=torch.uint8, device="cuda") if split else None
    act = torch.zeros((R, I), dtype=torch.uint8, device="cuda")
    act_sc = torch.zeros((R, I // 32), dtype=torch.uint8, device="cuda")
    y = empty_u16(R, H)
    mok.mok_expert_ffn(d, ring, ring_sc, R, s["offsets"], 0, R, w_gu, w_d, act, act_sc, R, y, R, ws)
    torch.cuda.synchronize()
    slots = np.arange(R)
    xr = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], slots, True)
    mxw = (oracle.mx_quantize_rows(wl.w_gu), oracle.mx_quantize_rows(wl.w_d))
    y_ref = oracle.ffn_rows(xr, oracle.expert_of_slots(ref["offsets"], slots), wl.w_gu, wl.w_d, True,
                            mx_weights=mxw)
    assert_close_rms(to_host(y), y_ref, 6e-2, "y")


def test_mxfp8_weight_gemms_long_k_split():
    """K = 4096 down GEMM over two tiles: the split cuts each tile into 8 pieces."""
    import token_dispatch_grouped_top_amd as mok
    wl = _case(seed=72, counts=(200, 100), H=512, I=4096, n_partitions=8, part_rows=128)
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R, H, I = ref["R"], wl.H, wl.I
    ring = torch.zeros((R, H), dtype=torch.uint8, device="cuda")
    ring_sc = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda")
    mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, ring_sc,
                            R, wl.act_format)
    d = dw.desc()
    w_gu, w_d = dw.weights(d)
    outs = []
    for ws in (torch.zeros(mok.mok_gemm_workspace_size(), dtype=torch.uint8, device="cuda"), None):
        act = torch.zeros((R, I), dtype=torch.uint8, device="cuda")
        act_sc = torch.zeros((R, I // 32), dtype=torch.uint8, device="cuda")
        y = empty_u16(R, H)
        mok.mok_expert_ffn(d, ring, ring_sc, R, s["offsets"], 0, R, w_gu, w_d, act, act_sc, R, y, R,
                           ws)
        torch.cuda.synchronize()
        if ws is not None:
            n_cus = torch.cuda.get_device_properties(0).multi_processor_count
            cnt_bytes = -(-n_cus * 4 // 256) * 256
            assert int(ws[:cnt_bytes].count_nonzero()) == 0     # counters back at zero
            assert int(ws[cnt_bytes:].count_nonzero()) > 0      # the pieces ran
        outs.append(to_host(y))
    slots = np.arange(R)
    xr = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], slots, True)
    mxw = (oracle.mx_quantize_rows(wl.w_gu), oracle.mx_quantize_rows(wl.w_d))
    y_ref = oracle.ffn_rows(xr, oracle.expert_of_slots(ref["offsets"], slots), wl.w_gu, wl.w_d, True,
                            mx_weights=mxw)
    assert_close_rms(outs[0], y_ref, 6e-2, "y split")
    assert_close_rms(outs[1], y_ref, 6e-2, "y whole")


@pytest.mark.parametrize("M", [64, 256, 1000])
def test_mxfp8_weight_forward_stream(M):
    import token_dispatch_grouped_top_amd as mok
    wl = _case(seed=73)
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward(minibatch=M)
    assert mok.mok_device_status(ws) == 0
    r = oracle.forward(wl)
    check_layer_out(dw.out_rows(dw.outs[0]), wl, r, f"out stream M={M}")


@pytest.mark.parametrize("M", [64, 256, 1000])
def test_mxfp8_weight_forward_persistent(M):
    import token_dispatch_grouped_top_amd as mok
    wl = _case(seed=75)
    dw = DeviceWorkload(wl, n_out=2)
    ws, _ = dw.forward(out=dw.outs[0], minibatch=M, mode=1, wait_timeout_us=500_000)
    assert mok.mok_device_status(ws) == 0
    ws2, _ = dw.forward(out=dw.outs[1], minibatch=M, no_split_k=1)
    assert mok.mok_device_status(ws2) == 0
    got, ref_stream = dw.out_rows(dw.outs[0]), dw.out_rows(dw.outs[1])
    assert np.array_equal(got, ref_stream)
    r = oracle.forward(wl)
    check_layer_out(got, wl, r, f"out persistent M={M}")


def test_mxfp8_weight_refusals():
    import token_dispatch_grouped_top_amd as mok
    wl = _case(seed=74)
    dw = DeviceWorkload(wl)
    d = dw.desc()
    d.weights_packed = 0                                             # MXFP8 weights are packed
    ring = torch.zeros((64, wl.H), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((64, wl.H // 32), dtype=torch.uint8, device="cuda")
    act = torch.zeros((64, wl.I), dtype=torch.uint8, device="cuda")
    asc = torch.zeros((64, wl.I // 32), dtype=torch.uint8, device="cuda")
    offs = torch.zeros(wl.n_local + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(mok.MokError) as e:
        mok.mok_expert_gate_up(d, ring, sc, 64, offs, 0, 64, dw.w_gu, act, asc, 64)
    assert e.value.status == mok.MOK_ERR_INVALID_ARG
    bad = dw.desc()
    bad.act_format = mok.MOK_ACT_BF16                                # needs MXFP8 activations
    with pytest.raises(mok.MokError):
        mok.mok_packed_weights_size(bad)
