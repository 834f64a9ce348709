"""Packed weights (mok_pack_weights): the grouped GEMMs read the same values in
another memory order, so every output must equal the unpacked run bit for bit.

Cases: ragged shapes (I = 320 gives a partial gate/up column tile, H = 576 a
partial down tile, expert counts with an empty and a one-row expert), bf16
and MXFP8 activations, stream-ordered and persistent paths, the standalone
gate/up and down calls, and the Zipf-skewed MXFP8 expert share at full size.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_harness import DeviceWorkload, gpu_schedule

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _case(mx, seed=60):
    return W.small_pool(seed, n_partitions=4, part_rows=250, H=576, I=320, E=32, k=4,
                        expert_base=3, counts=[300, 17, 0, 260, 1],
                        act_format=W.ACT_MXFP8 if mx else W.ACT_BF16)


def _equal_outs(dw, a, b):
    return all(torch.equal(x, y) for x, y in zip(a.parts, b.parts))


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("mode,M", [(0, 64), (0, 1000), (1, 128)])
def test_packed_forward_bit_identical(mx, mode, M):
    import token_dispatch_grouped_top_amd as mok
    dw = DeviceWorkload(_case(mx), n_out=2)
    kw = dict(minibatch=M, mode=mode, wait_timeout_us=500_000)
    ws0, _ = dw.forward(out=dw.outs[0], **kw)
    ws1, _ = dw.forward(out=dw.outs[1], weights_packed=1, **kw)
    assert mok.mok_device_status(ws0) == 0 and mok.mok_device_status(ws1) == 0
    assert _equal_outs(dw, dw.outs[0], dw.outs[1])


@pytest.mark.parametrize("mx", [False, True])
def test_packed_expert_calls_bit_identical(mx):
    import token_dispatch_grouped_top_amd as mok
    wl = _case(mx, 61)
    dw = DeviceWorkload(wl)
    sch = gpu_schedule(dw.topk_idx, wl.T, wl.k, wl.expert_base, wl.n_local)
    R = int(sch["offsets"][-1].item())
    S, H, I = R, wl.H, wl.I
    dt = torch.uint8 if mx else torch.int16
    ring = torch.empty((S, H), dtype=dt, device="cuda")
    ring_sc = torch.empty((S, H // 32), dtype=torch.uint8, device="cuda") if mx else None
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    mok.mok_dispatch_gather(dw.x, H, wl.k, sch["aos"], sch["offsets"], wl.n_local, 0, S, ring,
                            ring_sc, S, wl.act_format, st)
    res = []
    for packed in (0, 1):
        d = dw.desc(weights_packed=packed)
        w_gu, w_d = dw.weights(d)
        act = torch.empty((S, I), dtype=dt, device="cuda")
        act_sc = torch.empty((S, I // 32), dtype=torch.uint8, device="cuda") if mx else None
        y = torch.empty((S, H), dtype=torch.int16, device="cuda")
        mok.mok_expert_gate_up(d, ring, ring_sc, S, sch["offsets"], 0, S, w_gu, act, act_sc, S)
        mok.mok_expert_down(d, act, act_sc, S, sch["offsets"], 0, S, w_d, y, S)
        torch.cuda.synchronize()
        res.append((act, act_sc, y))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][2], res[1][2])
    if mx:
        assert torch.equal(res[0][1], res[1][1])


def test_packed_full_size_zipf_mxfp8():
    import token_dispatch_grouped_top_amd as mok
    dw = DeviceWorkload(W.kimi_zipf_mxfp8(), n_out=2)
    ws0, _ = dw.forward(out=dw.outs[0], max_rows=8192, minibatch=4096)
    ws1, _ = dw.forward(out=dw.outs[1], max_rows=8192, minibatch=4096, weights_packed=1)
    assert mok.mok_device_status(ws0) == 0 and mok.mok_device_status(ws1) == 0
    assert _equal_outs(dw, dw.outs[0], dw.outs[1])
