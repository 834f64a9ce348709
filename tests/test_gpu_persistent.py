"""GPU tests of the persistent pipeline (one cooperative kernel: movers +
MFMA workers signalling through device counters; tahou.com MoK article,
megakernel / minibatch / ring-buffer paragraphs).

Bars: outputs within 2e-2 * RMS (bf16) / 6e-2 * RMS (MXFP8) of the oracle,
and bit-identical to the stream-ordered path with whole tiles (no_split_k = 1:
same per-element arithmetic);
macrobatches streamed through one ring equal standalone runs bit for bit.
Every device wait is bounded, so these tests use a short bound: a stuck
pipeline ends with MOK_ERR_DEVICE instead of hanging.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceWorkload, check_layer_out

pytestmark = pytest.mark.gpu
PERSIST = 1
TIMEOUT_US = 500_000


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _case(mx, seed):
    return W.small_pool(seed, n_partitions=4, part_rows=250, H=576, I=320, E=32, k=4,
                        expert_base=3, counts=[300, 17, 0, 260, 1],
                        act_format=W.ACT_MXFP8 if mx else W.ACT_BF16)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("M", [64, 200, 256, 1000])
def test_persistent_matches_oracle_and_stream(mx, M):
    import token_dispatch_grouped_top_amd as mok
    wl = _case(mx, 40)
    dw = DeviceWorkload(wl, n_out=2)
    ws, _ = dw.forward(out=dw.outs[0], minibatch=M, mode=PERSIST, wait_timeout_us=TIMEOUT_US)
    assert mok.mok_device_status(ws) == 0
    ws2, _ = dw.forward(out=dw.outs[1], minibatch=M, no_split_k=1)
    assert mok.mok_device_status(ws2) == 0
    got, ref_stream = dw.out_rows(dw.outs[0]), dw.out_rows(dw.outs[1])
    assert np.array_equal(got, ref_stream)
    r = oracle.forward(wl)
    check_layer_out(got, wl, r, f"out persistent M={M}")


@pytest.mark.parametrize("n_move", [8, 16, 64])
def test_persistent_mover_counts(n_move):
    import token_dispatch_grouped_top_amd as mok
    wl = _case(False, 41)
    dw = DeviceWorkload(wl, n_out=2)
    ws, _ = dw.forward(out=dw.outs[0], minibatch=128, mode=PERSIST, n_move_cus=n_move,
                       wait_timeout_us=TIMEOUT_US)
    assert mok.mok_device_status(ws) == 0
    dw.forward(out=dw.outs[1], minibatch=128, no_split_k=1)
    assert np.array_equal(dw.out_rows(dw.outs[0]), dw.out_rows(dw.outs[1]))


def test_persistent_macrobatches_equal_standalone():
    """Several macrobatches through one ring: each equals its standalone run."""
    import token_dispatch_grouped_top_amd as mok
    base = _case(False, 42)
    wls = [base] + [W.pool_workload(f"m{m}", 42, 4, 250, 576, 320, 32, 4, 3,
                                    [300, 17, 0, 260, 1], x_std=1.0, w_std=0.02,
                                    route_share=64, routing_seed=500 + m, base=base)
                    for m in range(1, 5)]
    dws = [DeviceWorkload(w) for w in wls]
    d0 = dws[0]
    desc = d0.desc(minibatch=128, mode=PERSIST, wait_timeout_us=TIMEOUT_US)
    ws = torch.empty(mok.mok_forward_workspace_size(desc, base.T, len(wls)), dtype=torch.uint8,
                     device="cuda")
    outs = [d0.new_out() for _ in wls]
    mok.mok_moe_forward_batches(desc, len(wls), [d.topk_idx for d in dws],
                                [d.topk_gate for d in dws], base.T, d0.x, d0.w_gu, d0.w_d,
                                outs, ws)
    assert mok.mok_device_status(ws) == 0
    for m, d in enumerate(dws):
        d.forward(minibatch=128, no_split_k=1)
        assert np.array_equal(d0.out_rows(outs[m]), d.out_rows(d.outs[0])), m
    r = oracle.forward(wls[3])
    check_layer_out(d0.out_rows(outs[3]), wls[3], r, "out m3")


def test_persistent_capacity_and_empty():
    import token_dispatch_grouped_top_amd as mok
    wl = W.small_pool(43, n_partitions=2, part_rows=64, H=128, I=128, E=16, k=2,
                      expert_base=0, counts=[40, 30])
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward(max_rows=50, minibatch=16, mode=PERSIST, wait_timeout_us=TIMEOUT_US)
    assert mok.mok_device_status(ws) == mok.MOK_ERR_CAPACITY
    assert np.all(dw.out_rows(dw.outs[0]) == 0x7FC1)
    wl = W.small_pool(44, n_partitions=2, part_rows=64, H=128, I=128, E=16, k=2,
                      expert_base=0, counts=[0, 0])
    dw = DeviceWorkload(wl)
    ws, _ = dw.forward(minibatch=16, mode=PERSIST, wait_timeout_us=TIMEOUT_US)
    assert mok.mok_device_status(ws) == 0
    assert np.all(dw.out_rows(dw.outs[0]) == 0x7FC1)


def test_persistent_tiny_wait_bound_ends_cleanly():
    """A 1-microsecond bound on every wait: the kernel either finishes (waits
    were already satisfied) or stops with MOK_ERR_DEVICE; it never hangs, and a
    following call on the same workspace works."""
    import token_dispatch_grouped_top_amd as mok
    wl = _case(False, 45)
    dw = DeviceWorkload(wl, n_out=2)
    ws, _ = dw.forward(out=dw.outs[0], minibatch=64, mode=PERSIST, wait_timeout_us=1)
    st = mok.mok_device_status(ws)
    assert st in (0, mok.MOK_ERR_DEVICE)
    ws, _ = dw.forward(out=dw.outs[1], minibatch=64, mode=PERSIST, wait_timeout_us=TIMEOUT_US)
    assert mok.mok_device_status(ws) == 0
    r = oracle.forward(wl)
    check_layer_out(dw.out_rows(dw.outs[1]), wl, r, "out after a timed-out call")
