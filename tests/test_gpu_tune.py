"""GPU tests of the fused call's tuner (mok_tune_forward; tahou.com MoK
article, minibatch paragraph: the minibatch and the mover share are retuned
per shape).  The tuner picks one of the candidates it was given, reports a
positive time, and the layer run with its pick still meets the output bar
against the oracle; candidates that do not fit the workspace are skipped,
and with none left the call says so."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceWorkload, check_layer_out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _case():
    return W.small_pool(90, n_partitions=4, part_rows=250, H=576, I=320, E=32, k=4,
                        expert_base=3, counts=[300, 17, 0, 260, 1])


@pytest.mark.parametrize("mode,Ms,moves", [(0, [64, 256, 1000], []), (1, [128, 256], [8, 16])])
def test_tune_picks_a_candidate_that_runs(mode, Ms, moves):
    import token_dispatch_grouped_top_amd as mok
    wl = _case()
    dw = DeviceWorkload(wl)
    idx, gate = dw.routing()
    d = dw.desc(mode=mode, wait_timeout_us=500_000)
    need = max(mok.mok_forward_workspace_size(dw.desc(mode=mode, minibatch=M), wl.T, 1) for M in Ms)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    w_gu, w_d = dw.weights(d)
    best, ms = mok.mok_tune_forward(d, Ms, moves, 3, [idx], [gate], wl.T, dw.x, w_gu, w_d,
                                    [dw.outs[0]], ws)
    assert best.minibatch in Ms and ms > 0
    if moves:
        assert best.n_move_cus in moves
    assert best.mode == mode and best.hidden == wl.H
    out = dw.new_out()
    mok.mok_moe_forward_routed(best, idx, gate, wl.T, dw.x, w_gu, w_d, out, ws)
    assert mok.mok_device_status(ws) == 0
    r = oracle.forward(wl)
    check_layer_out(dw.out_rows(out), wl, r, "out of the tuned descriptor")


def test_tune_without_a_fitting_candidate():
    import token_dispatch_grouped_top_amd as mok
    wl = _case()
    dw = DeviceWorkload(wl)
    idx, gate = dw.routing()
    d = dw.desc()
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")   # smaller than any candidate needs
    w_gu, w_d = dw.weights(d)
    with pytest.raises(mok.MokError) as e:
        mok.mok_tune_forward(d, [64, 256], [], 2, [idx], [gate], wl.T, dw.x, w_gu, w_d,
                             [dw.outs[0]], ws)
    assert e.value.status == mok.MOK_ERR_UNSUPPORTED
