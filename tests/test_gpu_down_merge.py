"""GPU tests of the down GEMM that merges single-slot tokens in its epilogue
(mok_expert_down_merge + mok_combine_slots_multi; the article's push combine:
a result goes straight back to its token).

The pair must write the same output rows, bit for bit, as mok_expert_down +
mok_combine_slots (which the oracle tests pin), leave the rows of tokens
without a local slot untouched, and store y exactly for the slots of tokens
with several local slots.  Cases: a ragged pool (tiles with tails, an empty
expert, tokens with up to k local slots) with bf16 activations, MXFP8
activations and MXFP8 weights, whole tiles and with the K split of the last
partial round.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import SENTINEL, DeviceWorkload, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("fmt,split,k", [("bf16", False, 4), ("bf16", True, 4), ("mx", False, 4),
                                         ("mx8", True, 4), ("bf16", False, 12)])
def test_down_merge_matches_down_and_merge(fmt, split, k):
    """k = 12: more picks per token than the 8 slot_of_assign entries the tile
    loads ahead."""
    import token_dispatch_grouped_top_amd as mok
    wl = W.small_pool(61, n_partitions=4, part_rows=250, H=576, I=320, E=16 if k == 4 else 40,
                      k=k, expert_base=3, counts=[300, 17, 0, 260, 1, 200] + [150] * (k - 4),
                      act_format=W.ACT_BF16 if fmt == "bf16" else W.ACT_MXFP8)
    if fmt == "mx8":
        wl.weight_format = 1
    dw = DeviceWorkload(wl, n_out=2)
    H, I = wl.H, wl.I
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R = int(ref["R"])
    d = dw.desc()
    w_gu, w_d = dw.weights(d)
    mx = fmt != "bf16"
    ring = torch.zeros((R, H), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    ring_sc = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda") if mx else None
    act = torch.zeros((R, I), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    act_sc = torch.zeros((R, I // 32), dtype=torch.uint8, device="cuda") if mx else None
    mok.mok_dispatch_gather(dw.x, H, k, s["aos"], s["offsets"], wl.n_local, 0, R, ring, ring_sc,
                            R, wl.act_format)
    ws = torch.zeros(mok.mok_gemm_workspace_size(), dtype=torch.uint8, device="cuda") if split \
        else None
    mok.mok_expert_gate_up(d, ring, ring_sc, R, s["offsets"], 0, R, w_gu, act, act_sc, R, ws)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # reference pair: y for every slot, then the full merge
    y_ref = torch.full((R, H), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_down(d, act, act_sc, R, s["offsets"], 0, R, w_d, y_ref, R, ws)
    mok.mok_combine_slots(y_ref, R, s["aos"], s["offsets"], wl.n_local, R, s["soa"],
                          dw.topk_gate, k, H, dw.outs[0], status)
    # merging pair
    y = torch.full((R, H), SENTINEL, dtype=torch.int16, device="cuda")
    plan = torch.empty((R, 16), dtype=torch.uint8, device="cuda")
    mok.mok_expert_down_merge(d, act, act_sc, R, s["offsets"], 0, R, w_d, y, R, s["aos"],
                              s["soa"], dw.topk_gate, dw.outs[1], plan, ws)
    mok.mok_combine_slots_multi(y, R, s["aos"], s["offsets"], wl.n_local, R, s["soa"],
                                dw.topk_gate, k, H, dw.outs[1], status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    out_ref, out = dw.out_rows(dw.outs[0]), dw.out_rows(dw.outs[1])
    assert np.array_equal(out, out_ref)
    soa = ref["slot_of_assign"].reshape(wl.T, k)
    n_local_slots = (soa >= 0).sum(1)
    assert np.all(out[n_local_slots == 0] == SENTINEL)
    assert (n_local_slots == 1).sum() > 0 and (n_local_slots >= 2).sum() > 0
    # y: exactly the rows of tokens with several local slots
    t_of = ref["assign_of_slot"][:R] // k
    multi = n_local_slots[t_of] >= 2
    yh, yr = to_host(y), to_host(y_ref)
    assert np.array_equal(yh[multi], yr[multi])
    assert np.all(yh[~multi] == SENTINEL)
    print(f"[down-merge] {fmt} split={split}: {int((n_local_slots == 1).sum())} tokens merged in "
          f"the epilogue, {int((n_local_slots >= 2).sum())} by the merge", flush=True)

