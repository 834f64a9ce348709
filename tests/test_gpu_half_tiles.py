"""GPU test of the half-width tail tiles of the y-storing grouped GEMMs.

The expert FFN's down GEMM (tahou.com MoK article, layout-planning and
megakernel paragraphs) runs 256 x 256 tiles in rounds over the CUs.  Where the
last round of an XCD's tiles would fill at most half of its CUs (and no K split
is taken), each of those tail tiles runs as two 256 x 128 jobs instead, half of
them dealt before the whole tiles and half after.  The shape here gives every
XCD 48 tiles on 32 CUs: 32 whole tiles and 32 half-width jobs per XCD.
Checked: every y element of every routed slot is written (no job dropped or
mapped twice onto the same columns), sampled slots (the first and last rows of
each expert, tile edges, random ones) equal the oracle within the rounding
bands, and the merging down GEMM plus the merge of multi-slot tokens equals the
plain down GEMM plus the slot-driven merge bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import SENTINEL, DeviceWorkload, check_y_rows, empty_u16, to_host

pytestmark = pytest.mark.gpu
BM = BN = 256


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("mx", [False, True])
def test_half_width_tail_tiles(mx):
    import token_dispatch_grouped_top_amd as mok
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    counts, H, I = [1536] * 16, 1024, 256
    tiles = sum(-(-c // BM) for c in counts) * (H // BN)
    per_xcd, P = tiles // 8, n_cus // 8
    if not (tiles % 8 == 0 and 0 < per_xcd % P <= P // 2):
        pytest.skip(f"the shape leaves no half-width tail on {n_cus} CUs")
    wl = W.pool_workload("half_tiles", 91, 16, 1024, H, I, 64, 8, 3, counts, x_std=1.0,
                         w_std=0.02, route_share=64,
                         act_format=W.ACT_MXFP8 if mx else W.ACT_BF16)
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R, fmt = ref["R"], wl.act_format
    ring = torch.zeros((R, H), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    ring_sc = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda") if mx else None
    mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, 0, R, ring,
                            ring_sc, R, fmt)
    d = dw.desc()
    ws = torch.zeros(mok.mok_gemm_workspace_size(), dtype=torch.uint8, device="cuda")
    act = torch.zeros((R, I), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    act_sc = torch.zeros((R, I // 32), dtype=torch.uint8, device="cuda") if mx else None
    mok.mok_expert_gate_up(d, ring, ring_sc, R, s["offsets"], 0, R, dw.w_gu, act, act_sc, R, ws)
    y = torch.full((R, H), SENTINEL, dtype=torch.int16, device="cuda")
    mok.mok_expert_down(d, act, act_sc, R, s["offsets"], 0, R, dw.w_d, y, R, ws)
    torch.cuda.synchronize()
    assert int((y == SENTINEL).sum()) == 0, "y elements left unwritten"
    assert int(ws.count_nonzero()) == 0, "no K split expected here (workspace untouched)"

    # sampled slots against the oracle: every expert's first and last rows, the
    # rows around its 256-row tile edges, and random slots
    rng = np.random.default_rng(92)
    offs = ref["offsets"]
    sl = set(int(v) for v in rng.integers(0, R, 192))
    for e in range(len(counts)):
        lo, hi = int(offs[e]), int(offs[e + 1])
        sl.update(v for v in (lo, lo + 255, lo + 256, lo + 1279, lo + 1280, hi - 1) if lo <= v < hi)
    slots = np.array(sorted(sl), np.int64)
    xr = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], slots, mx)
    eos = oracle.expert_of_slots(offs, slots)
    st = check_y_rows(to_host(y[torch.as_tensor(slots, device="cuda")]), wl, xr, eos,
                      f"y half-width tails ({'mxfp8' if mx else 'bf16'})")
    print(f"[half tiles] {'mxfp8' if mx else 'bf16'}: {len(slots)} sampled slots, "
          f"max|d|/RMS = {st['strict']:.3e}")

    # the merging down GEMM (same tiles and jobs) + the multi-slot merge against the
    # plain down GEMM + the slot-driven merge
    out_a, out_b = dw.new_out(), dw.new_out()
    mok.mok_combine_slots(y, R, s["aos"], s["offsets"], wl.n_local, R, s["soa"], dw.topk_gate,
                          wl.k, H, out_a)
    y_m = empty_u16(R, H)
    plan = torch.zeros((R, 16), dtype=torch.uint8, device="cuda")
    mok.mok_expert_down_merge(d, act, act_sc, R, s["offsets"], 0, R, dw.w_d, y_m, R, s["aos"],
                              s["soa"], dw.topk_gate, out_b, plan, ws)
    mok.mok_combine_slots_multi(y_m, R, s["aos"], s["offsets"], wl.n_local, R, s["soa"],
                                dw.topk_gate, wl.k, H, out_b)
    torch.cuda.synchronize()
    assert np.array_equal(dw.out_rows(out_a), dw.out_rows(out_b)), "merged outputs differ"
