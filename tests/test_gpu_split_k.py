"""GPU tests of the K split of the grouped GEMMs' last, partial round of tiles.

The expert FFN (tahou.com MoK article, layout-planning and megakernel
paragraphs) is computed as whole 256 x 256 tiles; when the tiles of an XCD
leave a last round that would keep most of its CUs idle, those tiles are cut
into pieces of k-steps whose fp32 sums meet in a workspace.  This changes the
fp32 summation order only, so the bar is the layer's (gpu_harness
.assert_close_rms against the oracle), and in addition:
  - the pieces really ran: exactly the predicted partial slots of the
    workspace hold data (its counters are back at zero afterwards);
  - the result is deterministic: a second call gives the same bits;
  - whole tiles (no workspace) and split tiles agree within the bar.
Shapes: a last round after full ones, a single partial round and a few tall
tiles, bf16 and MXFP8; the test predicts which tiles are split and into how
many pieces (3 to 8) and checks the workspace against that.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceWorkload, check_y_rows, empty_u16, to_host

pytestmark = pytest.mark.gpu
BM = BN = 256


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _n_cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def _expected_slots(counts, n_tiles, nk, n_cus):
    """Partial slots the split fills, by the same rule as the kernel's decode and the
    launch's grid (rows of the window plus a partial tile per expert, plus n_cus / 32
    spare workgroups per XCD)."""
    mt = sum(-(-int(c) // BM) for c in counts)
    total, P, used = mt * n_tiles, n_cus // 8, set()
    grid_tiles = (-(-sum(counts) // BM) + len(counts)) * n_tiles
    gx = -(-grid_tiles // 8) + n_cus // 32
    for x in range(8):
        c = total // 8 + (1 if x < total % 8 else 0)
        rx = c % P
        if rx == 0:
            continue
        sp = min(P // rx, nk // 8, 8, 1 + (gx - c) // rx)
        if sp < 3:
            continue
        used.update(x * P + tt * sp + piece for tt in range(rx) for piece in range(sp))
    return used


def _check_workspace(ws, used, n_cus):
    import token_dispatch_grouped_top_amd as mok
    assert ws.numel() == mok.mok_gemm_workspace_size()
    cnt_bytes = -(-n_cus * 4 // 256) * 256
    assert int(ws[:cnt_bytes].count_nonzero()) == 0, "counters not back at zero"
    slots = ws[cnt_bytes:].view(n_cus, BM * BN * 4)
    filled = {int(i) for i in torch.nonzero(slots.ne(0).any(1)).flatten().tolist()}
    assert filled == used


def _case(name):
    # (counts, H, I) -- pool of 8 x 1024 tokens, top-8 over 64 experts.  Pieces per split
    # tile on 256 CUs (gate/up; down), bf16 / MXFP8:
    if name == "rounds":       # 276 tiles each: 4; -  /  -; -
        return [2300, 2100, 2000, 1900, 2200, 2050, 1950, 2100], 1024, 512
    if name == "rounds_k":     # down 280 tiles, 3-4 per XCD left: -; 3 or 4  /  -; -
        return [2600, 2100, 2000, 1900, 2200, 2050, 1950, 2100], 1024, 1024
    if name == "one_round":    # one busy expert, 2 tiles per XCD: 8; 4  /  4; -
        return [300, 0, 0, 0, 0, 0, 0, 0], 2048, 1024
    if name == "tall":         # down 2 tiles of K = 4096: -; 8  /  -; 8
        return [200, 100], 512, 4096
    raise ValueError(name)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("name", ["rounds", "rounds_k", "one_round", "tall"])
def test_split_tail_gemms(name, mx):
    import token_dispatch_grouped_top_amd as mok
    counts, H, I = _case(name)
    wl = W.pool_workload(f"split_{name}", 61, 8, 1024, H, I, 64, 8, 5, counts, x_std=1.0,
                         w_std=0.02, route_share=64,
                         act_format=W.ACT_MXFP8 if mx else W.ACT_BF16)
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    ref = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    R, n_cus, fmt = ref["R"], _n_cus(), wl.act_format
    assert np.array_equal(np.diff(ref["offsets"]), counts)
    ring = torch.zeros((R, H), dtype=torch.uint8 if mx else torch.int16, device="cuda")
    ring_sc = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda") if mx else None
    mok.mok_dispatch_gather(dw.x, H, wl.k, s["aos"], s["offsets"], wl.n_local, 0, R, ring,
                            ring_sc, R, fmt)
    d = dw.desc()
    bk = 64 if mx else 32
    wsb = mok.mok_gemm_workspace_size()

    def gate_up(ws):
        act = torch.zeros((R, I), dtype=torch.uint8 if mx else torch.int16, device="cuda")
        act_sc = torch.zeros((R, I // 32), dtype=torch.uint8, device="cuda") if mx else None
        mok.mok_expert_gate_up(d, ring, ring_sc, R, s["offsets"], 0, R, dw.w_gu, act, act_sc, R,
                               ws)
        return act, act_sc

    def down(act, act_sc, ws):
        y = empty_u16(R, H)
        mok.mok_expert_down(d, act, act_sc, R, s["offsets"], 0, R, dw.w_d, y, R, ws)
        return y

    # gate/up alone, split: the predicted slots are filled, counters end at zero
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    act_s, act_sc_s = gate_up(ws)
    torch.cuda.synchronize()
    _check_workspace(ws, _expected_slots(counts, -(-I // (BN // 2)), H // bk, n_cus), n_cus)
    act_s2, act_sc_s2 = gate_up(ws)                    # reuse: deterministic, counters reset
    assert torch.equal(act_s, act_s2)
    if mx:
        assert torch.equal(act_sc_s, act_sc_s2)
    # down alone, split, on the split activations
    ws2 = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    y_s = down(act_s, act_sc_s, ws2)
    torch.cuda.synchronize()
    _check_workspace(ws2, _expected_slots(counts, -(-H // BN), I // bk, n_cus), n_cus)
    assert torch.equal(y_s, down(act_s, act_sc_s, ws2))
    # whole tiles
    act_w, act_sc_w = gate_up(None)
    y_w = down(act_w, act_sc_w, None)
    torch.cuda.synchronize()
    # against the oracle on sampled slots (every expert's first, tile-edge and last rows)
    rng = np.random.default_rng(62)
    offs = ref["offsets"]
    sl = set(int(v) for v in rng.integers(0, R, 256))
    for e in range(len(counts)):
        lo, hi = int(offs[e]), int(offs[e + 1])
        sl.update(v for v in (lo, lo + 255, lo + 256, hi - 1) if lo <= v < hi)
    slots = np.array(sorted(sl), np.int64)
    xr = oracle.gather_rows(wl.x, wl.k, ref["assign_of_slot"], slots, mx)
    eos = oracle.expert_of_slots(offs, slots)
    idx = torch.as_tensor(slots, device="cuda")
    check_y_rows(to_host(y_s[idx]), wl, xr, eos, "y split")
    check_y_rows(to_host(y_w[idx]), wl, xr, eos, "y whole")


def test_split_workspace_errors():
    import token_dispatch_grouped_top_amd as mok
    wl = W.small_pool(63, n_partitions=2, part_rows=64, H=128, I=128, E=16, k=2,
                      expert_base=0, counts=[40, 30])
    dw = DeviceWorkload(wl)
    s = dw.schedule(dw.topk_idx)
    R = 70
    ring = torch.zeros((R, wl.H), dtype=torch.int16, device="cuda")
    act = torch.zeros((R, wl.I), dtype=torch.int16, device="cuda")
    ws = torch.zeros(mok.mok_gemm_workspace_size() - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mok.MokError) as e:
        mok.mok_expert_gate_up(dw.desc(), ring, None, R, s["offsets"], 0, R, dw.w_gu, act, None,
                               R, ws)
    assert e.value.status == mok.MOK_ERR_WORKSPACE
    # no_split_k = 1 ignores the workspace (every tile whole)
    mok.mok_expert_gate_up(dw.desc(no_split_k=1), ring, None, R, s["offsets"], 0, R, dw.w_gu,
                           act, None, R, ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
