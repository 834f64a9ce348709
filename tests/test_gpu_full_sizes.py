"""Parity at the full workload sizes, in the launch configuration bench.py times.

Workloads (seeded, synthetic): the hidden 7168 / intermediate 2048 expert
share with balanced counts (8192 routed rows from 72 partitions x 1024
tokens, 8 of 384 experts, top-8), the same shape with Zipf-skewed counts and
MXFP8 activations, the Mixtral-shaped layer (4096 tokens, hidden 4096,
intermediate 14336, 8 experts, top-2) and 8 macrobatches streamed through one
ring.  Bit-exact in full: routing ids, counts, offsets, slot_of_assign,
assign_of_slot, windows; dispatched rows on sampled slots.  Sampled against
the oracle row by row: expert outputs y and merged rows out (bar: see
gpu_harness.assert_close_rms).  In full on the GPU: rows of tokens with no
local assignment keep their sentinel; persistent == stream-ordered with whole
tiles (no_split_k = 1), bit for bit.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import SENTINEL, DeviceWorkload, assert_close_rms, colblk_rows, colblk_scales, to_host

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _sample_slots(offsets, rng, extra=8):
    s = set()
    R = int(offsets[-1])
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for v in (lo, lo + 1, lo + 255, lo + 256, (lo + hi) // 2, hi - 1):
            if lo <= v < hi:
                s.add(v)
    s.update(int(v) for v in rng.integers(0, R, extra))
    return np.array(sorted(s), np.int64)


def _sample_tokens(soa, k, rng, n=48):
    routed = np.nonzero((soa.reshape(-1, k) >= 0).any(1))[0]
    return np.sort(rng.choice(routed, size=min(n, routed.size), replace=False))


def _unwritten_keep_sentinel(dw, out, written_tokens):
    full = torch.cat(out.parts, 0)
    mask = torch.ones(full.shape[0], dtype=torch.bool, device="cuda")
    mask[torch.as_tensor(written_tokens, device="cuda")] = False
    rows = full[mask]
    assert bool((rows == SENTINEL).all()), "a token without local assignments was written"


def _run_bench_step(wl):
    import bench
    dw = DeviceWorkload(wl)
    max_rows = bench.BENCH_MAX_ROWS if not wl.routing_from_logits else wl.T * wl.k
    st = bench.Step(dw, max_rows)
    st.run()
    torch.cuda.synchronize()
    assert int(st.status.item()) == 0
    return dw, st


def _check_pool_case(wl, tol):
    dw, st = _run_bench_step(wl)
    rng = np.random.default_rng(wl.seed)
    mx = wl.act_format == W.ACT_MXFP8
    # route of this GPU's own source tokens, in full
    idx_o, gate_o = oracle.route_topk(wl.logits, wl.k)
    assert np.array_equal(to_host(st.r_idx), idx_o)
    g = to_host(st.r_gate).astype(np.float64)
    assert np.all(np.abs(g - gate_o) <= 2.0 ** -19 * gate_o)
    # schedule and windows, in full
    sch = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    assert np.array_equal(to_host(st.counts), sch["counts"])
    assert np.array_equal(to_host(st.offsets), sch["offsets"])
    assert np.array_equal(to_host(st.soa), sch["slot_of_assign"])
    assert np.array_equal(to_host(st.aos)[:sch["R"]], sch["assign_of_slot"])
    assert np.array_equal(to_host(st.win), oracle.windows(sch["offsets"], st.M, st.nwin))
    # dispatched rows (bit-exact) and expert outputs on sampled slots
    slots = _sample_slots(sch["offsets"], rng)
    xr = oracle.gather_rows(wl.x, wl.k, sch["assign_of_slot"], slots, mx)
    ring = colblk_rows(st.ring, st.cap)[slots]
    if mx:
        assert np.array_equal(ring, xr[0])
        assert np.array_equal(colblk_scales(st.ring_sc, st.cap)[slots], xr[1])
    else:
        assert np.array_equal(ring, xr)
    y_ref = oracle.ffn_rows(xr, oracle.expert_of_slots(sch["offsets"], slots), wl.w_gu, wl.w_d, mx)
    y_got = to_host(st.y[torch.as_tensor(slots, device="cuda")])
    assert_close_rms(y_got, y_ref, tol, "y")
    # merged rows on sampled tokens; untouched rows in full
    toks = _sample_tokens(sch["slot_of_assign"], wl.k, rng)
    r = oracle.forward(wl, tokens=toks)
    got = dw.out_rows(dw.outs[0], toks)
    assert r["written"].all()
    rel = assert_close_rms(got, r["out"], tol, "out")
    written = np.nonzero((sch["slot_of_assign"].reshape(wl.T, wl.k) >= 0).any(1))[0]
    _unwritten_keep_sentinel(dw, dw.outs[0], written)
    return dw, st, rel


def _persistent_equals(dw, st, **kw):
    """Persistent == stream-ordered with whole tiles, bit for bit; both within the bar of
    the bench step's output (which splits the GEMMs' last round along K)."""
    import token_dispatch_grouped_top_amd as mok
    out, ref = dw.new_out(), dw.new_out()
    ws, _ = dw.forward(out=out, max_rows=st.cap, mode=1, **kw)
    assert mok.mok_device_status(ws) == 0
    ws, _ = dw.forward(out=ref, max_rows=st.cap, no_split_k=1, **kw)
    assert mok.mok_device_status(ws) == 0
    for a, b in zip(out.parts, ref.parts):
        assert torch.equal(a, b)
    return out


def test_kimi_share_balanced():
    dw, st, rel = _check_pool_case(W.kimi_share(), 2e-2)
    print(f"kimi share: max|d|/RMS = {rel:.3e}")
    _persistent_equals(dw, st, minibatch=2560)


def test_kimi_share_zipf_mxfp8():
    dw, st, rel = _check_pool_case(W.kimi_zipf_mxfp8(), 6e-2)
    print(f"kimi zipf mxfp8: max|d|/RMS = {rel:.3e}")
    _persistent_equals(dw, st, minibatch=2560)


def test_mixtral_layer():
    wl = W.mixtral()
    dw, st = _run_bench_step(wl)
    rng = np.random.default_rng(7)
    idx_o, gate_o = oracle.route_topk(wl.logits, wl.k)
    assert np.array_equal(to_host(dw.topk_idx), idx_o)
    g = to_host(dw.topk_gate).astype(np.float64)
    assert np.all(np.abs(g - gate_o) <= 2.0 ** -19 * gate_o)
    sch = oracle.build_schedule(idx_o, 0, 8)
    assert np.array_equal(to_host(st.offsets), sch["offsets"])
    assert np.array_equal(to_host(st.aos)[:sch["R"]], sch["assign_of_slot"])
    toks = np.sort(rng.choice(wl.T, 24, replace=False))
    r = oracle.forward(wl, tokens=toks)
    rel = assert_close_rms(dw.out_rows(dw.outs[0], toks), r["out"], 2e-2, "out")
    print(f"mixtral: max|d|/RMS = {rel:.3e}")


def test_streaming_macrobatches():
    import token_dispatch_grouped_top_amd as mok
    wls = W.streaming(8)
    dws = [DeviceWorkload(wls[0])]
    for w in wls[1:]:      # share the pool and weights on the device too
        d = DeviceWorkload.__new__(DeviceWorkload)
        d.wl, d.x_parts, d.x, d.w_gu, d.w_d = w, dws[0].x_parts, dws[0].x, dws[0].w_gu, dws[0].w_d
        from gpu_harness import to_dev
        d.logits, d.topk_idx, d.topk_gate = to_dev(w.logits), to_dev(w.topk_idx), to_dev(w.topk_gate)
        d.outs = [d.new_out()]
        dws.append(d)
    d0 = dws[0]
    desc = d0.desc(max_rows=8192, minibatch=2560, mode=1)
    ws = torch.empty(mok.mok_forward_workspace_size(desc, d0.wl.T, 8), dtype=torch.uint8,
                     device="cuda")
    outs = [d0.new_out() for _ in dws]
    mok.mok_moe_forward_batches(desc, 8, [d.topk_idx for d in dws], [d.topk_gate for d in dws],
                                d0.wl.T, d0.x, d0.w_gu, d0.w_d, outs, ws)
    assert mok.mok_device_status(ws) == 0
    for m, d in enumerate(dws):
        d.forward(max_rows=8192, minibatch=2560, no_split_k=1)   # standalone, stream-ordered
        for a, b in zip(outs[m].parts, d.outs[0].parts):
            assert torch.equal(a, b), m
    rng = np.random.default_rng(9)
    wl7 = wls[7]
    sch = oracle.build_schedule(wl7.topk_idx, wl7.expert_base, wl7.n_local)
    toks = _sample_tokens(sch["slot_of_assign"], wl7.k, rng, n=24)
    r = oracle.forward(wl7, tokens=toks)
    assert_close_rms(d0.out_rows(outs[7], toks), r["out"], 2e-2, "out m7")
