#!/usr/bin/env python3
"""Benchmark of one GPU's share of the MoK forward MoE layer (libmok, MI355X).

Workload: the hidden 7168 / expert intermediate 2048 expert share -- 8192
routed rows for 8 local experts (of 384, top-8) pulled from a pool of
72 source partitions x 1024 tokens in HBM, balanced counts, bf16, seeded
synthetic data.  The route step runs on this GPU's own 1024 source tokens.

One step = the whole hot path through the C-ABI on one stream:
route -> schedule -> windows -> pull gather -> gate/up + SwiGLU grouped GEMM
-> down grouped GEMM -> weighted combine.  HIP events between the calls (on
the launch stream) give each kernel's duration; the dominant kernel (the
gate/up grouped GEMM) is priced against the bf16 MFMA peak.  Inputs are
resident in HBM before timing starts.

Prints ONE JSON line.  Extra reports go to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "MoE fwd ms/layer + grouped-GEMM TFLOP/s, dispatch/combine GB/s (7168/2048)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (the block-scaled MXFP8 GEMMs)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
BENCH_MAX_ROWS = 8192         # row capacity handed to the layer (= routed rows here)

# HBM bytes moved by one gate/up launch, from two rocprofv3 --pmc runs of this bench (FETCH_SIZE
# scaled by 2.0 and WRITE_SIZE by 1.0: what the counters read for a plain 1 GiB copy), keyed by
# workload and by a hash of the GEMM sources they were taken on; any other source gives null.
GATE_UP_TRAFFIC = {
    "kimi_share_R8192_H7168_I2048_E384_k8_local8": ("136c9b7ea24adaa0", 740556123),
    "kimi_zipf_mxfp8_R8192_H7168_I2048_E384_k8_local8": ("136c9b7ea24adaa0", 1016708215),
    "kimi_full_mxfp8_R8192_H7168_I2048_E384_k8_local8": ("136c9b7ea24adaa0", 382201381),
}
GEMM_SOURCES = ("token_dispatch_grouped_top_amd/csrc/gemm_tile.h",
                "token_dispatch_grouped_top_amd/csrc/gemm.hip",
                "token_dispatch_grouped_top_amd/csrc/mok_internal.h",
                "token_dispatch_grouped_top_amd/csrc/gemm_tile_mx8.h")


def gate_up_traffic(workload: str):
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), f), "rb") as fh:
            h.update(fh.read())
    rec = GATE_UP_TRAFFIC.get(workload)
    return rec[1] if rec and rec[0] == h.hexdigest()[:16] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_workload(name: str):
    import workloads as W
    if name == "kimi":
        return W.kimi_share()
    if name == "kimi_zipf_mxfp8":
        return W.kimi_zipf_mxfp8()
    if name == "kimi_full_mxfp8":
        return W.kimi_full_mxfp8()
    if name == "kimi_zipf_full_mxfp8":
        return W.kimi_zipf_full_mxfp8()
    if name == "mixtral":
        return W.mixtral()
    if name == "tiny":
        return W.tiny()
    raise ValueError(name)


class Step:
    """Buffers and the call sequence of one step of the layer."""

    def __init__(self, dw, max_rows: int):
        import torch
        import token_dispatch_grouped_top_amd as mok
        self.mok, self.dw, wl = mok, dw, dw.wl
        self.cap = max_rows
        # weights packed once into the GEMMs' tile order (set-up, like loading a checkpoint)
        self.desc = dw.desc(max_rows=max_rows, weights_packed=1)
        self.w_gu, self.w_d = dw.weights(self.desc)
        self.M = mok.mok_forward_minibatch(self.desc, wl.T)
        mx = wl.act_format == mok.MOK_ACT_MXFP8_E4M3
        dev = "cuda"
        A = wl.T * wl.k
        self.route_T, self.route_E = dw.logits.shape
        self.r_idx = torch.empty((self.route_T, wl.k), dtype=torch.int32, device=dev)
        self.r_gate = torch.empty((self.route_T, wl.k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(wl.n_local, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(wl.n_local + 1, dtype=torch.int32, device=dev)
        self.soa = torch.empty(A, dtype=torch.int32, device=dev)
        self.aos = torch.empty(A, dtype=torch.int32, device=dev)
        self.sched_ws = torch.empty(mok.mok_schedule_workspace_size(wl.T, wl.k, wl.n_local),
                                    dtype=torch.uint8, device=dev)
        self.nwin = -(-max_rows // self.M)
        self.win = torch.empty((self.nwin, wl.n_local + 1), dtype=torch.int32, device=dev)
        cap, H, I = max_rows, wl.H, wl.I
        self.ring = torch.empty((cap, H), dtype=torch.uint8 if mx else torch.int16, device=dev)
        self.ring_sc = torch.empty((cap, H // 32), dtype=torch.uint8, device=dev) if mx else None
        self.act = torch.empty((cap, I), dtype=torch.uint8 if mx else torch.int16, device=dev)
        self.act_sc = torch.empty((cap, I // 32), dtype=torch.uint8, device=dev) if mx else None
        self.y = torch.empty((cap, H), dtype=torch.int16, device=dev)
        self.plan = torch.empty((cap, 16), dtype=torch.uint8, device=dev)   # merge plan records
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        # K split of the GEMMs' last partial round: counters must start at zero
        self.gemm_ws = torch.zeros(mok.mok_gemm_workspace_size(), dtype=torch.uint8, device=dev)
        self.names = ["route", "schedule", "gather", "gate_up", "down", "combine"]

    def run(self, ev=None):
        """The hot path.  ev: {i: event} recorded before call i (i = len(names): after the
        last call); every event marker on the stream costs a kernel drain, so the timed
        region records only the two around the dominant launch."""
        mok, dw, wl = self.mok, self.dw, self.dw.wl
        rec = (lambda i: ev[i].record() if i in ev else None) if ev else (lambda i: None)
        rec(0)
        if wl.routing_from_logits:      # every token routed here
            mok.mok_route_topk(dw.logits, self.route_T, self.route_E, wl.k, dw.topk_idx,
                               dw.topk_gate)
        else:                           # this GPU's own source tokens; the pool's routing is given
            mok.mok_route_topk(dw.logits, self.route_T, self.route_E, wl.k, self.r_idx, self.r_gate)
        rec(1)
        idx, gate = dw.topk_idx, dw.topk_gate
        # the schedule and its window table (two launches: count, then the
        # scatter whose first block also writes the windows)
        mok.mok_build_schedule_windows(idx, wl.T, wl.k, wl.expert_base, wl.n_local, self.counts,
                                       self.offsets, self.soa, self.aos, self.M, self.nwin,
                                       self.win, self.sched_ws)
        rec(2)
        mok.mok_dispatch_gather(dw.x, wl.H, wl.k, self.aos, self.offsets, wl.n_local, 0, self.cap,
                                self.ring, self.ring_sc, self.cap, wl.act_format, self.status)
        rec(3)
        mok.mok_expert_gate_up(self.desc, self.ring, self.ring_sc, self.cap, self.offsets, 0,
                               self.cap, self.w_gu, self.act, self.act_sc, self.cap, self.gemm_ws)
        rec(4)
        # the down GEMM writes each single-slot token's output row itself (bf16(g y));
        # the merge then takes the tokens with several local slots
        mok.mok_expert_down_merge(self.desc, self.act, self.act_sc, self.cap, self.offsets, 0,
                                  self.cap, self.w_d, self.y, self.cap, self.aos, self.soa, gate,
                                  dw.outs[0], self.plan, self.gemm_ws)
        rec(5)
        mok.mok_combine_slots_multi(self.y, self.cap, self.aos, self.offsets, wl.n_local, self.cap,
                                    self.soa, gate, wl.k, wl.H, dw.outs[0], self.status)
        rec(6)


def time_streaming(mok, DeviceWorkload, n_macro: int = 8):
    """8 Kimi-shaped macrobatches (one pool, one weight set, own routing each)
    through one ring: ms per macrobatch of mok_moe_forward_batches per mode."""
    import torch
    import workloads as W
    from gpu_harness import to_dev
    wls = W.streaming(n_macro)
    d0 = DeviceWorkload(wls[0])
    idx = [d0.topk_idx] + [to_dev(w.topk_idx) for w in wls[1:]]
    gate = [d0.topk_gate] + [to_dev(w.topk_gate) for w in wls[1:]]
    outs = [d0.new_out() for _ in wls]
    res = {}
    for mode, M, n_move in ((0, 2560, 0), (0, 8192, 0), (1, 2560, 0), (1, 4096, 0), (1, 8192, 0)):
        d = d0.desc(max_rows=BENCH_MAX_ROWS, minibatch=M, mode=mode, n_move_cus=n_move,
                    weights_packed=1)
        w_gu, w_d = d0.weights(d)
        ws = torch.empty(mok.mok_forward_workspace_size(d, d0.wl.T, n_macro), dtype=torch.uint8,
                         device="cuda")
        run = lambda: mok.mok_moe_forward_batches(d, n_macro, idx, gate, d0.wl.T, d0.x, w_gu,
                                                  w_d, outs, ws)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            run()
        e1.record()
        torch.cuda.synchronize()
        assert mok.mok_device_status(ws) == 0
        key = ("stream" if mode == 0 else "persistent_auto_split") + f"_M{M}"
        res[key] = round(e0.elapsed_time(e1) / 3 / n_macro, 4)
        log(f"[bench] streaming {n_macro} macrobatches, {key}: {res[key]:.4f} ms per macrobatch")
    return res


def time_merge_all_slots(mok, st, reps: int = 20) -> dict:
    """The weighted merge as one standalone kernel over every routed slot
    (mok_combine_slots, the slot-driven merge of all R slots from a y that
    holds every slot's row), timed with HIP events after the timed region: the
    layer step itself merges the single-slot tokens in the down GEMM's epilogue
    and only the rest in mok_combine_slots_multi.  Algorithmic bytes: every
    slot's y row read and every written token's row stored, R H 2 + T_out H 2,
    plus the routing words R (1 + k) 4."""
    import numpy as np
    import torch
    from gpu_harness import to_host
    dw, wl = st.dw, st.dw.wl
    mok.mok_expert_down(st.desc, st.act, st.act_sc, st.cap, st.offsets, 0, st.cap, st.w_d, st.y,
                        st.cap, st.gemm_ws)
    run = lambda: mok.mok_combine_slots(st.y, st.cap, st.aos, st.offsets, wl.n_local, st.cap,
                                        st.soa, dw.topk_gate, wl.k, wl.H, dw.outs[0], st.status)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for i in range(reps):
        ev[2 * i].record()
        run()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    ms = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)]))
    R = int(to_host(st.offsets)[-1])
    soa = to_host(st.soa).reshape(wl.T, wl.k)
    T_out = int(((soa >= 0).sum(1) > 0).sum())
    b = R * wl.H * 2 + T_out * wl.H * 2 + R * (1 + wl.k) * 4
    gbs = b / (ms * 1e-3) / 1e9
    return {"kernel": "mok_combine_slots over all R slots", "ms": round(ms, 4),
            "algorithmic_bytes": b, "GBps": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def mover_sweep(mok, DeviceWorkload) -> dict:
    """The persistent kernel's mover count against the stream path: ms per macrobatch of
    mok_moe_forward_batches on the streaming workload, one macrobatch at M = 1024, 2560 and
    4096 and 8 macrobatches at M = 2560, 4096 and 8192, for n_move_cus in 40 .. 128."""
    import torch
    import workloads as W
    from gpu_harness import to_dev
    n_macro = 8
    wls = W.streaming(n_macro)
    d0 = DeviceWorkload(wls[0])
    idx = [d0.topk_idx] + [to_dev(w.topk_idx) for w in wls[1:]]
    gate = [d0.topk_gate] + [to_dev(w.topk_gate) for w in wls[1:]]
    outs = [d0.new_out() for _ in wls]
    d = d0.desc(max_rows=BENCH_MAX_ROWS, minibatch=BENCH_MAX_ROWS, mode=0, weights_packed=1)
    w_gu, w_d = d0.weights(d)
    ws = torch.empty(mok.mok_forward_workspace_size(d, d0.wl.T, n_macro), dtype=torch.uint8,
                     device="cuda")
    for _ in range(30):            # the chip's clock falls within milliseconds of idling
        mok.mok_moe_forward_batches(d, n_macro, idx, gate, d0.wl.T, d0.x, w_gu, w_d, outs, ws)
    torch.cuda.synchronize()
    del ws
    res = {}
    for nm, M in ((1, 1024), (1, 2560), (1, 4096), (n_macro, 2560), (n_macro, 4096), (n_macro, 8192)):
        row = {}
        for mode, n_move in [(0, 0)] + [(1, n) for n in (40, 48, 56, 64, 80, 96, 128)]:
            d = d0.desc(max_rows=BENCH_MAX_ROWS, minibatch=M, mode=mode, n_move_cus=n_move,
                        weights_packed=1)
            ws = torch.empty(mok.mok_forward_workspace_size(d, d0.wl.T, nm), dtype=torch.uint8,
                             device="cuda")
            run = lambda: mok.mok_moe_forward_batches(d, nm, idx[:nm], gate[:nm], d0.wl.T, d0.x,
                                                      w_gu, w_d, outs[:nm], ws)
            for _ in range(3):
                run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 6 if nm == 1 else 3
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            assert mok.mok_device_status(ws) == 0
            row["stream" if mode == 0 else str(n_move)] = round(e0.elapsed_time(e1) / reps / nm, 4)
            del ws
        res[f"macrobatches{nm}_M{M}"] = row
        log(f"[bench] mover sweep, {nm} macrobatch(es), M={M}: {row}")
    return res


def measured_peaks(reps: int = 10) -> dict:
    """Measured references on this GPU: a plain 1 GiB device-to-device copy
    (torch copy_, bytes read + written over its time: the HBM rate a pure
    stream reaches here) and a dense bf16 GEMM from the vendor library
    (torch.matmul on contiguous 8192 x 8192 x 8192 operands, hipBLASLt)."""
    import numpy as np
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record()
            fn()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        return float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)]))
    copy_ms = timed(lambda: dst.copy_(src))
    mm_ms = timed(lambda: torch.matmul(a, b))
    del src, dst, a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_1GiB_GBps": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
            "hipblaslt_bf16_8192cube_tflops": round(2 * 8192 ** 3 / (mm_ms * 1e-3) / 1e12, 1)}


def time_router_gemm(mok, wl, reps: int = 20):
    """mok_route_topk_gemm on this workload's routed tokens' shape (T_route x H
    against E router rows, seeded N(0, 1) tokens and N(0, 1/H) router
    weights): not part of the timed step, whose routing comes from the
    workload's logits."""
    import numpy as np
    import torch
    import workloads as W
    T, E, H, k = int(wl.logits.shape[0]), wl.E, wl.H, wl.k
    x, w = W.router_inputs(77, T, H, E)
    xd, wd = torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(w.view(np.int16)).cuda()
    ws = torch.empty(max(mok.mok_route_gemm_workspace_size(T, E, H), 1), dtype=torch.uint8,
                     device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    for _ in range(3):
        mok.mok_route_topk_gemm(xd, wd, T, H, E, k, ws, idx, gate)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mok.mok_route_topk_gemm(xd, wd, T, H, E, k, ws, idx, gate)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flop = 2.0 * T * E * H
    return {"T": T, "E": E, "H": H, "k": k, "ms": round(ms, 5),
            "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
            "input_GBps": round((T + E) * H * 2 / (ms * 1e-3) / 1e9, 1)}


def time_backward(mok, dw, st, reps: int = 10):
    """The backward of the layer share after a forward step (bf16 activations
    and weights; MXFP8 activations through the _mx calls, with bf16 or MXFP8
    weights, the latter packed for each GEMM's contraction): merge backward
    (dy, dgate), the expert FFN backward (recompute of h, down dgrad with the
    SwiGLU backward, gate/up dgrad), dispatch backward (dx), weight gradients
    (transposes + two GEMMs over each expert's slots).  Seeded N(0, 1) dout for
    every pool token; per-call means over `reps` calls."""
    import numpy as np
    import torch
    import workloads as W
    from gpu_harness import to_dev
    wl = dw.wl
    mx = wl.act_format == mok.MOK_ACT_MXFP8_E4M3
    H, I, k, cap = wl.H, wl.I, wl.k, st.cap
    R = int(st.offsets[-1].item())
    d = dw.desc(max_rows=cap, weights_packed=1)        # h recomputed with the packed gate/up
    dout = mok.Tokens([to_dev(W.normal_bf16(np.random.SeedSequence(900 + p), wl.part_rows * H, 1.0)
                              .reshape(wl.part_rows, H)) for p in range(wl.n_partitions)],
                      wl.part_rows)
    dx = dw.new_out()
    a, b = mok.mok_packed_weights_bwd_size(d)
    gu_t = torch.empty(a, dtype=torch.uint8, device="cuda")
    d_t = torch.empty(b, dtype=torch.uint8, device="cuda")
    mok.mok_pack_weights_bwd(d, dw.w_gu, dw.w_d, gu_t, d_t)
    tok = torch.uint8 if mx else torch.int16
    scales = (lambda n: torch.empty((cap, n // 32), dtype=torch.uint8, device="cuda")) if mx \
        else (lambda n: None)
    dy, dy_sc = torch.empty((cap, H), dtype=tok, device="cuda"), scales(H)
    dgate = torch.empty((wl.T, k), dtype=torch.float32, device="cuda")
    h = torch.empty((cap, 2 * I), dtype=torch.int16, device="cuda")
    dh, dh_sc = torch.empty((cap, 2 * I), dtype=tok, device="cuda"), scales(2 * I)
    dxs = torch.empty((cap, H), dtype=torch.int16, device="cuda")
    dwgu = torch.empty((wl.n_local, 2 * I, H), dtype=torch.int16, device="cuda")
    dwd = torch.empty((wl.n_local, H, I), dtype=torch.int16, device="cuda")
    wws = torch.empty(mok.mok_wgrad_workspace_size(d, cap), dtype=torch.uint8, device="cuda")
    hsv = torch.empty((cap, 2 * I), dtype=torch.int16, device="cuda")
    dispatch_bwd = lambda: mok.mok_dispatch_backward(dxs, cap, st.aos, st.offsets, wl.n_local, cap,
                                                     st.soa, k, H, dx, st.status)
    gate_up_plain = lambda: mok.mok_expert_gate_up(d, st.ring, st.ring_sc, cap, st.offsets, 0, cap,
                                                   st.w_gu, st.act, st.act_sc, cap, st.gemm_ws)
    if mx:
        calls = {
            "combine_bwd": lambda: mok.mok_combine_backward_mx(dout, st.y, cap, st.aos, st.offsets,
                                                               wl.n_local, cap, dw.topk_gate, k, H,
                                                               dy, dy_sc, cap, dgate, st.status),
            "ffn_bwd": lambda: mok.mok_expert_ffn_backward_mx(d, st.ring, st.ring_sc, cap, dy, dy_sc,
                                                              st.offsets, 0, cap, st.w_gu, gu_t, d_t,
                                                              h, False, dh, dh_sc, dxs, cap),
            "dispatch_bwd": dispatch_bwd,
            "wgrad": lambda: mok.mok_expert_wgrad_mx(d, st.ring, st.ring_sc, cap, st.act, st.act_sc,
                                                     cap, dy, dy_sc, dh, dh_sc, cap, st.offsets,
                                                     dwgu, dwd, wws),
            "gate_up_save_h": lambda: mok.mok_expert_gate_up_save_h_mx(
                d, st.ring, st.ring_sc, cap, st.offsets, 0, cap, st.w_gu, st.act, st.act_sc, cap,
                hsv, st.gemm_ws),
            "gate_up_plain": gate_up_plain,
            "ffn_bwd_saved": lambda: mok.mok_expert_ffn_backward_mx(
                d, None, None, cap, dy, dy_sc, st.offsets, 0, cap, None, gu_t, d_t, hsv, True, dh,
                dh_sc, dxs, cap),
        }
    else:
        calls = {
            "combine_bwd": lambda: mok.mok_combine_backward(dout, st.y, cap, st.aos, st.offsets,
                                                            wl.n_local, cap, dw.topk_gate, k, H, dy,
                                                            cap, dgate, st.status),
            "ffn_bwd": lambda: mok.mok_expert_ffn_backward(d, st.ring, cap, dy, st.offsets, 0, cap,
                                                           st.w_gu, gu_t, d_t, h, dh, dxs, cap),
            "dispatch_bwd": dispatch_bwd,
            "wgrad": lambda: mok.mok_expert_wgrad(d, st.ring, cap, st.act, cap, dy, dh, cap,
                                                  st.offsets, dwgu, dwd, wws),
            # h kept by the forward instead of recomputed: the forward's gate/up that also
            # stores h (timed whole, to set against the plain gate/up), then the backward from it
            "gate_up_save_h": lambda: mok.mok_expert_gate_up_save_h(d, st.ring, cap, st.offsets, 0,
                                                                    cap, st.w_gu, st.act, cap, hsv,
                                                                    st.gemm_ws),
            "gate_up_plain": gate_up_plain,
            "ffn_bwd_saved": lambda: mok.mok_expert_ffn_backward_saved(d, dy, st.offsets, 0, cap,
                                                                       gu_t, d_t, hsv, dh, dxs, cap),
        }
    out = {}
    for name, f in calls.items():
        f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / reps, 4)
    assert int(st.status.item()) == 0
    flop = 4.0 * R * H * I + 2.0 * R * H * I + 4.0 * R * H * I   # h, da, dx_s
    out["ffn_bwd_tflops"] = round(flop / (out["ffn_bwd"] * 1e-3) / 1e12, 1)
    out["wgrad_tflops"] = round(6.0 * R * H * I / (out["wgrad"] * 1e-3) / 1e12, 1)
    out["total_ms"] = round(out["combine_bwd"] + out["ffn_bwd"] + out["dispatch_bwd"] + out["wgrad"], 4)
    # with h saved: the backward drops the recompute, the forward pays the extra h stores
    out["total_saved_ms"] = round(out["combine_bwd"] + out["ffn_bwd_saved"] + out["dispatch_bwd"] +
                                  out["wgrad"], 4)
    out["save_h_forward_extra_ms"] = round(out["gate_up_save_h"] - out["gate_up_plain"], 4)
    return out


def cpu_baseline(wl, sample_rows: int, got=None, got_y=None):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Route and schedule run in full; gather, FFN and combine run for random
    routed tokens until about `sample_rows` rows are covered, and their time
    is scaled by R / rows.  Returns the estimated ms per layer.  With `got`
    (the GPU step's output rows of every token, bf16 bits), the oracle's rows
    of the sampled tokens are also compared with the GPU's, after the timing:
    the stated bar's statistic max|got - ref| / RMS(ref) over every element of
    those rows, with no allowance (`parity`).  With `got_y` (the GPU's y of every
    slot, bf16 bits [>= R, H]) the same statistic for y against the oracle's y,
    and the oracle's merge applied to the GPU's own y against the GPU's rows:
    where that merge reproduces the GPU's value at every element above the bar,
    each such element differs only through a y that differs from the oracle's
    (by its rounding), not through the merge."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    if wl.routing_from_logits:
        idx, gate = oracle.route_topk(wl.logits, wl.k)
    else:
        idx, gate = wl.topk_idx, wl.topk_gate
        oracle.route_topk(wl.logits, wl.k)
    sch = oracle.build_schedule(idx, wl.expert_base, wl.n_local)
    t1 = time.perf_counter()
    soa = sch["slot_of_assign"].reshape(wl.T, wl.k)
    routed = np.nonzero((soa >= 0).any(1))[0]
    rng = np.random.default_rng(0)
    toks, rows = [], 0
    for t in rng.permutation(routed):
        toks.append(t)
        rows += int((soa[t] >= 0).sum())
        if rows >= sample_rows:
            break
    toks = np.array(toks, np.int64)
    s = soa[toks].reshape(-1)
    slots = np.unique(s[s >= 0])
    mx = wl.act_format == 1
    t2 = time.perf_counter()
    xr = oracle.gather_rows(wl.x, wl.k, sch["assign_of_slot"], slots, mx)
    mxw = None
    if getattr(wl, "weight_format", 0) == 1:   # the oracle quantises the weights itself
        mxw = (oracle.mx_quantize_rows(wl.w_gu), oracle.mx_quantize_rows(wl.w_d))
    y = oracle.ffn_rows(xr, oracle.expert_of_slots(sch["offsets"], slots), wl.w_gu, wl.w_d, mx,
                        mx_weights=mxw)
    yr = np.full(sch["R"], -1, np.int64)
    yr[slots] = np.arange(slots.size)
    ref, written = oracle.combine_tokens(y, yr, sch["slot_of_assign"], gate, toks, wl.k)
    t3 = time.perf_counter()
    est_s = (t1 - t0) + (t3 - t2) * sch["R"] / max(slots.size, 1)
    whole = slots.size == sch["R"]
    tail = ("the whole layer, not scaled" if whole else
            f"{toks.size} tokens = {slots.size} of {sch['R']} rows, scaled by R/rows")
    res = dict(value=est_s * 1e3, unit="ms/layer", cores=oracle.max_threads(), kind="oracle",
               cpu_model=cpu_model(),
               sample=(f"route+schedule in full ({(t1 - t0) * 1e3:.0f} ms); gather+FFN+combine "
                       f"in {t3 - t2:.1f} s for {tail}"))
    if got is not None:
        bf = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)) \
            .view(np.float32).astype(np.float64)
        g, r = bf(got[toks][written]), bf(ref[written])
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        stat = float(np.abs(g - r).max()) / rms if rms > 0 else 0.0
        bar = 2e-2 if wl.act_format == 0 and getattr(wl, "weight_format", 0) == 0 else 6e-2
        gw = got[toks][written]
        res["parity"] = {"max_abs_over_rms": round(stat, 5), "bar": bar, "strict_pass": stat <= bar,
                         "tokens": int(written.sum()), "elements": int(r.size),
                         "bits_differ": int(np.count_nonzero(gw != ref[written])),
                         "above_bar": int(np.count_nonzero(np.abs(g - r) > bar * rms)),
                         "finite": bool(np.all(np.isfinite(g))),
                         "note": ("strict: the stated bar with no allowance over every element "
                                  "of these rows; the GPU tests check every element of the "
                                  "whole share against its derived rounding band")}
        if got_y is not None:
            yg, yo = bf(got_y[slots]), bf(y)
            yrms = float(np.sqrt(np.mean(yo * yo))) if yo.size else 0.0
            ystat = float(np.abs(yg - yo).max()) / yrms if yrms > 0 else 0.0
            ident = np.arange(max(int(sch["R"]), 1), dtype=np.int64)
            m_out, _ = oracle.combine_tokens(got_y, ident, sch["slot_of_assign"], gate, toks, wl.k)
            mw = m_out[written]
            above = np.abs(g - r) > bar * rms
            mv = bf(mw)
            mstat = float(np.abs(g - mv).max()) / rms if rms > 0 else 0.0
            res["parity"].update({
                "y_max_abs_over_rms": round(ystat, 5), "y_strict_pass": ystat <= bar,
                "y_slots": int(slots.size), "y_bits_differ": int(np.count_nonzero(got_y[slots] != y)),
                "merge_of_device_y_max_abs_over_rms": round(mstat, 5),
                "merge_of_device_y_bits_differ": int(np.count_nonzero(gw != mw)),
                "above_bar_from_y_only": bool(np.all(gw[above] == mw[above]))})
    return res


def measure(st, steps: int, warmup: int) -> dict:
    """`warmup` untimed steps, then `steps` timed ones (only the gate/up launch bracketed by
    events: every event marker drains the stream), then an instrumented pass with an event
    between every call for the per-call breakdown."""
    import numpy as np
    import torch
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    ig = st.names.index("gate_up")
    evg = [{ig: torch.cuda.Event(enable_timing=True), ig + 1: torch.cuda.Event(enable_timing=True)}
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st.run(evg[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    gate_up_ms = float(np.mean([e[ig].elapsed_time(e[ig + 1]) for e in evg]))
    assert int(st.status.item()) == 0, "device status set during the benchmark"
    n_ev = len(st.names) + 1
    evs = [{j: torch.cuda.Event(enable_timing=True) for j in range(n_ev)} for _ in range(steps)]
    for i in range(steps):
        st.run(evs[i])
    torch.cuda.synchronize()
    per = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
           for j, n in enumerate(st.names)}
    per_sum = sum(per.values())
    per["gate_up"] = gate_up_ms                    # the timed region's own measurement
    return dict(wall_ms=wall_ms, per=per, per_sum=per_sum)


def step_rates(wl, st, per: dict, wall_ms: float) -> dict:
    """Algorithmic work of the step's kernels over their measured times: GEMM flop
    (4 R H I gate/up, 2 R H I down) against the MFMA peak of the weights' format, gather
    bytes R H (2 + b_out) + R 8 against HBM, and the merge's bytes: the down GEMM writes
    the output rows of tokens with one local slot itself (in place of their y rows), so
    the merge moves the y rows of the R_multi slots of the T_multi tokens with several
    local slots and their output rows, R_multi H 2 + T_multi H 2, plus every slot's
    routing words R (1 + k) 4."""
    from gpu_harness import to_host
    R = int(to_host(st.offsets)[-1])
    soa = to_host(st.soa).reshape(wl.T, wl.k)
    n_loc = (soa >= 0).sum(1)
    T_out = int((n_loc > 0).sum())
    T_multi, R_multi = int((n_loc >= 2).sum()), int(n_loc[n_loc >= 2].sum())
    H, I = wl.H, wl.I
    mx = wl.act_format == 1
    peak = PEAK_FP8_TFLOPS if getattr(wl, "weight_format", 0) else PEAK_BF16_TFLOPS
    flop_gu, flop_dn = 4.0 * R * H * I, 2.0 * R * H * I
    b_out = (1 + 1 / 32) if mx else 2
    disp_bytes = R * H * (2 + b_out) + R * 8
    comb_bytes = R_multi * H * 2 + T_multi * H * 2 + R * (1 + wl.k) * 4
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    return dict(R=R, T_out=T_out, T_multi=T_multi, R_multi=R_multi, peak=peak,
                flop_gate_up=flop_gu,
                gate_up_tflops=tf(flop_gu, per["gate_up"]), down_tflops=tf(flop_dn, per["down"]),
                gemm_tflops=tf(flop_gu + flop_dn, per["gate_up"] + per["down"]),
                dispatch_GBps=gbs(disp_bytes, per["gather"]),
                combine_GBps=gbs(comb_bytes, per["combine"]),
                layer_roofline_ms=((flop_gu + flop_dn) / (peak * 1e12) +
                                   (disp_bytes + comb_bytes) / (PEAK_HBM_GBS * 1e9)) * 1e3)


def config_summary(wl, st, m: dict) -> dict:
    """One configuration's line: ms per layer, per-call ms, rates and roofline fractions."""
    rr = step_rates(wl, st, m["per"], m["wall_ms"])
    pk = rr["peak"]
    return {"ms_per_layer": round(m["wall_ms"], 4),
            "breakdown_ms": {k: round(v, 4) for k, v in m["per"].items()},
            "routed_rows": rr["R"], "tokens_out": rr["T_out"],
            "tokens_merged_by_combine": rr["T_multi"], "minibatch": st.M,
            "gate_up_tflops": round(rr["gate_up_tflops"], 1),
            "gate_up_frac": round(rr["gate_up_tflops"] / pk, 4),
            "down_tflops": round(rr["down_tflops"], 1),
            "down_frac": round(rr["down_tflops"] / pk, 4),
            "mfma_peak_tflops": pk,
            "dispatch_GBps": round(rr["dispatch_GBps"], 1),
            "dispatch_frac_hbm": round(rr["dispatch_GBps"] / PEAK_HBM_GBS, 4),
            "combine_GBps": round(rr["combine_GBps"], 1),
            "combine_frac_hbm": round(rr["combine_GBps"] / PEAK_HBM_GBS, 4),
            "layer_roofline_frac": round(rr["layer_roofline_ms"] / m["wall_ms"], 4)}


def time_fused(mok, d, run, reps: int = 10) -> float:
    """Mean ms of a fused call over `reps` calls after 3 untimed ones."""
    import torch
    for _ in range(3):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_extras(mok, DeviceWorkload, dw, wl, st, args) -> dict:
    """The other configurations, each as its own step (or fused call): the Mixtral-shaped
    layer (also as one fused call from its logits, and from its tokens and router weights),
    the Zipf MXFP8 and full-MXFP8 shares, the minibatch sweep of the fused call in stream and
    persistent mode on the headline's share, and 8 macrobatches streamed through one ring."""
    import numpy as np
    import torch
    steps, warm = max(5, args.steps // 2), 10
    res = {"configs": {}}
    for name in ("mixtral", "kimi_zipf_mxfp8", "kimi_full_mxfp8"):
        t = time.time()
        wl2 = make_workload(name)
        dw2 = DeviceWorkload(wl2)
        cap = wl2.T * wl2.k if wl2.routing_from_logits else BENCH_MAX_ROWS
        st2 = Step(dw2, cap)
        cs = config_summary(wl2, st2, measure(st2, steps, warm))
        cs["workload"] = wl2.name
        if not wl2.routing_from_logits:   # the merge of every routed slot as one kernel
            ma = time_merge_all_slots(mok, st2)
            cs["merge_all_slots"] = ma
            cs["step_merge_multi_GBps"] = cs["combine_GBps"]
            cs["step_merge_multi_frac_hbm"] = cs["combine_frac_hbm"]
            cs["combine_GBps"], cs["combine_frac_hbm"] = ma["GBps"], ma["frac_hbm"]
        if wl2.routing_from_logits:       # the whole layer as one call from the logits
            d = dw2.desc(max_rows=cap, weights_packed=1)
            w_gu, w_d = dw2.weights(d)
            ws = torch.empty(mok.mok_forward_workspace_size(d, wl2.T, 1), dtype=torch.uint8,
                             device="cuda")
            cs["fused_from_logits_ms"] = round(time_fused(mok, d, lambda: mok.mok_moe_forward(
                d, dw2.logits, wl2.T, dw2.x, w_gu, w_d, dw2.outs[0], ws)), 4)
            assert mok.mok_device_status(ws) == 0
            del ws
            # and from the tokens and router weights (router GEMM + pick + counts in the
            # same call; seeded N(0, 1/H) router rows, so its picks are this call's own)
            import workloads as W
            _, w_r = W.router_inputs(78, 1, wl2.H, wl2.E)
            wrd = torch.from_numpy(w_r.view(np.int16)).cuda()
            ws = torch.empty(mok.mok_forward_router_workspace_size(d, wl2.T), dtype=torch.uint8,
                             device="cuda")
            cs["fused_from_router_weights_ms"] = round(time_fused(
                mok, d, lambda: mok.mok_moe_forward_router(d, wrd, wl2.T, dw2.x, w_gu, w_d,
                                                           dw2.outs[0], ws)), 4)
            assert mok.mok_device_status(ws) == 0
            del ws, wrd
        res["configs"][name] = cs
        log(f"[bench] {wl2.name}: {cs['ms_per_layer']:.4f} ms/layer, gate/up {cs['gate_up_frac']:.3f}"
            f" / down {cs['down_frac']:.3f} of peak, gather {cs['dispatch_frac_hbm']:.3f} / merge "
            f"{cs['combine_frac_hbm']:.3f} of HBM ({time.time() - t:.1f} s)"
            + (f"; one fused call from the logits {cs['fused_from_logits_ms']:.4f} ms, from the "
               f"router weights {cs['fused_from_router_weights_ms']:.4f} ms"
               if "fused_from_logits_ms" in cs else ""))
        del st2, dw2, wl2
        torch.cuda.empty_cache()
    res["streaming"] = time_streaming(mok, DeviceWorkload)
    torch.cuda.empty_cache()
    # the backward of the headline's share: bf16, with MXFP8 activations, and with
    # MXFP8 activations and weights (the same tokens, weights and routing)
    res["backward"] = time_backward(mok, dw, st)
    log(f"[bench] backward bf16 (ms): {res['backward']}")
    for key, wfmt, suffix in (("backward_mxfp8", 0, "_mxfp8act"),
                              ("backward_full_mxfp8", 1, "_full_mxfp8")):
        wl_mx = dataclasses.replace(wl, act_format=1, weight_format=wfmt, name=wl.name + suffix)
        dw_mx = DeviceWorkload(wl_mx)
        st_mx = Step(dw_mx, BENCH_MAX_ROWS)
        for _ in range(3):
            st_mx.run()
        res[key] = time_backward(mok, dw_mx, st_mx)
        log(f"[bench] {key} (ms): {res[key]}")
        del st_mx, dw_mx, wl_mx
        torch.cuda.empty_cache()
    # minibatch sweep of the fused call on the headline's share: last, so that the
    # headline's warm-up follows GPU work rather than host-side set-up
    sweep = {}
    idx, gate = dw.topk_idx, dw.topk_gate
    for mode in (mok.MOK_MODE_STREAM, mok.MOK_MODE_PERSISTENT):
        for M in list(wl.minibatches) + [8192]:
            d = dw.desc(max_rows=BENCH_MAX_ROWS, minibatch=M, mode=mode, weights_packed=1)
            w_gu, w_d = dw.weights(d)
            ws = torch.empty(mok.mok_forward_workspace_size(d, wl.T, 1), dtype=torch.uint8,
                             device="cuda")
            key = ("stream" if mode == 0 else "persistent") + f"_M{M}"
            sweep[key] = round(time_fused(mok, d, lambda: mok.mok_moe_forward_routed(
                d, idx, gate, wl.T, dw.x, w_gu, w_d, dw.outs[0], ws)), 4)
            assert mok.mok_device_status(ws) == 0
            del ws
            log(f"[bench] fused mok_moe_forward_routed {key}: {sweep[key]:.4f} ms")
    res["sweep"] = sweep
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="kimi",
                    choices=["kimi", "kimi_zipf_mxfp8", "kimi_full_mxfp8", "kimi_zipf_full_mxfp8",
                             "mixtral", "tiny"])
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="routed rows of the oracle's CPU-baseline sample; >= R runs the whole "
                         "layer (about 10 s on 16 host threads for the default workload); 0 = skip")
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="time the headline only (default: also the Mixtral-shaped layer, the "
                         "Zipf MXFP8 and full-MXFP8 shares, the minibatch sweep of the fused "
                         "call in both modes, 8 streamed macrobatches, and the backward of the "
                         "headline share in bf16 and with MXFP8 activations)")
    ap.add_argument("--fused-only", default="",
                    help="MODE:M:N_MOVE -- only run the fused call 5 times (for profiling), "
                         "MODE 0 stream / 1 persistent")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward of the layer share with --no-extras or another "
                         "workload (bf16 weights; the default run times it in bf16 and with "
                         "MXFP8 activations)")
    ap.add_argument("--mover-sweep", action="store_true",
                    help="only time the persistent kernel's mover counts against the stream path "
                         "on the streaming workload, and print them as one JSON line")
    ap.add_argument("--tune", action="store_true",
                    help="also run mok_tune_forward over minibatches (and mover counts) per mode")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 3 times (counter scale)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the layer on a single GPU; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported: run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import token_dispatch_grouped_top_amd as mok
    from gpu_harness import DeviceWorkload, to_host

    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "reps": 3}), flush=True)
        return
    if args.mover_sweep:
        print(json.dumps({"mover_sweep_ms_per_macrobatch": mover_sweep(mok, DeviceWorkload)}),
              flush=True)
        return
    t = time.time()
    wl = make_workload(args.workload)
    log(f"[bench] workload {wl.name} generated in {time.time() - t:.1f} s")
    dw = DeviceWorkload(wl)
    max_rows = BENCH_MAX_ROWS if not wl.routing_from_logits else wl.T * wl.k
    if args.fused_only:
        mode, M, n_move = (int(v) for v in args.fused_only.split(":"))
        d = dw.desc(max_rows=max_rows, minibatch=M, mode=mode, n_move_cus=n_move,
                    weights_packed=1)
        ws = torch.empty(mok.mok_forward_workspace_size(d, wl.T, 1), dtype=torch.uint8,
                         device="cuda")
        dw.routing()
        w_gu, w_d = dw.weights(d)
        for _ in range(5):
            mok.mok_moe_forward_routed(d, dw.topk_idx, dw.topk_gate, wl.T, dw.x, w_gu, w_d,
                                dw.outs[0], ws)
        torch.cuda.synchronize()
        print(json.dumps({"fused_only": args.fused_only,
                          "status": mok.mok_device_status(ws)}), flush=True)
        return
    st = Step(dw, max_rows)

    # The chip lowers its clock within milliseconds of idling and needs tens of
    # milliseconds of load to raise it again.  The first timed pass of the headline runs
    # right after the warm-up (reported as first_pass_ms); the other configurations are
    # measured next, ending with the fused-call sweep on this same share (GPU work with no
    # host-side set-up between calls), and the headline's timed region of record follows
    # them, at the working clock a serving loop would see.
    first = measure(st, args.steps, args.warmup)
    log(f"[bench] first pass (after {args.warmup} warm-up steps): {first['wall_ms']:.4f} ms/step")
    extras = {}
    if args.extras and args.workload == "kimi":
        extras = measure_extras(mok, DeviceWorkload, dw, wl, st, args)
    m = measure(st, args.steps, args.warmup)
    # the timed step's output rows (host copy) for the parity report of the cpu_baseline leg
    step_out = dw.out_rows(dw.outs[0]) if args.cpu_rows > 0 else None
    wall_ms, per, per_sum = m["wall_ms"], m["per"], m["per_sum"]
    rr = step_rates(wl, st, per, wall_ms)
    R, T_out, peak = rr["R"], rr["T_out"], rr["peak"]
    gu_tf, flop_gu = rr["gate_up_tflops"], rr["flop_gate_up"]
    log(f"[bench] R={R} T_out={T_out} M={st.M} wall {wall_ms:.3f} ms/step (instrumented pass "
        f"{per_sum:.3f}); per call (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in per.items()))
    log(f"[bench] gate/up {gu_tf:.0f} TF/s, down {rr['down_tflops']:.0f} TF/s, both "
        f"{rr['gemm_tflops']:.0f} TF/s; gather {rr['dispatch_GBps']:.0f} GB/s, combine "
        f"{rr['combine_GBps']:.0f} GB/s")
    mx = wl.act_format == 1
    wfmt = getattr(wl, "weight_format", 0)
    H, I = wl.H, wl.I
    flop_dn = 2.0 * R * H * I

    tuned = None
    if args.tune and not wl.routing_from_logits:
        tuned = {}
        for mode, moves in ((mok.MOK_MODE_STREAM, []), (mok.MOK_MODE_PERSISTENT, [32, 48])):
            Ms = [m for m in wl.minibatches if m >= 2048] + [0]
            d = dw.desc(max_rows=max_rows, mode=mode, weights_packed=1)
            need = max(mok.mok_forward_workspace_size(dw.desc(max_rows=max_rows, mode=mode, minibatch=M,
                                                              weights_packed=1), wl.T, 1) for M in Ms)
            ws_t = torch.empty(need, dtype=torch.uint8, device="cuda")
            w_gu, w_d = dw.weights(d)
            best, ms = mok.mok_tune_forward(d, Ms, moves, 5, [dw.topk_idx], [dw.topk_gate], wl.T,
                                            dw.x, w_gu, w_d, [dw.outs[0]], ws_t)
            key = "stream" if mode == mok.MOK_MODE_STREAM else "persistent"
            tuned[key] = {"minibatch": mok.mok_forward_minibatch(best, wl.T),
                          "n_move_cus": best.n_move_cus if moves else None, "ms": round(ms, 4)}
            log(f"[bench] tuner ({key}): {tuned[key]}")
            del ws_t

    backward = extras.get("backward")
    if backward is None and args.backward and not wfmt:
        backward = time_backward(mok, dw, st)
        log(f"[bench] backward (ms): {backward}")

    merge_all = time_merge_all_slots(mok, st) if not wl.routing_from_logits else None
    # y of every slot (the plain down GEMM of time_merge_all_slots), for the parity report
    step_y = to_host(st.y) if merge_all and args.cpu_rows > 0 else None
    if merge_all:
        log(f"[bench] merge of all {R} slots (mok_combine_slots): {merge_all['ms'] * 1e3:.1f} us, "
            f"{merge_all['GBps']:.0f} GB/s, {merge_all['frac_hbm']:.3f} of HBM")

    peaks = measured_peaks()
    log(f"[bench] measured references: {peaks}")

    router = time_router_gemm(mok, wl)
    log(f"[bench] router GEMM + route (mok_route_topk_gemm) T={router['T']} E={router['E']} "
        f"H={router['H']}: {router['ms'] * 1e3:.1f} us, {router['tflops']:.0f} TF/s")

    cpu = parity = None
    if args.cpu_rows > 0:
        t = time.time()
        cpu = cpu_baseline(wl, args.cpu_rows, got=step_out, got_y=step_y)
        parity = cpu.pop("parity")
        log(f"[bench] cpu baseline: {cpu['value']:.0f} ms/layer est. ({time.time() - t:.1f} s)")
        log(f"[bench] step output against the oracle's rows of the sampled tokens: {parity}")

    out = {
        "metric": METRIC,
        "value": round(wall_ms, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8" if wfmt else "mxfp8-act/bf16") if mx else "bf16",
        "data": "synthetic (seeded; random-init weights, no dataset)",
        "config": {"workload": wl.name, "pool_tokens": wl.T, "partitions": wl.n_partitions,
                   "routed_rows": R, "tokens_out": T_out, "hidden": H, "inter": I,
                   "experts": wl.E, "n_local": wl.n_local, "top_k": wl.k, "minibatch": st.M,
                   "max_rows": max_rows, "path": "stream-ordered C-ABI calls"},
        "roofline": {"bound": "mfma", "kernel": "gate_up grouped GEMM + SwiGLU",
                     "achieved": round(gu_tf, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(gu_tf / peak, 4),
                     "traffic": gate_up_traffic(wl.name),
                     "traffic_unit": "bytes per launch (HBM read + write)",
                     "algorithmic_flop_per_launch": flop_gu},
        "breakdown_ms": {k: round(v, 4) for k, v in per.items()},
        "breakdown_note": "gate_up from the timed region's events; the other calls from a separate "
                          "pass with an event between every call (each marker drains the stream); "
                          "down = mok_expert_down_merge (also writes the output rows of tokens "
                          "with one local slot), combine = mok_combine_slots_multi (the tokens "
                          "with several local slots)",
        "merge_split": {"tokens_out": T_out, "tokens_merged_in_down": T_out - rr["T_multi"],
                        "tokens_merged_by_combine": rr["T_multi"],
                        "slots_of_those": rr["R_multi"]},
        "first_pass_ms": round(first["wall_ms"], 4),
        "first_pass_note": "the same K steps timed right after the W warm-up steps, before the "
                           "other configurations ran (the chip below its working clock)",
        "gemm_tflops": {"gate_up": round(gu_tf, 1), "down": round(rr["down_tflops"], 1),
                        "both": round(rr["gemm_tflops"], 1),
                        "frac_of_peak": round(rr["gemm_tflops"] / peak, 4),
                        "down_frac_of_peak": round(rr["down_tflops"] / peak, 4)},
        "dispatch_GBps": round(rr["dispatch_GBps"], 1),
        "dispatch_frac_hbm": round(rr["dispatch_GBps"] / PEAK_HBM_GBS, 4),
        # combine: the weighted merge of every routed slot as one kernel (merge_all_slots);
        # the layer step splits it between the down GEMM's epilogue (single-slot tokens)
        # and a merge of the rest, whose own rate is step_merge_multi_*
        "combine_GBps": merge_all["GBps"] if merge_all else round(rr["combine_GBps"], 1),
        "combine_frac_hbm": (merge_all["frac_hbm"] if merge_all
                             else round(rr["combine_GBps"] / PEAK_HBM_GBS, 4)),
        "step_merge_multi_GBps": round(rr["combine_GBps"], 1),
        "step_merge_multi_frac_hbm": round(rr["combine_GBps"] / PEAK_HBM_GBS, 4),
        "merge_all_slots": merge_all,
        # the same rates against what this GPU measures for a plain copy and a dense
        # library GEMM (context beside the nominal peaks)
        "measured_peaks": dict(peaks, gate_up_vs_hipblaslt=round(gu_tf / peaks[
            "hipblaslt_bf16_8192cube_tflops"], 4), gather_vs_copy=round(rr["dispatch_GBps"] / peaks[
            "hbm_copy_1GiB_GBps"], 4), merge_all_vs_copy=(round(merge_all["GBps"] / peaks[
            "hbm_copy_1GiB_GBps"], 4) if merge_all else None)),
        "schedule_share": round(per["schedule"] / wall_ms, 4),
        # the layer against its roofline: both GEMMs at the MFMA peak plus the
        # gather and merge bytes at the HBM peak, over the timed wall
        "layer_roofline_ms": round(rr["layer_roofline_ms"], 4),
        "layer_roofline_frac": round(rr["layer_roofline_ms"] / wall_ms, 4),
        "configs": extras.get("configs"),
        "fused_forward_ms": extras.get("sweep"),
        "streaming_ms_per_macrobatch": extras.get("streaming"),
        "router_gemm": router,
        "backward_ms": backward,
        "backward_mxfp8_ms": extras.get("backward_mxfp8"),
        "backward_full_mxfp8_ms": extras.get("backward_full_mxfp8"),
        "tuned_forward": tuned,
        "cpu_baseline": cpu,
        # the timed step's output rows against the oracle's, from the cpu_baseline leg
        "parity_vs_oracle": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
