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
    "kimi_share_R8192_H7168_I2048_E384_k8_local8": ("2ad9731a5b564065", 738608725),
    "kimi_zipf_mxfp8_R8192_H7168_I2048_E384_k8_local8": ("2ad9731a5b564065", 990437491),
    "kimi_full_mxfp8_R8192_H7168_I2048_E384_k8_local8": ("2ad9731a5b564065", 381108334),
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
        mok.mok_build_schedule(idx, wl.T, wl.k, wl.expert_base, wl.n_local, self.counts,
                               self.offsets, self.soa, self.aos, self.sched_ws)
        mok.mok_build_windows(self.offsets, wl.n_local, self.M, self.nwin, self.win)
        rec(2)
        mok.mok_dispatch_gather(dw.x, wl.H, wl.k, self.aos, self.offsets, wl.n_local, 0, self.cap,
                                self.ring, self.ring_sc, self.cap, wl.act_format, self.status)
        rec(3)
        mok.mok_expert_gate_up(self.desc, self.ring, self.ring_sc, self.cap, self.offsets, 0,
                               self.cap, self.w_gu, self.act, self.act_sc, self.cap, self.gemm_ws)
        rec(4)
        mok.mok_expert_down(self.desc, self.act, self.act_sc, self.cap, self.offsets, 0, self.cap,
                            self.w_d, self.y, self.cap, self.gemm_ws)
        rec(5)
        mok.mok_combine_slots(self.y, self.cap, self.aos, self.offsets, wl.n_local, self.cap,
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
    """The backward of the layer share after a forward step (bf16 only): merge
    backward (dy, dgate), the expert FFN backward (recompute of h, down dgrad
    with the SwiGLU backward, gate/up dgrad), dispatch backward (dx), weight
    gradients (transposes + two GEMMs over each expert's slots).  Seeded
    N(0, 1) dout for every pool token; per-call means over `reps` calls."""
    import numpy as np
    import torch
    import workloads as W
    from gpu_harness import to_dev
    wl = dw.wl
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
    dy = torch.empty((cap, H), dtype=torch.int16, device="cuda")
    dgate = torch.empty((wl.T, k), dtype=torch.float32, device="cuda")
    h = torch.empty((cap, 2 * I), dtype=torch.int16, device="cuda")
    dh = torch.empty((cap, 2 * I), dtype=torch.int16, device="cuda")
    dxs = torch.empty((cap, H), dtype=torch.int16, device="cuda")
    dwgu = torch.empty((wl.n_local, 2 * I, H), dtype=torch.int16, device="cuda")
    dwd = torch.empty((wl.n_local, H, I), dtype=torch.int16, device="cuda")
    wws = torch.empty(mok.mok_wgrad_workspace_size(d, cap), dtype=torch.uint8, device="cuda")
    hsv = torch.empty((cap, 2 * I), dtype=torch.int16, device="cuda")
    calls = {
        "combine_bwd": lambda: mok.mok_combine_backward(dout, st.y, cap, st.aos, st.offsets,
                                                        wl.n_local, cap, dw.topk_gate, k, H, dy,
                                                        cap, dgate, st.status),
        "ffn_bwd": lambda: mok.mok_expert_ffn_backward(d, st.ring, cap, dy, st.offsets, 0, cap,
                                                       st.w_gu, gu_t, d_t, h, dh, dxs, cap),
        "dispatch_bwd": lambda: mok.mok_dispatch_backward(dxs, cap, st.aos, st.offsets, wl.n_local,
                                                          cap, st.soa, k, H, dx, st.status),
        "wgrad": lambda: mok.mok_expert_wgrad(d, st.ring, cap, st.act, cap, dy, dh, cap, st.offsets,
                                              dwgu, dwd, wws),
        # h kept by the forward instead of recomputed: the forward's gate/up that also
        # stores h (timed whole, to set against the plain gate/up), then the backward from it
        "gate_up_save_h": lambda: mok.mok_expert_gate_up_save_h(d, st.ring, cap, st.offsets, 0, cap,
                                                                st.w_gu, st.act, cap, hsv,
                                                                st.gemm_ws),
        "gate_up_plain": lambda: mok.mok_expert_gate_up(d, st.ring, None, cap, st.offsets, 0, cap,
                                                        st.w_gu, st.act, None, cap, st.gemm_ws),
        "ffn_bwd_saved": lambda: mok.mok_expert_ffn_backward_saved(d, dy, st.offsets, 0, cap, gu_t,
                                                                   d_t, hsv, dh, dxs, cap),
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


def cpu_baseline(wl, sample_rows: int):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Route and schedule run in full; gather, FFN and combine run for random
    routed tokens until about `sample_rows` rows are covered, and their time
    is scaled by R / rows.  Returns the estimated ms per layer."""
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
    oracle.combine_tokens(y, yr, sch["slot_of_assign"], gate, toks, wl.k)
    t3 = time.perf_counter()
    est_s = (t1 - t0) + (t3 - t2) * sch["R"] / max(slots.size, 1)
    whole = slots.size == sch["R"]
    tail = ("the whole layer, not scaled" if whole else
            f"{toks.size} tokens = {slots.size} of {sch['R']} rows, scaled by R/rows")
    return dict(value=est_s * 1e3, unit="ms/layer", cores=oracle.max_threads(), kind="oracle",
                sample=(f"route+schedule in full ({(t1 - t0) * 1e3:.0f} ms); gather+FFN+combine "
                        f"in {t3 - t2:.1f} s for {tail}"))


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
    ap.add_argument("--sweep", action="store_true", help="also time the fused call per minibatch")
    ap.add_argument("--fused-only", default="",
                    help="MODE:M:N_MOVE -- only run the fused call 5 times (for profiling), "
                         "MODE 0 stream / 1 persistent")
    ap.add_argument("--streaming", action="store_true",
                    help="also time 8 Kimi-shaped macrobatches through one ring, per mode")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward of the layer share (bf16 workloads)")
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
            mok.mok_moe_forward(d, dw.topk_idx, dw.topk_gate, wl.T, dw.x, w_gu, w_d,
                                dw.outs[0], ws)
        torch.cuda.synchronize()
        print(json.dumps({"fused_only": args.fused_only,
                          "status": mok.mok_device_status(ws)}), flush=True)
        return
    st = Step(dw, max_rows)
    stream = torch.cuda.current_stream()

    # The chip lowers its clock within milliseconds of idling and needs tens of
    # milliseconds of load to raise it again: the default warmup (60 steps, about 40 ms)
    # covers that, so the timed region starts at the working clock.
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    # timed region: only the dominant launch (gate/up) is bracketed by events
    ig = st.names.index("gate_up")
    evg = [{ig: torch.cuda.Event(enable_timing=True), ig + 1: torch.cuda.Event(enable_timing=True)}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.run(evg[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    gate_up_ms = float(np.mean([e[ig].elapsed_time(e[ig + 1]) for e in evg]))
    assert int(st.status.item()) == 0, "device status set during the benchmark"
    # per-call breakdown from a separate instrumented pass (an event between every call)
    n_ev = len(st.names) + 1
    evs = [{j: torch.cuda.Event(enable_timing=True) for j in range(n_ev)} for _ in range(args.steps)]
    for i in range(args.steps):
        st.run(evs[i])
    torch.cuda.synchronize()
    per = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
           for j, n in enumerate(st.names)}
    per_sum = sum(per.values())
    per["gate_up"] = gate_up_ms                    # the timed region's own measurement

    R = int(to_host(st.offsets)[-1])
    soa = to_host(st.soa).reshape(wl.T, wl.k)
    T_out = int((soa >= 0).any(1).sum())
    H, I = wl.H, wl.I
    mx = wl.act_format == 1
    wfmt = getattr(wl, "weight_format", 0)
    peak = PEAK_FP8_TFLOPS if wfmt else PEAK_BF16_TFLOPS
    flop_gu, flop_dn = 4.0 * R * H * I, 2.0 * R * H * I
    b_out = (1 + 1 / 32) if mx else 2
    disp_bytes = R * H * (2 + b_out) + R * 8
    comb_bytes = R * H * 2 + T_out * H * 2 + wl.T * wl.k * 8
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    gu_tf, dn_tf = tf(flop_gu, per["gate_up"]), tf(flop_dn, per["down"])
    gemm_tf = tf(flop_gu + flop_dn, per["gate_up"] + per["down"])
    disp_gbs, comb_gbs = gbs(disp_bytes, per["gather"]), gbs(comb_bytes, per["combine"])

    log(f"[bench] R={R} T_out={T_out} M={st.M} wall {wall_ms:.3f} ms/step (instrumented pass "
        f"{per_sum:.3f}); per call (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in per.items()))
    log(f"[bench] gate/up {gu_tf:.0f} TF/s, down {dn_tf:.0f} TF/s, both {gemm_tf:.0f} TF/s; "
        f"gather {disp_gbs:.0f} GB/s, combine {comb_gbs:.0f} GB/s")

    fused = {}
    if args.sweep and not wl.routing_from_logits:
        idx, gate = dw.topk_idx, dw.topk_gate
        for mode in (mok.MOK_MODE_STREAM, mok.MOK_MODE_PERSISTENT):
            for M in [0] + list(wl.minibatches):
                for n_move in ((0,) if mode == mok.MOK_MODE_STREAM else (32, 48)):
                    d = dw.desc(max_rows=max_rows, minibatch=M, mode=mode, n_move_cus=n_move,
                                weights_packed=1)
                    w_gu, w_d = dw.weights(d)
                    wsb = mok.mok_forward_workspace_size(d, wl.T, 1)
                    if wsb == 0:
                        continue
                    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
                    for _ in range(3):
                        mok.mok_moe_forward(d, idx, gate, wl.T, dw.x, w_gu, w_d, dw.outs[0], ws)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(10):
                        mok.mok_moe_forward(d, idx, gate, wl.T, dw.x, w_gu, w_d, dw.outs[0], ws)
                    e1.record()
                    torch.cuda.synchronize()
                    assert mok.mok_device_status(ws) == 0
                    Mu = mok.mok_forward_minibatch(d, wl.T)
                    key = ("stream" if mode == 0 else f"persistent_mv{n_move}") + f"_M{Mu}"
                    fused[key] = round(e0.elapsed_time(e1) / 10, 4)
                    log(f"[bench] fused mok_moe_forward {key}: {fused[key]:.4f} ms")

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

    backward = None
    if args.backward and not mx and not wfmt:
        backward = time_backward(mok, dw, st)
        log(f"[bench] backward (ms): {backward}")

    router = time_router_gemm(mok, wl)
    log(f"[bench] router GEMM + route (mok_route_topk_gemm) T={router['T']} E={router['E']} "
        f"H={router['H']}: {router['ms'] * 1e3:.1f} us, {router['tflops']:.0f} TF/s")

    streaming = None
    if args.streaming and wl.name.startswith("kimi_share"):
        streaming = time_streaming(mok, DeviceWorkload)

    cpu = None
    if args.cpu_rows > 0:
        t = time.time()
        cpu = cpu_baseline(wl, args.cpu_rows)
        log(f"[bench] cpu baseline: {cpu['value']:.0f} ms/layer est. ({time.time() - t:.1f} s)")

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
                          "pass with an event between every call (each marker drains the stream)",
        "gemm_tflops": {"gate_up": round(gu_tf, 1), "down": round(dn_tf, 1),
                        "both": round(gemm_tf, 1),
                        "frac_of_peak": round(gemm_tf / peak, 4)},
        "dispatch_GBps": round(disp_gbs, 1), "dispatch_frac_hbm": round(disp_gbs / PEAK_HBM_GBS, 4),
        "combine_GBps": round(comb_gbs, 1), "combine_frac_hbm": round(comb_gbs / PEAK_HBM_GBS, 4),
        "schedule_share": round(per["schedule"] / wall_ms, 4),
        # the layer against its roofline: both GEMMs at the MFMA peak plus the
        # gather and merge bytes at the HBM peak, over the timed wall
        "layer_roofline_ms": round(((flop_gu + flop_dn) / (peak * 1e12) +
                                    (disp_bytes + comb_bytes) / (PEAK_HBM_GBS * 1e9)) * 1e3, 4),
        "layer_roofline_frac": round(((flop_gu + flop_dn) / (peak * 1e12) +
                                      (disp_bytes + comb_bytes) / (PEAK_HBM_GBS * 1e9)) * 1e3 / wall_ms, 4),
        "fused_forward_ms": fused or None,
        "streaming_ms_per_macrobatch": streaming,
        "router_gemm": router,
        "backward_ms": backward,
        "tuned_forward": tuned,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
