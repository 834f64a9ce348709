"""Helpers for the GPU parity tests and the benchmark: move a workload to the
device and drive the libmok C-ABI through its Python binding.  No arithmetic
of the layer happens here."""
from __future__ import annotations

import numpy as np
import torch

import bars
import oracle
import token_dispatch_grouped_top_amd as mok

SENTINEL = 0x7FC1   # a bf16 NaN pattern: rows the layer must not write keep it


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def colblk_rows(t: torch.Tensor, rows: int) -> np.ndarray:
    """Row-major host copy of a column-blocked row buffer (the ring, act):
    64-byte block b of row r sits at byte (b * rows + r) * 64."""
    a = t.detach().contiguous().view(torch.uint8).reshape(-1).cpu().numpy()
    nb = a.size // (rows * 64)
    out = a[:nb * rows * 64].reshape(nb, rows, 64).transpose(1, 0, 2).reshape(rows, nb * 64)
    return out.view(np.uint16) if t.element_size() == 2 else out


def colblk_scales(t: torch.Tensor, rows: int) -> np.ndarray:
    """Row-major host copy of column-blocked E8M0 scales: scale j of row r
    sits at byte (j // 2 * rows + r) * 2 + j % 2."""
    a = t.detach().contiguous().reshape(-1).cpu().numpy()
    npair = a.size // (rows * 2)
    return a[:npair * rows * 2].reshape(npair, rows, 2).transpose(1, 0, 2).reshape(rows, 2 * npair)


def empty_u16(*shape) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.int16, device="cuda")


def gpu_schedule(idx, T: int, k: int, expert_base: int, n_local: int) -> dict:
    """mok_build_schedule on device buffers; assign_of_slot pre-filled with -7."""
    A = T * k
    counts = torch.empty(n_local, dtype=torch.int32, device="cuda")
    offsets = torch.empty(n_local + 1, dtype=torch.int32, device="cuda")
    soa = torch.empty(max(A, 1), dtype=torch.int32, device="cuda")
    aos = torch.full((max(A, 1),), -7, dtype=torch.int32, device="cuda")
    wsb = mok.mok_schedule_workspace_size(T, k, n_local)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    mok.mok_build_schedule(idx, T, k, expert_base, n_local, counts, offsets, soa, aos, ws)
    return dict(counts=counts, offsets=offsets, soa=soa, aos=aos)


class DeviceWorkload:
    """A ``workloads.Workload`` on the GPU: each source partition and each
    output partition in its own allocation."""

    def __init__(self, wl, n_out: int = 1):
        self.wl = wl
        P, rows, H = wl.n_partitions, wl.part_rows, wl.H
        self.x_parts = [to_dev(wl.x[p * rows:(p + 1) * rows]) for p in range(P)]
        self.x = mok.Tokens(self.x_parts, rows)
        self.w_gu = to_dev(wl.w_gu)
        self.w_d = to_dev(wl.w_d)
        self.logits = to_dev(wl.logits)
        if wl.topk_idx is not None:
            self.topk_idx = to_dev(wl.topk_idx)
            self.topk_gate = to_dev(wl.topk_gate)
        else:
            self.topk_idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
            self.topk_gate = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        self.outs = [self.new_out() for _ in range(n_out)]

    def new_out(self) -> mok.Tokens:
        wl = self.wl
        parts = [torch.full((wl.part_rows, wl.H), SENTINEL, dtype=torch.int16, device="cuda")
                 for _ in range(wl.n_partitions)]
        return mok.Tokens(parts, wl.part_rows)

    def out_rows(self, out: mok.Tokens, tokens=None) -> np.ndarray:
        full = torch.cat(out.parts, 0)
        if tokens is not None:
            full = full[torch.as_tensor(np.asarray(tokens), device="cuda")]
        return to_host(full)

    def reset_out(self, out: mok.Tokens) -> None:
        for p in out.parts:
            p.fill_(SENTINEL)

    def desc(self, **kw) -> mok.mok_layer_desc:
        wl = self.wl
        d = mok.mok_layer_desc(hidden=wl.H, inter=wl.I, n_experts=wl.E, top_k=wl.k,
                               expert_base=wl.expert_base, n_local=wl.n_local,
                               act_format=wl.act_format,
                               weight_format=getattr(wl, "weight_format", 0))
        if d.weight_format:                 # MXFP8 weights exist only packed
            d.weights_packed = 1
        for key, v in kw.items():
            setattr(d, key, v)
        return d

    # ---- steps through the C-ABI
    def route(self, logits=None, idx=None, gate=None):
        wl = self.wl
        logits = self.logits if logits is None else logits
        T, E = logits.shape
        idx = torch.empty((T, wl.k), dtype=torch.int32, device="cuda") if idx is None else idx
        gate = torch.empty((T, wl.k), dtype=torch.float32, device="cuda") if gate is None else gate
        mok.mok_route_topk(logits, T, E, wl.k, idx, gate)
        return idx, gate

    def routing(self):
        """Routing the layer consumes: routed from logits, or the given pool routing."""
        if self.wl.routing_from_logits:
            self.route(idx=self.topk_idx, gate=self.topk_gate)
        return self.topk_idx, self.topk_gate

    def schedule(self, idx):
        wl = self.wl
        return gpu_schedule(idx, wl.T, wl.k, wl.expert_base, wl.n_local)

    def packed(self):
        """(gate_up, down) weights packed by mok_pack_weights for this workload."""
        if getattr(self, "_packed", None) is None:
            d = self.desc()
            gu, dn = mok.mok_packed_weights_size(d)
            pgu = torch.empty(gu, dtype=torch.uint8, device="cuda")
            pdn = torch.empty(dn, dtype=torch.uint8, device="cuda")
            mok.mok_pack_weights(d, self.w_gu, self.w_d, pgu, pdn)
            self._packed = (pgu, pdn)
        return self._packed

    def weights(self, desc):
        """The weight buffers matching desc.weights_packed."""
        return self.packed() if desc.weights_packed else (self.w_gu, self.w_d)

    def forward(self, out=None, **desc_kw):
        wl = self.wl
        out = self.outs[0] if out is None else out
        idx, gate = self.routing()
        d = self.desc(**desc_kw)
        wsb = mok.mok_forward_workspace_size(d, wl.T, 1)
        assert wsb > 0
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        w_gu, w_d = self.weights(d)
        if wl.routing_from_logits:      # the fused call routes the logits itself
            mok.mok_moe_forward(d, self.logits, wl.T, self.x, w_gu, w_d, out, ws)
        else:
            mok.mok_moe_forward_routed(d, idx, gate, wl.T, self.x, w_gu, w_d, out, ws)
        return ws, d


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32) \
        .astype(np.float64)


def assert_close_rms(got_bits: np.ndarray, ref_bits: np.ndarray, tol_rms: float, what: str):
    """The stated bar with no allowance: max|got - ref| <= tol_rms * RMS(ref)
    (2e-2 bf16, 6e-2 MXFP8).  Returns max|got - ref| / RMS(ref)."""
    return bars.strict_stats(got_bits, ref_bits, tol_rms, what)


def bf16_layer(wl) -> bool:
    """bf16 activations and weights (stated bar 2e-2 RMS; MXFP8 6e-2)."""
    return wl.act_format == 0 and getattr(wl, "weight_format", 0) == 0


def check_y_rows(got_bits: np.ndarray, wl, x_rows, expert_of_row, what: str = "y") -> dict:
    """Expert outputs of dispatched rows against the oracle by the rounding
    bands of tests/bars.py (bit-exact outside a tie band); the stated bar's
    statistic (2e-2 RMS bf16, 6e-2 MXFP8) is reported.  Returns the statistics."""
    mx = wl.act_format == 1
    mxw = None
    if getattr(wl, "weight_format", 0) == 1:
        mxw = (oracle.mx_quantize_rows(wl.w_gu), oracle.mx_quantize_rows(wl.w_d))
    y, a_ex, y_ex = oracle.ffn_rows(x_rows, expert_of_row, wl.w_gu, wl.w_d, mx, mx_weights=mxw,
                                    exact=True)
    lo, hi, _ = bars.layer_y_band(wl, x_rows, expert_of_row, a_ex, y_ex)
    return bars.band_stats(got_bits, y, lo, hi, 2e-2 if bf16_layer(wl) else 6e-2, what)


def check_layer_out(got_rows: np.ndarray, wl, r: dict, what: str = "out") -> dict:
    """Merged rows of the tokens r['tokens'] (oracle.forward result r, rows
    aligned with them) against the oracle by the rounding bands of
    tests/bars.py; the stated bar's statistic is reported.  Only rows of
    tokens with a local assignment are compared; the others must keep the
    sentinel."""
    wr = r["written"]
    assert np.all(got_rows[~wr] == SENTINEL), f"{what}: a token without local slots was written"
    gate_rel = 2.0 ** -19 if wl.routing_from_logits else 0.0
    _, _, lo, hi = bars.forward_band(wl, r, gate_rel)
    return bars.band_stats(got_rows[wr], r["out"][wr], lo[wr], hi[wr],
                           2e-2 if bf16_layer(wl) else 6e-2, what)
