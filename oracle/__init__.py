"""CPU oracle for the MoK forward MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.

The arithmetic lives in ``mok_oracle.c`` (plain C, fp64, OpenMP over rows);
this module compiles it with gcc and wraps it with numpy-array helpers.
Every array here is plain numpy on the host.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mok_oracle.c")
_LIB = os.path.join(_HERE, "libmok_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.orc_route_topk.argtypes = [P, i64, i32, i32, P, P]
        L.orc_route_topk.restype = C.c_int
        L.orc_build_schedule.argtypes = [P, i64, i32, i32, i32, P, P, P, P]
        L.orc_build_schedule.restype = C.c_int
        L.orc_windows.argtypes = [P, i32, i32, i32, P]
        L.orc_windows.restype = None
        L.orc_choose_minibatch.argtypes = [i32, i32, i32, i32, i64]
        L.orc_choose_minibatch.restype = i32
        L.orc_e4m3_encode_n.argtypes = [P, i64, P]
        L.orc_e4m3_decode_n.argtypes = [P, i64, P]
        L.orc_bf16_round_n.argtypes = [P, i64, P]
        L.orc_mx_quantize.argtypes = [P, i64, P, P]
        L.orc_mx_dequantize.argtypes = [P, P, i64, P]
        L.orc_gather_rows.argtypes = [P, i32, i32, P, P, i64, i32, P, P, P]
        L.orc_ffn_rows.argtypes = [P, P, P, P, i64, i32, i32, P, P, i32, P, P, P, P, P, P, P]
        L.orc_mx_quantize_rows_bf16.argtypes = [P, i64, i32, P, P]
        L.orc_combine_tokens.argtypes = [P, P, P, P, P, i64, i32, i32, P, P, P]
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = C.c_int
        for f in ("orc_e4m3_encode_n", "orc_e4m3_decode_n", "orc_bf16_round_n",
                  "orc_mx_quantize", "orc_mx_dequantize", "orc_gather_rows",
                  "orc_ffn_rows", "orc_combine_tokens", "orc_mx_quantize_rows_bf16"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- formats
def bf16_round(v) -> np.ndarray:
    v = _c(v, np.float64).reshape(-1)
    out = np.empty(v.size, np.uint16)
    lib().orc_bf16_round_n(_p(v), v.size, _p(out))
    return out


def e4m3_encode(v) -> np.ndarray:
    v = _c(v, np.float64).reshape(-1)
    out = np.empty(v.size, np.uint8)
    lib().orc_e4m3_encode_n(_p(v), v.size, _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c(c, np.uint8).reshape(-1)
    out = np.empty(c.size, np.float64)
    lib().orc_e4m3_decode_n(_p(c), c.size, _p(out))
    return out


def mx_quantize(v):
    """MXFP8 (E4M3, blocks of 32) of a 1-D array whose length is a multiple of 32."""
    v = _c(v, np.float64).reshape(-1)
    assert v.size % 32 == 0
    codes = np.empty(v.size, np.uint8)
    scales = np.empty(v.size // 32, np.uint8)
    lib().orc_mx_quantize(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def mx_dequantize(codes, scales) -> np.ndarray:
    codes = _c(codes, np.uint8).reshape(-1)
    scales = _c(scales, np.uint8).reshape(-1)
    out = np.empty(codes.size, np.float64)
    lib().orc_mx_dequantize(_p(codes), _p(scales), codes.size, _p(out))
    return out


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- steps
def route_topk(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float32)
    rc = lib().orc_route_topk(_p(logits), T, E, k, _p(idx), _p(gate))
    if rc:
        raise ValueError(f"orc_route_topk rc={rc}")
    return idx, gate


def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray) -> np.ndarray:
    """Router scores (tahou.com MoK article, routing paragraph: every token is
    scored against every expert before the picks): logits[t][e] =
    sum_h x[t][h] * w_router[e][h] over the bf16 values of x (bf16 [T][H]) and
    w_router (bf16 [E][H], nn.Linear layout), in fp64 (a library matmul as the
    step).  Each product of two bf16 values is exact in fp64; the fp64 sum is
    the reference the fp32 sums of the device are held to."""
    xv = bf16_value(x_bits).astype(np.float64)
    wv = bf16_value(w_router_bits).astype(np.float64)
    return xv @ wv.T


def build_schedule(topk_idx: np.ndarray, expert_base: int, n_local: int):
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts = np.empty(n_local, np.int32)
    offsets = np.empty(n_local + 1, np.int32)
    soa = np.empty(T * k, np.int32)
    aos = np.full(T * k, -1, np.int32)
    rc = lib().orc_build_schedule(_p(idx), T, k, expert_base, n_local, _p(counts),
                                  _p(offsets), _p(soa), _p(aos))
    if rc:
        raise ValueError(f"orc_build_schedule rc={rc}")
    R = int(offsets[-1])
    return dict(counts=counts, offsets=offsets, slot_of_assign=soa,
                assign_of_slot=aos[:R].copy(), R=R)


def windows(offsets: np.ndarray, M: int, nwin: int) -> np.ndarray:
    offsets = _c(offsets, np.int32)
    n_local = offsets.size - 1
    out = np.empty((nwin, n_local + 1), np.int32)
    lib().orc_windows(_p(offsets), n_local, M, nwin, _p(out))
    return out


def choose_minibatch(n_cus: int, tile_m: int, tile_n: int, n_out: int, rows: int = 0) -> int:
    return int(lib().orc_choose_minibatch(n_cus, tile_m, tile_n, n_out, rows))


def gather_rows(x: np.ndarray, k: int, assign_of_slot: np.ndarray, slots, mxfp8: bool):
    """Dispatched rows for the given slots: bf16 bits [n,H] or (codes [n,H], scales [n,H/32])."""
    x = _c(x, np.uint16)
    H = x.shape[1]
    aos = _c(assign_of_slot, np.int32)
    slots = _c(slots, np.int64).reshape(-1)
    n = slots.size
    if mxfp8:
        codes = np.empty((n, H), np.uint8)
        scales = np.empty((n, H // 32), np.uint8)
        lib().orc_gather_rows(_p(x), H, k, _p(aos), _p(slots), n, 1, None, _p(codes), _p(scales))
        return codes, scales
    out = np.empty((n, H), np.uint16)
    lib().orc_gather_rows(_p(x), H, k, _p(aos), _p(slots), n, 0, _p(out), None, None)
    return out


def mx_quantize_rows(w_bits: np.ndarray):
    """MXFP8 of bf16 rows [..., K] in blocks of 32 along K -> (codes [..., K], scales [..., K/32])."""
    w = _c(w_bits, np.uint16)
    K = w.shape[-1]
    assert K % 32 == 0
    rows = w.size // K
    codes = np.empty(w.shape, np.uint8)
    scales = np.empty(w.shape[:-1] + (K // 32,), np.uint8)
    lib().orc_mx_quantize_rows_bf16(_p(w), rows, K, _p(codes), _p(scales))
    return codes, scales


def ffn_rows(xrows, expert_of_row, w_gu: np.ndarray, w_d: np.ndarray, mxfp8: bool,
             mx_weights=None, exact: bool = False):
    """Expert SwiGLU FFN of dispatched rows -> y bf16 bits [n, H].

    mx_weights: None (bf16 weights) or ((gu_codes, gu_scales), (d_codes, d_scales)) from
    mx_quantize_rows of w_gu and w_d, used in place of them.
    exact: also return the fp64 values before rounding, (y, a_exact [n, I], y_exact [n, H])."""
    w_gu = _c(w_gu, np.uint16)
    w_d = _c(w_d, np.uint16)
    I2, H = w_gu.shape[1], w_gu.shape[2]
    I = I2 // 2
    eor = _c(expert_of_row, np.int32).reshape(-1)
    n = eor.size
    y = np.empty((n, H), np.uint16)
    a_ex = np.empty((n, I), np.float64) if exact else None
    y_ex = np.empty((n, H), np.float64) if exact else None
    if mx_weights is None:
        wq = (None, None, None, None)
    else:
        (gc, gs), (dc, ds) = mx_weights
        wq = tuple(_c(a, np.uint8) for a in (gc, gs, dc, ds))
    wp = [_p(a) for a in wq]
    if mxfp8:
        codes, scales = xrows
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.uint8)
        lib().orc_ffn_rows(None, _p(codes), _p(scales), _p(eor), n, H, I, _p(w_gu), _p(w_d), 1,
                           *wp, _p(y), _p(a_ex), _p(y_ex))
    else:
        xb = _c(xrows, np.uint16)
        lib().orc_ffn_rows(_p(xb), None, None, _p(eor), n, H, I, _p(w_gu), _p(w_d), 0, *wp,
                           _p(y), _p(a_ex), _p(y_ex))
    return (y, a_ex, y_ex) if exact else y


def combine_tokens(y: np.ndarray, y_row_of_slot: np.ndarray, slot_of_assign: np.ndarray,
                   topk_gate: np.ndarray, tokens, k: int, exact: bool = False):
    """Weighted merge for the listed tokens -> (out bf16 [n,H], written bool [n]), plus the
    fp64 sums before rounding (out_exact [n, H]) when exact."""
    y = _c(y, np.uint16)
    H = y.shape[1]
    yr = _c(y_row_of_slot, np.int64)
    soa = _c(slot_of_assign, np.int32)
    gate = _c(topk_gate, np.float32)
    tokens = _c(tokens, np.int64).reshape(-1)
    n = tokens.size
    out = np.zeros((n, H), np.uint16)
    written = np.zeros(n, np.uint8)
    o_ex = np.zeros((n, H), np.float64) if exact else None
    lib().orc_combine_tokens(_p(y), _p(yr), _p(soa), _p(gate), _p(tokens), n, k, H,
                             _p(out), _p(written), _p(o_ex))
    return (out, written.astype(bool), o_ex) if exact else (out, written.astype(bool))


def expert_of_slots(offsets: np.ndarray, slots) -> np.ndarray:
    """Local expert owning each schedule slot (segment lookup in the offsets)."""
    offsets = np.asarray(offsets, np.int64)
    slots = np.asarray(slots, np.int64)
    return (np.searchsorted(offsets, slots, side="right") - 1).astype(np.int32)


# ---------------------------------------------------------------- chain
def forward(wl, tokens=None, slots_extra=None) -> Dict[str, np.ndarray]:
    """The whole layer for a workload (``workloads.Workload``).

    Route (when the workload routes from logits), schedule, then gather, FFN
    and combine for the listed pool tokens (all tokens when ``tokens`` is
    None).  Only the slots those tokens need are computed, plus
    ``slots_extra`` if given.  Returns routing, schedule, the y rows of the
    computed slots and the merged output rows, and the fp64 values before their
    rounding (a_exact, y_exact per computed slot, out_exact per listed token).
    """
    res: Dict[str, np.ndarray] = {}
    if wl.routing_from_logits:
        idx, gate = route_topk(wl.logits, wl.k)
    else:
        idx, gate = wl.topk_idx, wl.topk_gate
        res["route_idx"], res["route_gate"] = route_topk(wl.logits, wl.k)
    res["topk_idx"], res["topk_gate"] = idx, gate
    sch = build_schedule(idx, wl.expert_base, wl.n_local)
    res.update(sch)
    soa = sch["slot_of_assign"]
    T, k = wl.T, wl.k
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = np.asarray(tokens, np.int64)
    s = soa.reshape(T, k)[tokens].reshape(-1)
    slots = np.unique(s[s >= 0])
    if slots_extra is not None:
        slots = np.unique(np.concatenate([slots, np.asarray(slots_extra, np.int64)]))
    mx = wl.act_format == 1
    xr = gather_rows(wl.x, k, sch["assign_of_slot"], slots, mx)
    eor = expert_of_slots(sch["offsets"], slots)
    mxw = None
    if getattr(wl, "weight_format", 0) == 1:
        mxw = (mx_quantize_rows(wl.w_gu), mx_quantize_rows(wl.w_d))
    y, a_ex, y_ex = ffn_rows(xr, eor, wl.w_gu, wl.w_d, mx, mx_weights=mxw, exact=True)
    y_row_of_slot = np.full(max(sch["R"], 1), -1, np.int64)
    y_row_of_slot[slots] = np.arange(slots.size)
    out, written, o_ex = combine_tokens(y, y_row_of_slot, soa, gate, tokens, k, exact=True)
    res.update(slots=slots, x_rows=xr, y=y, tokens=tokens, out=out, written=written,
               a_exact=a_ex, y_exact=y_ex, out_exact=o_ex, expert_of_slot=eor)
    return res


# ---------------------------------------------------------------- backward
# The backward of the layer's share, in fp64 from the stored bf16 values
# (the pages report the backward pass beside the forward; its steps are the
# chain rule through the forward's, in reverse order: the merge, the down
# projection, SwiGLU, the gate/up projection, the pull dispatch).

def silu_and_grad(g: np.ndarray):
    """SiLU(g) = g s and its derivative s (1 + g (1 - s)), s = 1 / (1 + e^-g)."""
    s = 1.0 / (1.0 + np.exp(-g))
    return g * s, s * (1.0 + g * (1.0 - s))


def swiglu_backward_values(h: np.ndarray, da: np.ndarray) -> np.ndarray:
    """Backward of a = SiLU(g) u per row, fp64: h = [g, u] [n, 2I], da [n, I]
    -> dh = [dg, du] = [da u SiLU'(g), da SiLU(g)] [n, 2I]."""
    h = np.asarray(h, np.float64)
    da = np.asarray(da, np.float64)
    I = da.shape[1]
    g, u = h[:, :I], h[:, I:]
    sl, dsl = silu_and_grad(g)
    return np.concatenate([da * u * dsl, da * sl], axis=1)


def ffn_backward_values(x: np.ndarray, expert_of_row, w_gu: np.ndarray, w_d: np.ndarray,
                        dy: np.ndarray):
    """Backward of the expert SwiGLU FFN per row, all fp64 values: with
    h = W_gu[e] x = [g, u] and a = SiLU(g) u, y = W_d[e] a, returns
    (dh, dx): da = W_d[e]^T dy, dg = da u SiLU'(g), du = da SiLU(g),
    dh = [dg, du], dx = W_gu[e]^T dh.  x [n, H], w_gu [n_local, 2I, H],
    w_d [n_local, H, I], dy [n, H]."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    eor = np.asarray(expert_of_row, np.int64).reshape(-1)
    I = w_gu.shape[1] // 2
    dh = np.zeros((x.shape[0], 2 * I))
    dx = np.zeros_like(x)
    for e in np.unique(eor):
        r = np.nonzero(eor == e)[0]
        dh[r] = swiglu_backward_values(x[r] @ w_gu[e].T, dy[r] @ w_d[e])
        dx[r] = dh[r] @ w_gu[e]
    return dh, dx


def ffn_wgrad_values(x: np.ndarray, expert_of_row, w_gu: np.ndarray, dy: np.ndarray,
                     dh: np.ndarray, n_local: int, H: int):
    """Weight gradients of the expert FFN, fp64: per expert e over its rows,
    dW_d[e] = sum dy a^T with a = SiLU(g) u, h = W_gu[e] x = [g, u], and
    dW_gu[e] = sum dh x^T.  Returns (dW_gu [n_local, 2I, H], dW_d [n_local, H, I])."""
    x = np.asarray(x, np.float64)
    eor = np.asarray(expert_of_row, np.int64).reshape(-1)
    I = w_gu.shape[1] // 2
    dw_d = np.zeros((n_local, H, I))
    dw_gu = np.zeros((n_local, 2 * I, H))
    for e in np.unique(eor):
        r = np.nonzero(eor == e)[0]
        h = x[r] @ w_gu[e].T
        a = silu_and_grad(h[:, :I])[0] * h[:, I:]
        dw_d[e] = dy[r].T @ a
        dw_gu[e] = dh[r].T @ x[r]
    return dw_gu, dw_d


def backward(wl, dout_bits: np.ndarray) -> Dict[str, np.ndarray]:
    """Backward of the whole layer share for a workload with bf16 activations
    and weights, given dout (bf16 bits [T, H], the gradient of out): the
    schedule and the forward's stored rows (gathered x, y as bf16), then per
    routed slot s of token t, pick j, gate w: dy_s = w dout[t] and
    dgate[t, j] = <dout[t], y_s>; dx_s through ffn_backward_values; and
    dx[t] = sum over t's local slots of dx_s.  fp64 throughout.  Returns
    dy [R, H], dgate [T, k] (NaN where not local), dx [T, H] and written [T], and per
    slot the forward's rows: x_rows (bf16 bits), h = [g, u] and a (fp64), y (bf16)."""
    idx, gate = (route_topk(wl.logits, wl.k) if wl.routing_from_logits
                 else (wl.topk_idx, wl.topk_gate))
    sch = build_schedule(idx, wl.expert_base, wl.n_local)
    R, aos, soa = sch["R"], sch["assign_of_slot"], sch["slot_of_assign"]
    slots = np.arange(R)
    xr = gather_rows(wl.x, wl.k, aos, slots, False)
    eos = expert_of_slots(sch["offsets"], slots)
    y = ffn_rows(xr, eos, wl.w_gu, wl.w_d, False)
    t_of = aos[:R] // wl.k
    w = np.asarray(gate, np.float64).reshape(-1)[aos[:R]]
    dout_v = bf16_value(dout_bits).astype(np.float64)
    dy = w[:, None] * dout_v[t_of]
    dgate = np.full(idx.size, np.nan)
    dgate[aos[:R]] = np.sum(dout_v[t_of] * bf16_value(y).astype(np.float64), axis=1)
    dh, dx_s = ffn_backward_values(bf16_value(xr), eos, bf16_value(wl.w_gu).astype(np.float64),
                                   bf16_value(wl.w_d).astype(np.float64), dy)
    T = idx.shape[0]
    dx = np.zeros((T, wl.H))
    np.add.at(dx, t_of, dx_s)
    written = (soa.reshape(T, wl.k) >= 0).any(axis=1)
    dw_gu, dw_d = ffn_wgrad_values(bf16_value(xr), eos, bf16_value(wl.w_gu).astype(np.float64),
                                   dy, dh, wl.n_local, wl.H)
    xv = bf16_value(xr).astype(np.float64)
    wgu = bf16_value(wl.w_gu).astype(np.float64)
    h = np.zeros((R, 2 * wl.I))
    for e in np.unique(eos):
        r = np.nonzero(eos == e)[0]
        h[r] = xv[r] @ wgu[e].T
    a = silu_and_grad(h[:, :wl.I])[0] * h[:, wl.I:]
    return {"R": R, "dy": dy, "dgate": dgate.reshape(idx.shape), "dx": dx, "written": written,
            "y": y, "dh": dh, "expert_of_slot": eos, "token_of_slot": t_of, "dw_d": dw_d,
            "dw_gu": dw_gu, "x_rows": xr, "h": h, "a": a}


# ---------------------------------------------------------------- MXFP8 backward
def mx_quantize_values(v: np.ndarray):
    """MXFP8 of fp64 rows [n, K] in blocks of 32 along K -> (codes [n, K] u8,
    scales [n, K / 32] u8)."""
    v = np.asarray(v, np.float64)
    n, K = v.shape
    assert K % 32 == 0
    codes, scales = mx_quantize(v.reshape(-1))
    return codes.reshape(n, K), scales.reshape(n, K // 32)


def mx_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of MXFP8 rows: codes [n, K], scales [n, K / 32] -> fp64 [n, K]."""
    n, K = codes.shape
    return mx_dequantize(codes.reshape(-1), scales.reshape(-1)).reshape(n, K)


def backward_mx(wl, dout_bits: np.ndarray) -> Dict[str, np.ndarray]:
    """Backward of the whole layer share with MXFP8 activations and bf16
    weights (the article reports the MXFP8 backward beside the bf16 one; the
    MXFP8 quantisation sits in the data path, so here the backward's token
    operands dy and dh are MXFP8 like the forward's x and a).

    Each buffer the path stores is rounded once, from the fp64 value of its
    inputs as stored, where the path stores it:
      x_q     the forward's ring (MXFP8 of the gathered bf16 rows, along H)
      a_q     the forward's act (MXFP8 of SiLU(g) u, along I)
      y       the forward's y (bf16)
      dy_q    MXFP8 along H of w * dout[t], the product taken in fp32
      dgate   <dout[t], y_s> (fp64)
      h       bf16 of W_gu[e] x_q                  (g = h[:I], u = h[I:])
      dh_q    MXFP8 along 2I of swiglu_backward_values(h, W_d[e]^T dy_q)
              (I a multiple of 32: the dg and du blocks are separate)
      dx_s    bf16 of W_gu[e]^T dh_q
      dx[t]   bf16 of the sum of t's local dx_s
      dW_d[e] bf16 of sum_s dy_q a_q^T;  dW_gu[e] bf16 of sum_s dh_q x_q^T
    With MXFP8 weights (weight_format 1) every GEMM takes its weights quantised
    along its own contraction dimension, the forward's rule for each GEMM: the
    forward and the recompute of h use W_gu along H and W_d along I, the down
    dgrad W_d along H (its columns) and the gate/up dgrad W_gu along 2I (its
    columns).  The weight gradients contract over the slots and take no
    weights.
    Returns the stored values (bf16 bits, or MXFP8 codes and scales) and the
    fp64 values before each rounding (keys ending in _exact)."""
    assert wl.act_format == 1
    idx, gate = (route_topk(wl.logits, wl.k) if wl.routing_from_logits
                 else (wl.topk_idx, wl.topk_gate))
    sch = build_schedule(idx, wl.expert_base, wl.n_local)
    R, aos, soa = sch["R"], sch["assign_of_slot"], sch["slot_of_assign"]
    k, H, I = wl.k, wl.H, wl.I
    slots = np.arange(R)
    xc, xs = gather_rows(wl.x, k, aos, slots, True)
    xq = mx_values(xc, xs)
    eos = expert_of_slots(sch["offsets"], slots)
    w_mx = getattr(wl, "weight_format", 0) == 1
    mxw = (mx_quantize_rows(wl.w_gu), mx_quantize_rows(wl.w_d)) if w_mx else None
    y, a_ex, y_ex = ffn_rows((xc, xs), eos, wl.w_gu, wl.w_d, True, mx_weights=mxw, exact=True)
    ac, asc = mx_quantize_values(a_ex)
    aq = mx_values(ac, asc)
    t_of = aos[:R] // k
    w32 = np.asarray(gate, np.float32).reshape(-1)[aos[:R]]
    dout32 = bf16_value(dout_bits)
    dy32 = w32[:, None] * dout32[t_of]                     # fp32 products
    dyc, dys = mx_quantize_values(dy32.astype(np.float64))
    dyq = mx_values(dyc, dys)
    dout_v = dout32.astype(np.float64)
    dgate = np.full(idx.size, np.nan)
    dgate[aos[:R]] = np.sum(dout_v[t_of] * bf16_value(y).astype(np.float64), axis=1)
    wgu = bf16_value(wl.w_gu).astype(np.float64)
    wd = bf16_value(wl.w_d).astype(np.float64)
    wgu_h, wd_da, wgu_dx = wgu, wd, wgu                    # the weights of h, da and dx_s
    if w_mx:
        deq = lambda cs: mx_dequantize(cs[0].reshape(-1), cs[1].reshape(-1))
        wgu_h = deq(mxw[0]).reshape(wgu.shape)
        t_d = mx_quantize_rows(np.ascontiguousarray(np.swapaxes(wl.w_d, 1, 2)))   # [n_local][I][H]
        wd_da = np.swapaxes(deq(t_d).reshape(wl.n_local, I, H), 1, 2)
        t_gu = mx_quantize_rows(np.ascontiguousarray(np.swapaxes(wl.w_gu, 1, 2)))  # [n_local][H][2I]
        wgu_dx = np.swapaxes(deq(t_gu).reshape(wl.n_local, H, 2 * I), 1, 2)
    h_ex = np.zeros((R, 2 * I))
    dh_ex = np.zeros((R, 2 * I))
    for e in np.unique(eos):
        r = np.nonzero(eos == e)[0]
        h_ex[r] = xq[r] @ wgu_h[e].T
    h_bits = bf16_round(h_ex).reshape(R, 2 * I)
    hv = bf16_value(h_bits).astype(np.float64)
    for e in np.unique(eos):
        r = np.nonzero(eos == e)[0]
        dh_ex[r] = swiglu_backward_values(hv[r], dyq[r] @ wd_da[e])
    dhc, dhs = mx_quantize_values(dh_ex)
    dhq = mx_values(dhc, dhs)
    dxs_ex = np.zeros((R, H))
    for e in np.unique(eos):
        r = np.nonzero(eos == e)[0]
        dxs_ex[r] = dhq[r] @ wgu_dx[e]
    dxs_bits = bf16_round(dxs_ex).reshape(R, H)
    T = idx.shape[0]
    dx_ex = np.zeros((T, H))
    np.add.at(dx_ex, t_of, bf16_value(dxs_bits).astype(np.float64))
    dx_bits = bf16_round(dx_ex).reshape(T, H)
    written = (soa.reshape(T, k) >= 0).any(axis=1)
    dwd_ex = np.zeros((wl.n_local, H, I))
    dwg_ex = np.zeros((wl.n_local, 2 * I, H))
    for e in range(wl.n_local):
        r = np.nonzero(eos == e)[0]
        dwd_ex[e] = dyq[r].T @ aq[r]
        dwg_ex[e] = dhq[r].T @ xq[r]
    return {"R": R, "expert_of_slot": eos, "token_of_slot": t_of, "written": written,
            "slot_of_assign": soa, "assign_of_slot": aos, "offsets": sch["offsets"],
            "topk_idx": idx, "topk_gate": gate, "x_codes": xc, "x_scales": xs, "a_exact": a_ex, "a_codes": ac, "a_scales": asc,
            "y": y, "y_exact": y_ex, "dy_exact": dy32.astype(np.float64), "dy_codes": dyc,
            "dy_scales": dys, "dgate": dgate.reshape(idx.shape), "h_exact": h_ex, "h": h_bits,
            "dh_exact": dh_ex, "dh_codes": dhc, "dh_scales": dhs, "dx_slots_exact": dxs_ex,
            "dx_slots": dxs_bits, "dx_exact": dx_ex, "dx": dx_bits, "dw_d_exact": dwd_ex,
            "dw_d": bf16_round(dwd_ex).reshape(dwd_ex.shape), "dw_gu_exact": dwg_ex,
            "dw_gu": bf16_round(dwg_ex).reshape(dwg_ex.shape),
            "w_gu_h": wgu_h, "w_d_da": wd_da, "w_gu_dx": wgu_dx}
