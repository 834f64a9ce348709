"""libmok: one GPU's share of the Mixture-of-Kittens forward MoE layer on MI355X.

A thin ctypes binding over ``libmok.so`` (built from ``csrc/`` with hipcc
for gfx950).  Every function here has the name of the C entry point it
marshals and does nothing but convert arguments: torch tensors become device
pointers, ``stream=None`` becomes torch's current HIP stream, a non-zero
status becomes a :class:`MokError`.  All arithmetic runs in the HIP kernels.

There is no fallback: importing this package without a built ``libmok.so``
raises ``ImportError``.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmok.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "mok.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python token_dispatch_grouped_top_amd/build.py`")
# torch ships its own HIP runtime under the same soname; importing torch first
# makes libmok bind to that one, so torch's streams and allocations are valid
# for the library's launches (loading libmok first would pull in a second copy).
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

MOK_OK, MOK_ERR_INVALID_ARG, MOK_ERR_UNSUPPORTED, MOK_ERR_WORKSPACE = 0, 1, 2, 3
MOK_ERR_HIP, MOK_ERR_DEVICE, MOK_ERR_CAPACITY = 4, 5, 6
MOK_ACT_BF16, MOK_ACT_MXFP8_E4M3 = 0, 1
MOK_MODE_STREAM, MOK_MODE_PERSISTENT = 0, 1
MOK_W_BF16, MOK_W_MXFP8_E4M3 = 0, 1


class MokError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {mok_status_str(status)} ({status})")


class mok_layer_desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "hidden", "inter", "n_experts", "top_k", "expert_base", "n_local", "act_format",
        "minibatch", "ring_slots", "max_rows", "n_move_cus", "mode", "wait_timeout_us",
        "weights_packed", "no_split_k", "weight_format")]


class mok_tokens(C.Structure):
    _fields_ = [("part_ptr", C.c_void_p), ("n_partitions", C.c_int32), ("part_rows", C.c_int32)]


_P, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_DESC, _TOK = C.POINTER(mok_layer_desc), C.POINTER(mok_tokens)
_SIGS = {
    "mok_route_topk": (C.c_int, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "mok_route_gemm_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "mok_route_topk_gemm": (C.c_int, [_P, _P, _I32, _I32, _I32, _I32, _P, _SZ, _P, _P, _P]),
    "mok_schedule_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "mok_build_schedule": (C.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "mok_schedule_noalloc_max_bytes": (_SZ, []),
    "mok_build_schedule_noalloc": (C.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "mok_choose_minibatch": (_I32, [_I32, _I32, _I32, _I32, _I64]),
    "mok_build_windows": (C.c_int, [_P, _I32, _I32, _I32, _P, _P]),
    "mok_build_schedule_windows": (C.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32,
                                             _I32, _P, _P, _SZ, _P]),
    "mok_dispatch_gather": (C.c_int, [_TOK, _I32, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _I32,
                                      _I32, _P, _P]),
    "mok_expert_ffn": (C.c_int, [_DESC, _P, _P, _I32, _P, _I32, _I32, _P, _P, _P, _P, _I32, _P,
                                 _I32, _P, _SZ, _P]),
    "mok_gemm_workspace_size": (_SZ, []),
    "mok_expert_gate_up": (C.c_int, [_DESC, _P, _P, _I32, _P, _I32, _I32, _P, _P, _P, _I32, _P,
                                     _SZ, _P]),
    "mok_packed_weights_size": (C.c_int, [_DESC, C.POINTER(_SZ), C.POINTER(_SZ)]),
    "mok_pack_weights": (C.c_int, [_DESC, _P, _P, _P, _P, _P]),
    "mok_expert_down": (C.c_int, [_DESC, _P, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P, _SZ,
                                  _P]),
    "mok_combine": (C.c_int, [_P, _I32, _P, _P, _I32, _I32, _I32, _TOK, _P, _P]),
    "mok_combine_slots": (C.c_int, [_P, _I32, _P, _P, _I32, _I32, _P, _P, _I32, _I32, _TOK, _P,
                                    _P]),
    "mok_forward_workspace_size": (_SZ, [_DESC, _I32, _I32]),
    "mok_moe_forward": (C.c_int, [_DESC, _P, _I32, _TOK, _P, _P, _TOK, _P, _SZ, _P]),
    "mok_moe_forward_routed": (C.c_int, [_DESC, _P, _P, _I32, _TOK, _P, _P, _TOK, _P, _SZ, _P]),
    "mok_forward_router_workspace_size": (_SZ, [_DESC, _I32]),
    "mok_moe_forward_router": (C.c_int, [_DESC, _P, _I32, _TOK, _P, _P, _TOK, _P, _SZ, _P]),
    "mok_moe_forward_batches": (C.c_int, [_DESC, _I32, _P, _P, _I32, _TOK, _P, _P, _TOK, _P,
                                          _SZ, _P]),
    "mok_tune_forward": (C.c_int, [_DESC, _P, _I32, _P, _I32, _I32, _I32, _P, _P, _I32, _TOK,
                                   _P, _P, _TOK, _P, _SZ, _DESC, C.POINTER(C.c_float), _P]),
    "mok_packed_weights_bwd_size": (C.c_int, [_DESC, C.POINTER(_SZ), C.POINTER(_SZ)]),
    "mok_pack_weights_bwd": (C.c_int, [_DESC, _P, _P, _P, _P, _P]),
    "mok_combine_backward": (C.c_int, [_TOK, _P, _I32, _P, _P, _I32, _I32, _P, _I32, _I32, _P,
                                       _I32, _P, _P, _P]),
    "mok_expert_ffn_backward": (C.c_int, [_DESC, _P, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P,
                                          _P, _P, _I32, _P]),
    "mok_expert_gate_up_save_h": (C.c_int, [_DESC, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P,
                                            _P, _SZ, _P]),
    "mok_expert_ffn_backward_saved": (C.c_int, [_DESC, _P, _P, _I32, _I32, _P, _P, _P, _P, _P,
                                                _I32, _P]),
    "mok_wgrad_workspace_size": (_SZ, [_DESC, _I32]),
    "mok_expert_wgrad": (C.c_int, [_DESC, _P, _I32, _P, _I32, _P, _P, _I32, _P, _P, _P, _P, _SZ,
                                   _P]),
    "mok_dispatch_backward": (C.c_int, [_P, _I32, _P, _P, _I32, _I32, _P, _I32, _I32, _TOK, _P,
                                        _P]),
    "mok_expert_down_merge": (C.c_int, [_DESC, _P, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P,
                                        _P, _P, _TOK, _P, _P, _SZ, _P]),
    "mok_combine_slots_multi": (C.c_int, [_P, _I32, _P, _P, _I32, _I32, _P, _P, _I32, _I32, _TOK,
                                          _P, _P]),
    "mok_combine_backward_mx": (C.c_int, [_TOK, _P, _I32, _P, _P, _I32, _I32, _P, _I32, _I32,
                                          _P, _P, _I32, _P, _P, _P]),
    "mok_expert_gate_up_save_h_mx": (C.c_int, [_DESC, _P, _P, _I32, _P, _I32, _I32, _P, _P, _P,
                                               _I32, _P, _P, _SZ, _P]),
    "mok_expert_ffn_backward_mx": (C.c_int, [_DESC, _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _P,
                                             _P, _P, _I32, _P, _P, _P, _I32, _P]),
    "mok_expert_wgrad_mx": (C.c_int, [_DESC, _P, _P, _I32, _P, _P, _I32, _P, _P, _P, _P, _I32,
                                      _P, _P, _P, _P, _SZ, _P]),
    "mok_device_status": (C.c_int, [_P, C.POINTER(C.c_int32), _P]),
    "mok_forward_minibatch": (_I32, [_DESC, _I32]),
    "mok_status_str": (C.c_char_p, [C.c_int]),
    "mok_last_hip_error": (C.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args


def header_functions() -> List[str]:
    """Names of the functions include/mok.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mok_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, call: str) -> None:
    if status != MOK_OK:
        if status == MOK_ERR_HIP:
            call = f"{call} [{_lib.mok_last_hip_error().decode()}]"
        raise MokError(status, call)


class Tokens:
    """Token partitions on the device (a ``mok_tokens`` plus what keeps it alive).

    ``parts`` are bf16-bit tensors (torch.int16/uint16/bfloat16) of shape
    [part_rows, H] on the GPU; the pointer array is itself a device tensor.
    """

    def __init__(self, parts: Sequence, part_rows: Optional[int] = None):
        import torch
        self.parts = list(parts)
        rows = part_rows if part_rows is not None else self.parts[0].shape[0]
        dev = self.parts[0].device
        self.ptrs = torch.tensor([p.data_ptr() for p in self.parts], dtype=torch.int64, device=dev)
        self.c = mok_tokens(self.ptrs.data_ptr(), len(self.parts), rows)

    @classmethod
    def from_tensor(cls, x):
        return cls([x], x.shape[0])


# ------------------------------------------------------------------ calls
def mok_status_str(status: int) -> str:
    return _lib.mok_status_str(status).decode()


def mok_route_topk(logits, T: int, E: int, k: int, topk_idx, topk_gate, stream=None) -> None:
    _check(_lib.mok_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_gate),
                               _stream(stream)), "mok_route_topk")


def mok_route_gemm_workspace_size(T: int, E: int, H: int) -> int:
    return int(_lib.mok_route_gemm_workspace_size(T, E, H))


def mok_route_topk_gemm(x, w_router, T: int, H: int, E: int, k: int, ws, topk_idx, topk_gate,
                        ws_bytes: Optional[int] = None, stream=None) -> None:
    _check(_lib.mok_route_topk_gemm(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(ws),
                                    _ws_bytes(ws, ws_bytes), _ptr(topk_idx), _ptr(topk_gate),
                                    _stream(stream)), "mok_route_topk_gemm")


def mok_schedule_workspace_size(T: int, k: int, n_local: int) -> int:
    return int(_lib.mok_schedule_workspace_size(T, k, n_local))


def mok_build_schedule(topk_idx, T: int, k: int, expert_base: int, n_local: int, counts, offsets,
                       slot_of_assign, assign_of_slot, ws, ws_bytes: Optional[int] = None,
                       stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.mok_build_schedule(_ptr(topk_idx), T, k, expert_base, n_local, _ptr(counts),
                                   _ptr(offsets), _ptr(slot_of_assign), _ptr(assign_of_slot),
                                   _ptr(ws), ws_bytes, _stream(stream)), "mok_build_schedule")


def mok_schedule_noalloc_max_bytes() -> int:
    return int(_lib.mok_schedule_noalloc_max_bytes())


def mok_build_schedule_noalloc(topk_idx, T: int, k: int, expert_base: int, n_local: int, counts,
                               offsets, slot_of_assign, assign_of_slot, stream=None) -> None:
    _check(_lib.mok_build_schedule_noalloc(_ptr(topk_idx), T, k, expert_base, n_local,
                                           _ptr(counts), _ptr(offsets), _ptr(slot_of_assign),
                                           _ptr(assign_of_slot), _stream(stream)),
           "mok_build_schedule_noalloc")


def mok_choose_minibatch(n_cus: int, tile_m: int, tile_n: int, n_out: int, rows: int = 0) -> int:
    return int(_lib.mok_choose_minibatch(n_cus, tile_m, tile_n, n_out, rows))


def mok_build_schedule_windows(topk_idx, T: int, k: int, expert_base: int, n_local: int, counts,
                               offsets, slot_of_assign, assign_of_slot, M: int, nwin: int,
                               win_seg, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.mok_build_schedule_windows(_ptr(topk_idx), T, k, expert_base, n_local,
                                           _ptr(counts), _ptr(offsets), _ptr(slot_of_assign),
                                           _ptr(assign_of_slot), M, nwin, _ptr(win_seg), _ptr(ws),
                                           ws_bytes, _stream(stream)), "mok_build_schedule_windows")


def mok_build_windows(offsets, n_local: int, M: int, nwin: int, win_seg, stream=None) -> None:
    _check(_lib.mok_build_windows(_ptr(offsets), n_local, M, nwin, _ptr(win_seg),
                                  _stream(stream)), "mok_build_windows")


def mok_dispatch_gather(src: Tokens, H: int, k: int, assign_of_slot, offsets, n_local: int,
                        slot_begin: int, slot_end: int, ring, ring_scales, ring_slots: int,
                        act_format: int, dev_status=None, stream=None) -> None:
    _check(_lib.mok_dispatch_gather(C.byref(src.c), H, k, _ptr(assign_of_slot), _ptr(offsets),
                                    n_local, slot_begin, slot_end, _ptr(ring), _ptr(ring_scales),
                                    ring_slots, act_format, _ptr(dev_status), _stream(stream)),
           "mok_dispatch_gather")


def _ws_bytes(ws, ws_bytes):
    if ws is None:
        return 0
    return ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes


def mok_gemm_workspace_size() -> int:
    return int(_lib.mok_gemm_workspace_size())


def mok_expert_ffn(desc: mok_layer_desc, ring, ring_scales, ring_slots: int, offsets,
                   slot_begin: int, slot_end: int, w_gate_up, w_down, act, act_scales,
                   act_rows: int, y, y_rows: int, ws=None, ws_bytes: Optional[int] = None,
                   stream=None) -> None:
    _check(_lib.mok_expert_ffn(C.byref(desc), _ptr(ring), _ptr(ring_scales), ring_slots,
                               _ptr(offsets), slot_begin, slot_end, _ptr(w_gate_up), _ptr(w_down),
                               _ptr(act), _ptr(act_scales), act_rows, _ptr(y), y_rows, _ptr(ws),
                               _ws_bytes(ws, ws_bytes), _stream(stream)), "mok_expert_ffn")


def mok_packed_weights_size(desc: mok_layer_desc):
    """(gate_up_bytes, down_bytes) of the packed weights for desc."""
    gu, dn = _SZ(0), _SZ(0)
    _check(_lib.mok_packed_weights_size(C.byref(desc), C.byref(gu), C.byref(dn)),
           "mok_packed_weights_size")
    return gu.value, dn.value


def mok_pack_weights(desc: mok_layer_desc, w_gate_up, w_down, packed_gate_up, packed_down,
                     stream=None) -> None:
    _check(_lib.mok_pack_weights(C.byref(desc), _ptr(w_gate_up), _ptr(w_down),
                                 _ptr(packed_gate_up), _ptr(packed_down), _stream(stream)),
           "mok_pack_weights")


def mok_expert_gate_up(desc: mok_layer_desc, ring, ring_scales, ring_slots: int, offsets,
                       slot_begin: int, slot_end: int, w_gate_up, act, act_scales, act_rows: int,
                       ws=None, ws_bytes: Optional[int] = None, stream=None) -> None:
    _check(_lib.mok_expert_gate_up(C.byref(desc), _ptr(ring), _ptr(ring_scales), ring_slots,
                                   _ptr(offsets), slot_begin, slot_end, _ptr(w_gate_up),
                                   _ptr(act), _ptr(act_scales), act_rows, _ptr(ws),
                                   _ws_bytes(ws, ws_bytes), _stream(stream)),
           "mok_expert_gate_up")


def mok_expert_down(desc: mok_layer_desc, act, act_scales, act_rows: int, offsets,
                    slot_begin: int, slot_end: int, w_down, y, y_rows: int, ws=None,
                    ws_bytes: Optional[int] = None, stream=None) -> None:
    _check(_lib.mok_expert_down(C.byref(desc), _ptr(act), _ptr(act_scales), act_rows,
                                _ptr(offsets), slot_begin, slot_end, _ptr(w_down), _ptr(y),
                                y_rows, _ptr(ws), _ws_bytes(ws, ws_bytes), _stream(stream)),
           "mok_expert_down")


def mok_combine(y, y_rows: int, slot_of_assign, topk_gate, T: int, k: int, H: int, out: Tokens,
                dev_status=None, stream=None) -> None:
    _check(_lib.mok_combine(_ptr(y), y_rows, _ptr(slot_of_assign), _ptr(topk_gate), T, k, H,
                            C.byref(out.c), _ptr(dev_status), _stream(stream)), "mok_combine")


def mok_combine_slots(y, y_rows: int, assign_of_slot, offsets, n_local: int, n_slots: int,
                      slot_of_assign, topk_gate, k: int, H: int, out: Tokens, dev_status=None,
                      stream=None) -> None:
    _check(_lib.mok_combine_slots(_ptr(y), y_rows, _ptr(assign_of_slot), _ptr(offsets), n_local,
                                  n_slots, _ptr(slot_of_assign), _ptr(topk_gate), k, H,
                                  C.byref(out.c), _ptr(dev_status), _stream(stream)),
           "mok_combine_slots")


def mok_forward_workspace_size(desc: mok_layer_desc, T: int, n_macro: int = 1) -> int:
    return int(_lib.mok_forward_workspace_size(C.byref(desc), T, n_macro))


def mok_forward_minibatch(desc: mok_layer_desc, T: int) -> int:
    return int(_lib.mok_forward_minibatch(C.byref(desc), T))


def mok_moe_forward(desc: mok_layer_desc, logits, T: int, x: Tokens, w_gate_up, w_down,
                    out: Tokens, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.mok_moe_forward(C.byref(desc), _ptr(logits), T, C.byref(x.c), _ptr(w_gate_up),
                                _ptr(w_down), C.byref(out.c), _ptr(ws), ws_bytes,
                                _stream(stream)), "mok_moe_forward")


def mok_forward_router_workspace_size(desc: mok_layer_desc, T: int) -> int:
    return int(_lib.mok_forward_router_workspace_size(C.byref(desc), T))


def mok_moe_forward_router(desc: mok_layer_desc, w_router, T: int, x: Tokens, w_gate_up, w_down,
                           out: Tokens, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.mok_moe_forward_router(C.byref(desc), _ptr(w_router), T, C.byref(x.c),
                                       _ptr(w_gate_up), _ptr(w_down), C.byref(out.c), _ptr(ws),
                                       ws_bytes, _stream(stream)), "mok_moe_forward_router")


def mok_moe_forward_routed(desc: mok_layer_desc, topk_idx, topk_gate, T: int, x: Tokens,
                           w_gate_up, w_down, out: Tokens, ws, ws_bytes: Optional[int] = None,
                           stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.mok_moe_forward_routed(C.byref(desc), _ptr(topk_idx), _ptr(topk_gate), T,
                                       C.byref(x.c), _ptr(w_gate_up), _ptr(w_down),
                                       C.byref(out.c), _ptr(ws), ws_bytes, _stream(stream)),
           "mok_moe_forward_routed")


def mok_moe_forward_batches(desc: mok_layer_desc, n_macro: int, topk_idx: Sequence,
                            topk_gate: Sequence, T: int, x: Tokens, w_gate_up, w_down,
                            out: Sequence[Tokens], ws, ws_bytes: Optional[int] = None,
                            stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    idx_arr = (C.c_void_p * n_macro)(*[_ptr(t) for t in topk_idx])
    gate_arr = (C.c_void_p * n_macro)(*[_ptr(t) for t in topk_gate])
    out_arr = (mok_tokens * n_macro)(*[o.c for o in out])
    _check(_lib.mok_moe_forward_batches(C.byref(desc), n_macro, C.cast(idx_arr, C.c_void_p),
                                        C.cast(gate_arr, C.c_void_p), T, C.byref(x.c),
                                        _ptr(w_gate_up), _ptr(w_down), out_arr, _ptr(ws),
                                        ws_bytes, _stream(stream)), "mok_moe_forward_batches")


def mok_tune_forward(desc: mok_layer_desc, minibatches: Sequence[int], n_moves: Sequence[int],
                     reps: int, topk_idx: Sequence, topk_gate: Sequence, T: int, x: Tokens,
                     w_gate_up, w_down, out: Sequence[Tokens], ws, ws_bytes: Optional[int] = None,
                     stream=None):
    """Returns (best descriptor, its mean ms per call)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    n_macro = len(topk_idx)
    mb = (C.c_int32 * len(minibatches))(*minibatches)
    mv = (C.c_int32 * max(len(n_moves), 1))(*(list(n_moves) or [0]))
    idx_arr = (C.c_void_p * n_macro)(*[_ptr(t) for t in topk_idx])
    gate_arr = (C.c_void_p * n_macro)(*[_ptr(t) for t in topk_gate])
    out_arr = (mok_tokens * n_macro)(*[o.c for o in out])
    best = mok_layer_desc()
    ms = C.c_float(0.0)
    _check(_lib.mok_tune_forward(C.byref(desc), mb, len(minibatches), mv, len(n_moves), reps,
                                 n_macro, C.cast(idx_arr, C.c_void_p), C.cast(gate_arr, C.c_void_p),
                                 T, C.byref(x.c), _ptr(w_gate_up), _ptr(w_down), out_arr, _ptr(ws),
                                 ws_bytes, C.byref(best), C.byref(ms), _stream(stream)),
           "mok_tune_forward")
    return best, float(ms.value)


def mok_packed_weights_bwd_size(desc: mok_layer_desc):
    a, b = _SZ(0), _SZ(0)
    _check(_lib.mok_packed_weights_bwd_size(C.byref(desc), C.byref(a), C.byref(b)),
           "mok_packed_weights_bwd_size")
    return int(a.value), int(b.value)


def mok_pack_weights_bwd(desc: mok_layer_desc, w_gate_up, w_down, packed_gate_up_t, packed_down_t,
                         stream=None) -> None:
    _check(_lib.mok_pack_weights_bwd(C.byref(desc), _ptr(w_gate_up), _ptr(w_down),
                                     _ptr(packed_gate_up_t), _ptr(packed_down_t), _stream(stream)),
           "mok_pack_weights_bwd")


def mok_combine_backward(dout: Tokens, y, y_rows: int, assign_of_slot, offsets, n_local: int,
                         n_slots: int, topk_gate, k: int, H: int, dy, dy_rows: int, dgate,
                         dev_status=None, stream=None) -> None:
    _check(_lib.mok_combine_backward(C.byref(dout.c), _ptr(y), y_rows, _ptr(assign_of_slot),
                                     _ptr(offsets), n_local, n_slots, _ptr(topk_gate), k, H,
                                     _ptr(dy), dy_rows, _ptr(dgate), _ptr(dev_status),
                                     _stream(stream)), "mok_combine_backward")


def mok_expert_ffn_backward(desc: mok_layer_desc, ring, ring_slots: int, dy, offsets,
                            slot_begin: int, slot_end: int, w_gate_up, packed_gate_up_t,
                            packed_down_t, h, dh, dx_slots, rows: int, stream=None) -> None:
    _check(_lib.mok_expert_ffn_backward(C.byref(desc), _ptr(ring), ring_slots, _ptr(dy),
                                        _ptr(offsets), slot_begin, slot_end, _ptr(w_gate_up),
                                        _ptr(packed_gate_up_t), _ptr(packed_down_t), _ptr(h),
                                        _ptr(dh), _ptr(dx_slots), rows, _stream(stream)),
           "mok_expert_ffn_backward")


def mok_expert_gate_up_save_h(desc: mok_layer_desc, ring, ring_slots: int, offsets,
                              slot_begin: int, slot_end: int, w_gate_up, act, act_rows: int, h,
                              ws=None, ws_bytes: Optional[int] = None, stream=None) -> None:
    _check(_lib.mok_expert_gate_up_save_h(C.byref(desc), _ptr(ring), ring_slots, _ptr(offsets),
                                          slot_begin, slot_end, _ptr(w_gate_up), _ptr(act),
                                          act_rows, _ptr(h), _ptr(ws), _ws_bytes(ws, ws_bytes),
                                          _stream(stream)),
           "mok_expert_gate_up_save_h")


def mok_expert_ffn_backward_saved(desc: mok_layer_desc, dy, offsets, slot_begin: int,
                                  slot_end: int, packed_gate_up_t, packed_down_t, h, dh, dx_slots,
                                  rows: int, stream=None) -> None:
    _check(_lib.mok_expert_ffn_backward_saved(C.byref(desc), _ptr(dy), _ptr(offsets), slot_begin,
                                              slot_end, _ptr(packed_gate_up_t),
                                              _ptr(packed_down_t), _ptr(h), _ptr(dh),
                                              _ptr(dx_slots), rows, _stream(stream)),
           "mok_expert_ffn_backward_saved")


def mok_wgrad_workspace_size(desc: mok_layer_desc, rows: int) -> int:
    return int(_lib.mok_wgrad_workspace_size(C.byref(desc), rows))


def mok_expert_wgrad(desc: mok_layer_desc, ring, ring_slots: int, act, act_rows: int, dy, dh,
                     rows: int, offsets, dw_gate_up, dw_down, ws, ws_bytes: Optional[int] = None,
                     stream=None) -> None:
    _check(_lib.mok_expert_wgrad(C.byref(desc), _ptr(ring), ring_slots, _ptr(act), act_rows,
                                 _ptr(dy), _ptr(dh), rows, _ptr(offsets), _ptr(dw_gate_up),
                                 _ptr(dw_down), _ptr(ws), _ws_bytes(ws, ws_bytes), _stream(stream)),
           "mok_expert_wgrad")


def mok_dispatch_backward(dx_slots, rows: int, assign_of_slot, offsets, n_local: int, n_slots: int,
                          slot_of_assign, k: int, H: int, dx: Tokens, dev_status=None,
                          stream=None) -> None:
    _check(_lib.mok_dispatch_backward(_ptr(dx_slots), rows, _ptr(assign_of_slot), _ptr(offsets),
                                      n_local, n_slots, _ptr(slot_of_assign), k, H, C.byref(dx.c),
                                      _ptr(dev_status), _stream(stream)), "mok_dispatch_backward")


def mok_expert_down_merge(desc: mok_layer_desc, act, act_scales, act_rows: int, offsets,
                          slot_begin: int, slot_end: int, w_down, y, y_rows: int, assign_of_slot,
                          slot_of_assign, topk_gate, out: Tokens, merge_plan, ws=None,
                          ws_bytes: Optional[int] = None, stream=None) -> None:
    _check(_lib.mok_expert_down_merge(C.byref(desc), _ptr(act), _ptr(act_scales), act_rows,
                                      _ptr(offsets), slot_begin, slot_end, _ptr(w_down), _ptr(y),
                                      y_rows, _ptr(assign_of_slot), _ptr(slot_of_assign),
                                      _ptr(topk_gate), C.byref(out.c), _ptr(merge_plan), _ptr(ws),
                                      _ws_bytes(ws, ws_bytes), _stream(stream)),
           "mok_expert_down_merge")


def mok_combine_slots_multi(y, y_rows: int, assign_of_slot, offsets, n_local: int, n_slots: int,
                            slot_of_assign, topk_gate, k: int, H: int, out: Tokens,
                            dev_status=None, stream=None) -> None:
    _check(_lib.mok_combine_slots_multi(_ptr(y), y_rows, _ptr(assign_of_slot), _ptr(offsets),
                                        n_local, n_slots, _ptr(slot_of_assign), _ptr(topk_gate), k,
                                        H, C.byref(out.c), _ptr(dev_status), _stream(stream)),
           "mok_combine_slots_multi")


def mok_combine_backward_mx(dout: Tokens, y, y_rows: int, assign_of_slot, offsets, n_local: int,
                            n_slots: int, topk_gate, k: int, H: int, dy, dy_scales, dy_rows: int,
                            dgate, dev_status=None, stream=None) -> None:
    _check(_lib.mok_combine_backward_mx(C.byref(dout.c), _ptr(y), y_rows, _ptr(assign_of_slot),
                                        _ptr(offsets), n_local, n_slots, _ptr(topk_gate), k, H,
                                        _ptr(dy), _ptr(dy_scales), dy_rows, _ptr(dgate),
                                        _ptr(dev_status), _stream(stream)),
           "mok_combine_backward_mx")


def mok_expert_gate_up_save_h_mx(desc: mok_layer_desc, ring, ring_scales, ring_slots: int,
                                 offsets, slot_begin: int, slot_end: int, w_gate_up, act,
                                 act_scales, act_rows: int, h, ws=None,
                                 ws_bytes: Optional[int] = None, stream=None) -> None:
    _check(_lib.mok_expert_gate_up_save_h_mx(C.byref(desc), _ptr(ring), _ptr(ring_scales),
                                             ring_slots, _ptr(offsets), slot_begin, slot_end,
                                             _ptr(w_gate_up), _ptr(act), _ptr(act_scales),
                                             act_rows, _ptr(h), _ptr(ws), _ws_bytes(ws, ws_bytes),
                                             _stream(stream)),
           "mok_expert_gate_up_save_h_mx")


def mok_expert_ffn_backward_mx(desc: mok_layer_desc, ring, ring_scales, ring_slots: int, dy,
                               dy_scales, offsets, slot_begin: int, slot_end: int, w_gate_up,
                               packed_gate_up_t, packed_down_t, h, h_kept: bool, dh, dh_scales,
                               dx_slots, rows: int, stream=None) -> None:
    _check(_lib.mok_expert_ffn_backward_mx(C.byref(desc), _ptr(ring), _ptr(ring_scales),
                                           ring_slots, _ptr(dy), _ptr(dy_scales), _ptr(offsets),
                                           slot_begin, slot_end, _ptr(w_gate_up),
                                           _ptr(packed_gate_up_t), _ptr(packed_down_t), _ptr(h),
                                           1 if h_kept else 0, _ptr(dh), _ptr(dh_scales),
                                           _ptr(dx_slots), rows, _stream(stream)),
           "mok_expert_ffn_backward_mx")


def mok_expert_wgrad_mx(desc: mok_layer_desc, ring, ring_scales, ring_slots: int, act,
                        act_scales, act_rows: int, dy, dy_scales, dh, dh_scales, rows: int,
                        offsets, dw_gate_up, dw_down, ws, ws_bytes: Optional[int] = None,
                        stream=None) -> None:
    _check(_lib.mok_expert_wgrad_mx(C.byref(desc), _ptr(ring), _ptr(ring_scales), ring_slots,
                                    _ptr(act), _ptr(act_scales), act_rows, _ptr(dy),
                                    _ptr(dy_scales), _ptr(dh), _ptr(dh_scales), rows,
                                    _ptr(offsets), _ptr(dw_gate_up), _ptr(dw_down), _ptr(ws),
                                    _ws_bytes(ws, ws_bytes), _stream(stream)),
           "mok_expert_wgrad_mx")


def mok_device_status(ws, stream=None) -> int:
    v = C.c_int32(-1)
    _check(_lib.mok_device_status(_ptr(ws), C.byref(v), _stream(stream)), "mok_device_status")
    return int(v.value)
