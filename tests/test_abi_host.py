"""Host-side checks of the libmok C-ABI (no GPU needed): the library loads,
exports every function include/mok.h declares, rejects bad arguments with
synchronous status codes before any launch, and its host-only minibatch rule
agrees with the oracle's independent one."""
import ctypes as C

import numpy as np
import pytest

import oracle
import token_dispatch_grouped_top_amd as mok


def test_exports_every_declared_symbol():
    names = mok.header_functions()
    assert len(names) >= 14
    missing = [n for n in names if not hasattr(mok._lib, n)]
    assert not missing, missing


def test_status_strings():
    for s in range(7):
        assert mok.mok_status_str(s)
    assert "capacity" in mok.mok_status_str(mok.MOK_ERR_CAPACITY)


def test_minibatch_rule_matches_oracle():
    rng = np.random.default_rng(0)
    for _ in range(500):
        n, tm, tn = int(rng.integers(1, 400)), int(rng.choice([16, 32, 64, 128, 256])), \
            int(rng.choice([16, 32, 64, 128, 256]))
        nout, rows = int(rng.integers(1, 40000)), int(rng.integers(0, 20000))
        assert mok.mok_choose_minibatch(n, tm, tn, nout, rows) == \
            oracle.choose_minibatch(n, tm, tn, nout, rows)
    assert mok.mok_choose_minibatch(148, 128, 256, 4096) == 2368


L = mok._lib


def test_invalid_arguments_rejected_without_launch():
    E = mok.MOK_ERR_INVALID_ARG
    assert L.mok_route_topk(1, 4, 8, 9, 1, 1, None) == E          # k > E
    assert L.mok_route_topk(1, 4, 8, 0, 1, 1, None) == E          # k = 0
    assert L.mok_route_topk(1, 4, 5000, 2, 1, 1, None) == E       # E too large
    assert L.mok_route_topk(0, 4, 8, 2, 1, 1, None) == E          # null logits
    ws = 1
    assert L.mok_build_schedule(1, 4, 2, 0, 0, 1, 1, 1, 1, ws, 1 << 20, None) == E  # n_local 0
    assert L.mok_build_schedule(1, 4, 2, 0, 300, 1, 1, 1, 1, ws, 1 << 20, None) == E
    assert L.mok_build_schedule(1, 4, 2, 0, 8, 1, 1, 1, 1, ws, 1, None) == mok.MOK_ERR_WORKSPACE
    assert L.mok_build_schedule(1, 1 << 28, 16, 0, 8, 1, 1, 1, 1, ws, 1 << 40, None) == \
        mok.MOK_ERR_UNSUPPORTED
    assert L.mok_build_windows(0, 8, 64, 4, 1, None) == E
    assert L.mok_build_windows(1, 8, 0, 4, 1, None) == E
    sw = L.mok_build_schedule_windows
    assert sw(1, 4, 2, 0, 8, 1, 1, 1, 1, 0, 4, 1, ws, 1 << 20, None) == E          # M = 0
    assert sw(1, 4, 2, 0, 8, 1, 1, 1, 1, 64, 4, None, ws, 1 << 20, None) == E      # no win_seg
    assert sw(1, 4, 2, 0, 0, 1, 1, 1, 1, 64, 4, 1, ws, 1 << 20, None) == E         # n_local 0
    assert sw(1, 4, 2, 0, 8, 1, 1, 1, 1, 64, 4, 1, ws, 1, None) == mok.MOK_ERR_WORKSPACE
    tok = mok.mok_tokens(1, 1, 16)
    assert L.mok_dispatch_gather(C.byref(tok), 60, 2, 1, 1, 8, 0, 10, 1, 1, 4, 1, None, None) == E
    assert L.mok_dispatch_gather(C.byref(tok), 64, 2, 1, 1, 8, 5, 4, 1, None, 4, 0, None, None) == E
    assert L.mok_dispatch_gather(C.byref(tok), 64, 2, 1, 1, 8, 0, 4, 1, None, 4, 1, None, None) == E
    assert L.mok_combine(1, 4, 1, 1, 17, 2, 64, C.byref(tok), None, None) == E  # T > rows
    assert L.mok_combine(1, 4, 1, 1, 16, 2, 60, C.byref(tok), None, None) == E  # H % 8
    # backward: the bf16 calls refuse an MXFP8 desc and the _mx calls a bf16
    # one; H % 64 for the merge backward, null buffers and scales
    dmx = _desc(act_format=1)
    a, b = C.c_size_t(0), C.c_size_t(0)
    assert L.mok_packed_weights_bwd_size(C.byref(dmx), C.byref(a), C.byref(b)) == 0
    a2, b2 = C.c_size_t(0), C.c_size_t(0)
    assert L.mok_packed_weights_bwd_size(C.byref(_desc()), C.byref(a2), C.byref(b2)) == 0
    assert (a.value, b.value) == (a2.value, b2.value) and a.value > 0
    assert L.mok_packed_weights_bwd_size(C.byref(_desc(act_format=1, weight_format=1)),
                                         C.byref(a), C.byref(b)) == E
    assert L.mok_combine_backward_mx(C.byref(tok), 1, 4, 1, 1, 8, 4, 1, 2, 64, 1, None, 4, 1,
                                     None, None) == E                  # null dy scales
    assert L.mok_combine_backward_mx(C.byref(tok), 1, 4, 1, 1, 8, 4, 1, 2, 96, 1, 1, 4, 1,
                                     None, None) == E                  # H % 64
    assert L.mok_expert_ffn_backward(C.byref(dmx), 1, 8, 1, 1, 0, 8, 1, 1, 1, 1, 1, 1, 8,
                                     None) == E
    assert L.mok_expert_ffn_backward_mx(C.byref(_desc()), 1, 1, 8, 1, 1, 1, 0, 8, 1, 1, 1, 1, 0,
                                        1, 1, 1, 8, None) == E         # bf16 desc
    assert L.mok_expert_ffn_backward_mx(C.byref(dmx), 1, 1, 8, 1, 1, 1, 0, 8, 1, 1, 1, 1, 0,
                                        1, None, 1, 8, None) == E      # null dh scales
    assert L.mok_expert_ffn_backward_mx(C.byref(dmx), None, None, 8, 1, 1, 1, 0, 8, None, 1, 1,
                                        1, 0, 1, 1, 1, 8, None) == E   # recompute needs the ring
    assert L.mok_expert_gate_up_save_h_mx(C.byref(_desc()), 1, 1, 64, 1, 0, 64, 1, 1, 1, 64, 1,
                                          None, 0, None) == E          # bf16 desc
    assert L.mok_expert_gate_up_save_h_mx(C.byref(dmx), 1, None, 64, 1, 0, 64, 1, 1, 1, 64, 1,
                                          None, 0, None) == E          # null ring scales
    assert L.mok_combine_backward(C.byref(tok), 1, 4, 1, 1, 8, 4, 1, 2, 60, 1, 4, 1, None, None) == E
    assert L.mok_combine_backward(C.byref(tok), None, 4, 1, 1, 8, 4, 1, 2, 64, 1, 4, 1, None, None) == E
    db = _desc()
    assert L.mok_expert_ffn_backward(C.byref(db), 1, 8, 1, 1, 0, 8, 1, 1, 1, None, 1, 1, 8, None) == E
    assert L.mok_dispatch_backward(None, 8, 1, 1, 8, 4, 1, 2, 64, C.byref(tok), None, None) == E
    need = L.mok_wgrad_workspace_size(C.byref(db), 64)
    assert need > 0 and L.mok_wgrad_workspace_size(C.byref(dmx), 64) == need
    assert L.mok_expert_wgrad(C.byref(dmx), 1, 64, 1, 64, 1, 1, 64, 1, 1, 1, 1, need, None) == E
    assert L.mok_expert_wgrad_mx(C.byref(db), 1, 1, 64, 1, 1, 64, 1, 1, 1, 1, 64, 1, 1, 1, 1,
                                 need, None) == E                      # bf16 desc
    assert L.mok_expert_wgrad_mx(C.byref(dmx), 1, 1, 64, 1, None, 64, 1, 1, 1, 1, 64, 1, 1, 1,
                                 1, need, None) == E                   # null act scales
    assert L.mok_expert_wgrad_mx(C.byref(dmx), 1, 1, 64, 1, 1, 64, 1, 1, 1, 1, 64, 1, 1, 1, 1,
                                 need - 1, None) == mok.MOK_ERR_WORKSPACE
    assert L.mok_expert_wgrad(C.byref(db), 1, 64, 1, 64, 1, 1, 64, 1, None, None, 1, need, None) == E
    assert L.mok_expert_wgrad(C.byref(db), 1, 64, 1, 64, 1, 1, 64, 1, 1, 1, 1, need - 1, None) == \
        mok.MOK_ERR_WORKSPACE
    # down GEMM merging single-slot tokens: routing arrays and out required
    assert L.mok_expert_down_merge(C.byref(db), 1, None, 64, 1, 0, 64, 1, 1, 64, None, 1, 1,
                                   C.byref(tok), 1, None, 0, None) == E
    assert L.mok_expert_down_merge(C.byref(db), 1, None, 64, 1, 0, 64, 1, 1, 64, 1, 1, 1, None,
                                   1, None, 0, None) == E
    assert L.mok_expert_down_merge(C.byref(db), 1, None, 64, 1, 0, 64, 1, 1, 64, 1, 1, 1,
                                   C.byref(tok), None, None, 0, None) == E   # no plan buffer
    assert L.mok_expert_down_merge(C.byref(db), 1, None, 64, 1, 0, 65, 1, 1, 64, 1, 1, 1,
                                   C.byref(tok), 1, None, 0, None) == E      # slot_end > y_rows
    assert L.mok_expert_down_merge(C.byref(dmx), 1, None, 64, 1, 0, 64, 1, 1, 64, 1, 1, 1,
                                   C.byref(tok), 1, None, 0, None) == E   # MXFP8 act, no scales
    assert L.mok_combine_slots_multi(1, 4, 1, 1, 8, 4, 1, 1, 2, 60, C.byref(tok), None,
                                     None) == E                        # H % 8
    assert L.mok_combine_slots_multi(None, 4, 1, 1, 8, 4, 1, 1, 2, 64, C.byref(tok), None,
                                     None) == E
    # tuner: no candidates, reps < 1, null result pointers
    d = _desc()
    one = (C.c_int32 * 1)(64)
    f = C.c_float(0.0)
    best = mok.mok_layer_desc()
    assert L.mok_tune_forward(C.byref(d), one, 0, None, 0, 1, 1, 1, 1, 4, C.byref(tok), 1, 1,
                              C.byref(tok), 1, 1 << 20, C.byref(best), C.byref(f), None) == E
    assert L.mok_tune_forward(C.byref(d), one, 1, None, 0, 0, 1, 1, 1, 4, C.byref(tok), 1, 1,
                              C.byref(tok), 1, 1 << 20, C.byref(best), C.byref(f), None) == E
    assert L.mok_tune_forward(C.byref(d), one, 1, None, 0, 1, 1, 1, 1, 4, C.byref(tok), 1, 1,
                              C.byref(tok), 1, 1 << 20, None, C.byref(f), None) == E
    # router GEMM + route: H % 16, k > E, null inputs, workspace below the query
    assert L.mok_route_topk_gemm(1, 1, 4, 60, 8, 2, 1, 1 << 20, 1, 1, None) == E
    assert L.mok_route_topk_gemm(1, 1, 4, 64, 8, 9, 1, 1 << 20, 1, 1, None) == E
    assert L.mok_route_topk_gemm(None, 1, 4, 64, 8, 2, 1, 1 << 20, 1, 1, None) == E
    need = L.mok_route_gemm_workspace_size(4, 8, 64)
    assert need >= 4 * 8 * 4
    assert L.mok_route_topk_gemm(1, 1, 4, 64, 8, 2, 1, need - 1, 1, 1, None) == mok.MOK_ERR_WORKSPACE
    assert L.mok_route_topk_gemm(None, None, 0, 64, 8, 2, None, 0, None, None, None) == mok.MOK_OK


def _desc(**kw):
    d = mok.mok_layer_desc(hidden=256, inter=512, n_experts=8, top_k=2, expert_base=0, n_local=8)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("bad", [dict(hidden=100), dict(inter=96), dict(n_local=0),
                                 dict(n_local=300), dict(top_k=9), dict(top_k=0),
                                 dict(expert_base=4), dict(act_format=3), dict(mode=7),
                                 dict(minibatch=-1), dict(ring_slots=64, minibatch=128)])
def test_bad_descriptors(bad):
    d = _desc(**bad)
    assert mok.mok_forward_workspace_size(d, 256, 1) == 0
    tok = mok.mok_tokens(1, 1, 256)
    st = L.mok_moe_forward_routed(C.byref(d), 1, 1, 256, C.byref(tok), 1, 1, C.byref(tok), 1,
                                  1 << 40, None)
    assert st in (mok.MOK_ERR_INVALID_ARG, mok.MOK_ERR_UNSUPPORTED)
    st = L.mok_moe_forward(C.byref(d), 1, 256, C.byref(tok), 1, 1, C.byref(tok), 1, 1 << 40, None)
    assert st in (mok.MOK_ERR_INVALID_ARG, mok.MOK_ERR_UNSUPPORTED)


def test_workspace_query_and_small_workspace():
    d = _desc(max_rows=512)
    n = mok.mok_forward_workspace_size(d, 256, 1)
    assert n > 0
    assert mok.mok_forward_workspace_size(d, 256, 2) > n
    tok = mok.mok_tokens(1, 1, 256)
    st = L.mok_moe_forward_routed(C.byref(d), 1, 1, 256, C.byref(tok), 1, 1, C.byref(tok), 1,
                                  n - 1, None)
    assert st == mok.MOK_ERR_WORKSPACE
    st = L.mok_moe_forward(C.byref(d), 1, 256, C.byref(tok), 1, 1, C.byref(tok), 1, n - 1, None)
    assert st == mok.MOK_ERR_WORKSPACE
    # the logits form needs logits when there are tokens
    st = L.mok_moe_forward(C.byref(d), None, 256, C.byref(tok), 1, 1, C.byref(tok), 1, n, None)
    assert st == mok.MOK_ERR_INVALID_ARG


def test_forward_minibatch_plan():
    # the rule for both GEMMs of a window, the larger; no GPU here: 256 CUs
    for H, I, T, k in ((7168, 2048, 1024, 8), (4096, 14336, 4096, 2), (256, 512, 256, 2)):
        d = mok.mok_layer_desc(hidden=H, inter=I, n_experts=8, top_k=k, expert_base=0, n_local=8)
        want = max(oracle.choose_minibatch(256, 256, 256, 2 * I, T * k),
                   oracle.choose_minibatch(256, 256, 256, H, T * k))
        assert mok.mok_forward_minibatch(d, T) == want
    # explicit minibatch is clipped to the row capacity; S defaults to 2M
    assert mok.mok_forward_minibatch(_desc(minibatch=100), 256) == 100
    assert mok.mok_forward_minibatch(_desc(minibatch=5000), 256) == 512
    assert mok.mok_forward_minibatch(_desc(minibatch=100, max_rows=64), 256) == 64


def test_packed_weight_sizes_and_argument_checks():
    d = mok.mok_layer_desc(hidden=576, inter=320, n_experts=32, top_k=4, expert_base=3,
                           n_local=5)
    gu, dn = mok.mok_packed_weights_size(d)
    # column tiles of 128 intermediate columns (gate + up rows: 256) and of 256 hidden rows
    assert gu == 5 * 3 * 256 * 576 * 2 and dn == 5 * 3 * 256 * 320 * 2
    E = mok.MOK_ERR_INVALID_ARG
    assert L.mok_pack_weights(C.byref(d), 1, None, None, None, None) == E     # source, no target
    assert L.mok_pack_weights(C.byref(d), None, None, None, None, None) == E  # nothing to pack
    assert L.mok_pack_weights(C.byref(d), None, 1, None, None, None) == E     # down half-pair
    bad = mok.mok_layer_desc(hidden=576, inter=320, n_experts=32, top_k=4, expert_base=3,
                             n_local=5, weights_packed=2)
    assert L.mok_packed_weights_size(C.byref(bad), None, None) == E


def test_gemm_operand_limits_and_workspace_checks():
    """Operands the GEMMs address with 32-bit byte offsets must be under 4 GiB; a GEMM
    workspace smaller than the query is rejected.  Both before any launch."""
    d = mok.mok_layer_desc(hidden=7168, inter=2048, n_experts=384, top_k=8, expert_base=0,
                           n_local=8)
    U = mok.MOK_ERR_UNSUPPORTED
    big_ring = (1 << 31) // 7168 + 1          # ring_slots * H * 2 bytes >= 4 GiB
    assert L.mok_expert_gate_up(C.byref(d), 1, None, big_ring, 1, 0, 8, 1, 1, None, 8, None, 0,
                                None) == U
    big_act = (1 << 31) // 2048 + 1
    assert L.mok_expert_down(C.byref(d), 1, None, big_act, 1, 0, 8, 1, 1, 8, None, 0, None) == U
    assert L.mok_expert_ffn(C.byref(d), 1, None, 8, 1, 0, 8, 1, 1, 1, None, big_act, 1, 8, None,
                            0, None) == U
    # the same ring is fine as E4M3 codes (1 byte per element) -- fails later on the scales
    mx = mok.mok_layer_desc(hidden=7168, inter=2048, n_experts=384, top_k=8, expert_base=0,
                            n_local=8, act_format=mok.MOK_ACT_MXFP8_E4M3)
    assert L.mok_expert_gate_up(C.byref(mx), 1, None, big_ring, 1, 0, 8, 1, 1, None, 8, None, 0,
                                None) == mok.MOK_ERR_INVALID_ARG
    # fused plan: a ring of 2 x minibatch rows past the limit
    big = mok.mok_layer_desc(hidden=7168, inter=2048, n_experts=384, top_k=8, expert_base=0,
                             n_local=8, minibatch=(1 << 30) // 7168 + 1,
                             max_rows=(1 << 30) // 7168 + 1)
    assert mok.mok_forward_workspace_size(big, 1 << 20, 1) == 0
    assert mok.mok_gemm_workspace_size() > 0
    assert L.mok_expert_down(C.byref(d), 1, None, 8, 1, 0, 8, 1, 1, 8, 1, 1024, None) == \
        mok.MOK_ERR_WORKSPACE


def test_saved_h_calls_validate_before_launch():
    E = mok.MOK_ERR_INVALID_ARG
    d = mok.mok_layer_desc(hidden=256, inter=128, n_experts=8, top_k=2, expert_base=0, n_local=4,
                           act_format=mok.MOK_ACT_BF16, weight_format=0)
    dmx = mok.mok_layer_desc(hidden=256, inter=128, n_experts=8, top_k=2, expert_base=0,
                             n_local=4, act_format=mok.MOK_ACT_MXFP8_E4M3, weight_format=0)
    # gate/up keeping h: bf16 only, h required
    assert L.mok_expert_gate_up_save_h(C.byref(dmx), 1, 64, 1, 0, 64, 1, 1, 64, 1, None, 0,
                                       None) == E
    assert L.mok_expert_gate_up_save_h(C.byref(d), 1, 64, 1, 0, 64, 1, 1, 64, None, None, 0,
                                       None) == E
    assert L.mok_expert_gate_up_save_h(C.byref(d), 1, 64, 1, 5, 4, 1, 1, 64, 1, None, 0,
                                       None) == E
    # backward from a saved h: every buffer required, bf16 only
    assert L.mok_expert_ffn_backward_saved(C.byref(d), 1, 1, 0, 64, 1, 1, None, 1, 1, 64,
                                           None) == E
    assert L.mok_expert_ffn_backward_saved(C.byref(dmx), 1, 1, 0, 64, 1, 1, 1, 1, 1, 64,
                                           None) == E
    assert L.mok_expert_ffn_backward_saved(C.byref(d), 1, 1, 0, 64, 1, 1, 1, 1, 1, 0,
                                           None) == E


def test_schedule_noalloc_refuses_beyond_its_array():
    """The no-allocation schedule checks its fixed scratch size before any device
    call: more assignments than its array holds is MOK_ERR_UNSUPPORTED."""
    cap = mok.mok_schedule_noalloc_max_bytes()
    assert cap == 4 << 20
    T, k, nl = 600_000, 8, 256                      # 4.8 M assignments x 256 experts
    assert mok.mok_schedule_workspace_size(T, k, nl) > cap
    st = L.mok_build_schedule_noalloc(1, T, k, 0, nl, 1, 1, 1, 1, None)
    assert st == mok.MOK_ERR_UNSUPPORTED
    st = L.mok_build_schedule_noalloc(1, 16, 2, 0, 0, 1, 1, 1, 1, None)
    assert st == mok.MOK_ERR_INVALID_ARG
