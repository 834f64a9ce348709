"""Pins for the oracle's dispatch gather, expert SwiGLU FFN and weighted combine.

Gather = pull of each slot's token row (tahou.com MoK article, pull-dispatch
paragraph); FFN = SwiGLU expert over the expert-contiguous rows (grouped GEMM
and SwiGLU named in the article); combine = push back and final weighted
merge (benchmark-scope paragraph).  The pages fix no layout or rounding; the
readings pinned here: W_gu rows 0..I-1 gate, I..2I-1 up; W_d is [H, I]; the
activation and the expert output rounded to bf16 (RNE) from fp32; the merge
sums gate * y over the token's local picks in ascending slot order j.

Pins: closed forms (the square expert: y = c * x*x since SiLU(z) - SiLU(-z)
= z; one-hot weights), a dense SwiGLU MLP computed by torch on the CPU in
fp64 (E = 1, k = 1), and combine invariants (identity bypass, power-of-two
gate scaling, token permutation).
"""
import numpy as np
import pytest
import torch

import workloads as W


def _bits(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _val(bits):
    return W.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def test_gather_is_bit_copy(orc):
    wl = W.small_pool(11, n_partitions=3, part_rows=40, H=64, I=32, E=16, k=4,
                      expert_base=4, counts=[7, 30, 1, 12])
    s = orc.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    slots = np.arange(s["R"])
    rows = orc.gather_rows(wl.x, wl.k, s["assign_of_slot"], slots, mxfp8=False)
    assert np.array_equal(rows, wl.x[s["assign_of_slot"] // wl.k])
    codes, scales = orc.gather_rows(wl.x, wl.k, s["assign_of_slot"], slots, mxfp8=True)
    for r in range(0, s["R"], 7):
        c, sc = orc.mx_quantize(_val(wl.x[s["assign_of_slot"][r] // wl.k]))
        assert np.array_equal(codes[r], c) and np.array_equal(scales[r], sc)


def _square_expert_weights(H, n_local):
    I = 2 * H
    eye = np.eye(H)
    gate = np.concatenate([eye, -eye])           # [I, H]
    up = np.concatenate([eye, eye])              # [I, H]
    w_gu = np.stack([np.concatenate([gate, up]) for _ in range(n_local)])
    c = np.array([2.0 ** (e - 4) for e in range(n_local)])
    w_d = np.stack([c[e] * np.concatenate([eye, -eye], axis=1) for e in range(n_local)])
    return _bits(w_gu), _bits(w_d), c


def test_square_expert_closed_form(orc):
    """gate = [Id; -Id], up = [Id; Id], W_d = c_e [Id, -Id]  =>  y = c_e * x*x
    up to the bf16 rounding of the two activation halves and of y."""
    H, n_local = 64, 4
    w_gu, w_d, c = _square_expert_weights(H, n_local)
    rng = np.random.default_rng(0)
    x = _bits(rng.standard_normal((40, H)))
    e = rng.integers(0, n_local, 40).astype(np.int32)
    y = _val(orc.ffn_rows(x, e, w_gu, w_d, mxfp8=False))
    xv = _val(x)
    ref = c[e][:, None] * xv * xv
    bound = c[e][:, None] * 2.0 ** -8 * xv * xv + 2.0 ** -8 * np.abs(ref) + 1e-30
    assert np.all(np.abs(y - ref) <= bound)
    # a planted swap of gate and up would give 2 c x^2 sigmoid(x): far outside
    assert np.median(np.abs(y - ref) / (np.abs(ref) + 1e-30)) < 2.0 ** -8


def test_square_expert_layer(orc):
    """Whole chain on a routed workload with square experts:
    out_t = x_t^2 * sum_j gate_tj * c_{e_tj} (within bf16 rounding)."""
    wl = W.logits_workload("sq", 5, T=96, H=64, I=128, E=4, k=2, x_std=1.0, w_std=0.02)
    wl.w_gu, wl.w_d, c = _square_expert_weights(64, 4)
    r = orc.forward(wl)
    xv = _val(wl.x)
    coef = (r["topk_gate"].astype(np.float64) * c[r["topk_idx"]]).sum(1)
    ref = xv * xv * coef[:, None]
    got = _val(r["out"])
    assert r["written"].all()
    assert np.all(np.abs(got - ref) <= 2.0 ** -6 * np.abs(ref) + 1e-30)


def test_one_hot_weights(orc):
    """One gate row picks x[h0], the matching up row x[h1], one W_d entry routes
    the activation to output h2: y[h2] = bf16(bf16(SiLU(x[h0]) x[h1])), rest 0."""
    H, I = 32, 64
    h0, h1, h2, i0 = 3, 17, 30, 41
    w_gu = np.zeros((1, 2 * I, H))
    w_gu[0, i0, h0] = 1.0
    w_gu[0, I + i0, h1] = 1.0
    w_d = np.zeros((1, H, I))
    w_d[0, h2, i0] = 1.0
    rng = np.random.default_rng(1)
    x = _bits(rng.standard_normal((20, H)) * 2)
    y = _val(orc.ffn_rows(x, np.zeros(20, np.int32), _bits(w_gu), _bits(w_d), mxfp8=False))
    xv = torch.from_numpy(_val(x))
    a = (torch.nn.functional.silu(xv[:, h0]) * xv[:, h1]).float().to(torch.bfloat16)
    expect = np.zeros((20, H))
    expect[:, h2] = a.double().numpy()
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("mxfp8", [False, True])
def test_dense_mlp_vs_torch(orc, mxfp8):
    """E = 1, k = 1: the layer is a dense SwiGLU MLP; torch fp64 on the CPU."""
    H, I, n = 128, 96, 24
    rng = np.random.default_rng(2)
    x = _bits(rng.standard_normal((n, H)))
    w_gu = _bits(rng.standard_normal((1, 2 * I, H)) * 0.05)
    w_d = _bits(rng.standard_normal((1, H, I)) * 0.05)
    xv, wg, wd = (torch.from_numpy(_val(t)) for t in (x, w_gu[0], w_d[0]))
    if mxfp8:
        codes, scales = zip(*(orc.mx_quantize(_val(row)) for row in x))
        xin = (np.stack(codes), np.stack(scales))
        xv = torch.from_numpy(np.stack([orc.mx_dequantize(c, s) for c, s in zip(codes, scales)]))
    else:
        xin = x
    h = xv @ wg.T
    a = (torch.nn.functional.silu(h[:, :I]) * h[:, I:]).float().double()
    if mxfp8:
        a = torch.from_numpy(np.stack([orc.mx_dequantize(*orc.mx_quantize(r)) for r in a.numpy()]))
    else:
        a = a.float().to(torch.bfloat16).double()
    ref = (a @ wd.T).float().to(torch.bfloat16).double().numpy()
    y = _val(orc.ffn_rows(xin, np.zeros(n, np.int32), w_gu, w_d, mxfp8=mxfp8))
    # fp64 sums in another order may flip a rounding of a or y by one bf16 ulp
    close = np.abs(y - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6
    assert close.all()
    assert (y == ref).mean() > 0.95


def test_combine_identity_bypass(orc):
    """y := dispatched x (all experts local): out = bf16(sum_j gate_j x) = x within 1 ulp."""
    wl = W.logits_workload("bypass", 3, T=200, H=64, I=32, E=8, k=3, x_std=1.0, w_std=0.02)
    idx, gate = orc.route_topk(wl.logits, wl.k)
    s = orc.build_schedule(idx, 0, 8)
    y = orc.gather_rows(wl.x, wl.k, s["assign_of_slot"], np.arange(s["R"]), mxfp8=False)
    out, written = orc.combine_tokens(y, np.arange(s["R"]), s["slot_of_assign"], gate,
                                      np.arange(wl.T), wl.k)
    assert written.all()
    xv, ov = _val(wl.x), _val(out)
    assert np.all(np.abs(ov - xv) <= 2.0 ** -8 * np.abs(xv))


def test_combine_scaling_and_permutation(orc):
    wl = W.small_pool(12, n_partitions=2, part_rows=64, H=64, I=32, E=16, k=4,
                      expert_base=2, counts=[20, 5, 33])
    s = orc.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
    rng = np.random.default_rng(3)
    y = _bits(rng.standard_normal((s["R"], 64)))
    toks = np.arange(wl.T)
    out, written = orc.combine_tokens(y, np.arange(s["R"]), s["slot_of_assign"],
                                      wl.topk_gate, toks, wl.k)
    # tokens with no local pick are not written
    local = (s["slot_of_assign"].reshape(wl.T, wl.k) >= 0).any(1)
    assert np.array_equal(written, local)
    # power-of-two gates scale the output exactly
    out2, _ = orc.combine_tokens(y, np.arange(s["R"]), s["slot_of_assign"],
                                 wl.topk_gate * np.float32(4.0), toks, wl.k)
    assert np.array_equal(_val(out2)[written], 4.0 * _val(out)[written])
    # listing tokens in another order permutes the rows
    perm = rng.permutation(wl.T)
    out3, w3 = orc.combine_tokens(y, np.arange(s["R"]), s["slot_of_assign"],
                                  wl.topk_gate, perm, wl.k)
    assert np.array_equal(out3, out[perm]) and np.array_equal(w3, written[perm])


def _mx_exact_rows(rng, rows, K):
    """bf16 rows that MXFP8 represents exactly: each block of 32 is E4M3 codes times 2^E, with
    one element of magnitude in [256, 448] * 2^E, so the block's scale is exactly 2^E."""
    codes = rng.integers(0, 0x7F, (rows, K)).astype(np.uint8)           # finite magnitudes
    codes |= (rng.integers(0, 2, (rows, K)) << 7).astype(np.uint8)      # signs
    codes[:, ::32] = (0x78 + rng.integers(0, 7, (rows, K // 32))).astype(np.uint8) | \
        (codes[:, ::32] & 0x80)                                          # 256 .. 448
    E = rng.integers(-24, -4, (rows, K // 32))
    mag = np.where((codes & 0x78) == 0, (codes & 7) * 2.0 ** -9,
                   (8 + (codes & 7)) * 2.0 ** (((codes >> 3) & 15).astype(np.int64) - 10))
    v = np.where(codes & 0x80, -mag, mag) * 2.0 ** np.repeat(E, 32, axis=1)
    return _bits(v), codes, (E + 127).astype(np.uint8)


@pytest.mark.parametrize("mxfp8", [False, True])
def test_mx_weights_exact_reduce_to_bf16_path(orc, mxfp8):
    """MXFP8 weights (blocks of 32 along K, per row).  Weights that the format holds exactly
    quantise to the codes and scales they were built from, and the FFN with them is the bf16
    weight FFN bit for bit (a wrong block or row index in the dequantisation breaks both)."""
    H, I, n_local = 96, 64, 3
    rng = np.random.default_rng(21)
    wg, cg, sg = _mx_exact_rows(rng, n_local * 2 * I, H)
    wd, cd, sd = _mx_exact_rows(rng, n_local * H, I)
    w_gu, w_d = wg.reshape(n_local, 2 * I, H), wd.reshape(n_local, H, I)
    qg, qd = orc.mx_quantize_rows(w_gu), orc.mx_quantize_rows(w_d)
    assert np.array_equal(qg[0].reshape(-1, H), cg) and np.array_equal(qg[1].reshape(-1, H // 32), sg)
    assert np.array_equal(qd[0].reshape(-1, I), cd) and np.array_equal(qd[1].reshape(-1, I // 32), sd)
    x = _bits(rng.standard_normal((30, H)))
    xr = orc.mx_quantize(_val(x).reshape(-1)) if mxfp8 else x
    if mxfp8:
        xr = (xr[0].reshape(30, H), xr[1].reshape(30, H // 32))
    e = rng.integers(0, n_local, 30).astype(np.int32)
    y_bf16w = orc.ffn_rows(xr, e, w_gu, w_d, mxfp8)
    y_mxw = orc.ffn_rows(xr, e, w_gu, w_d, mxfp8, mx_weights=(qg, qd))
    assert np.array_equal(y_bf16w, y_mxw)


def test_mx_weights_saturating_scale_closed_form(orc):
    """Hand-derived MXFP8 weights: a block of 0.9 takes E = floor(log2 0.9) - 8 = -9 and
    0.9 * 2^9 = 460.8 saturates to 448, i.e. 0.875; a block of 0.3 takes E = -10 and
    307.2 rounds to the E4M3 value 320, i.e. 0.3125.  With x = 1 and H = 32:
    g = 32 * 0.875, u = 32 * 0.3125, a = bf16(SiLU(g) u), y = bf16(0.3125 * I * a)."""
    H, I = 32, 32
    w_gu = np.concatenate([np.full((I, H), 0.9), np.full((I, H), 0.3)])[None]
    w_d = np.full((1, H, I), 0.3)
    w_gu, w_d = _bits(w_gu), _bits(w_d)
    q = (orc.mx_quantize_rows(w_gu), orc.mx_quantize_rows(w_d))
    assert set(np.unique(q[0][1])) == {127 - 9, 127 - 10}
    x = _bits(np.ones((2, H)))
    y = _val(orc.ffn_rows(x, np.zeros(2, np.int32), w_gu, w_d, False, mx_weights=q))
    g, u = 32 * 0.875, 32 * 0.3125
    a = _val(_bits(np.float32(g / (1 + np.exp(-g)) * u)))
    expect = _val(_bits(np.float32(0.3125 * I * a)))
    assert np.all(y == expect)
