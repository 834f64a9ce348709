"""Pins for the oracle's backward of the expert FFN (the chain rule through
gate/up, SwiGLU and down; the pages report the backward pass beside the
forward).

Pinned against things the oracle does not compute itself:
  - central finite differences of the scalar <dy, y(x)> of an fp64 forward,
    for dx and for dh (so a dropped term of SiLU', a swapped g/u or a
    transposed weight fails);
  - the closed form of the "square" expert (gate = [Id; -Id], up = [Id; Id],
    down = c [Id, -Id] gives y = c x*x, so dx = 2 c x dy exactly).
"""
import numpy as np
import pytest


def _forward(x, eor, w_gu, w_d):
    I = w_gu.shape[1] // 2
    y = np.zeros((x.shape[0], w_d.shape[1]))
    for r in range(x.shape[0]):
        h = w_gu[eor[r]] @ x[r]
        g, u = h[:I], h[I:]
        y[r] = w_d[eor[r]] @ (g / (1.0 + np.exp(-g)) * u)
    return y


def test_ffn_backward_finite_differences(orc):
    rng = np.random.default_rng(3)
    n, nl, H, I = 5, 2, 8, 4
    x = rng.standard_normal((n, H))
    w_gu = rng.standard_normal((nl, 2 * I, H)) * 0.5
    w_d = rng.standard_normal((nl, H, I)) * 0.5
    dy = rng.standard_normal((n, H))
    eor = np.array([0, 1, 1, 0, 1])
    dh, dx = orc.ffn_backward_values(x, eor, w_gu, w_d, dy)
    f = lambda xx: float(np.sum(dy * _forward(xx, eor, w_gu, w_d)))
    eps = 1e-6
    num = np.zeros_like(x)
    for r in range(n):
        for c in range(H):
            xp, xm = x.copy(), x.copy()
            xp[r, c] += eps
            xm[r, c] -= eps
            num[r, c] = (f(xp) - f(xm)) / (2 * eps)
    assert np.allclose(dx, num, rtol=1e-6, atol=1e-7)
    # dh against differences in h = [g, u] itself
    for r in range(n):
        h = w_gu[eor[r]] @ x[r]
        fh = lambda hh: float(dy[r] @ (w_d[eor[r]] @ (hh[:I] / (1.0 + np.exp(-hh[:I])) * hh[I:])))
        for c in range(2 * I):
            hp, hm = h.copy(), h.copy()
            hp[c] += eps
            hm[c] -= eps
            assert abs(dh[r, c] - (fh(hp) - fh(hm)) / (2 * eps)) <= 1e-6 * (1 + abs(dh[r, c]))


def test_ffn_backward_square_expert_closed_form(orc):
    rng = np.random.default_rng(4)
    H, c = 6, 0.75
    Id = np.eye(H)
    w_gu = np.concatenate([Id, -Id, Id, Id], axis=0)[None]        # gate [Id; -Id], up [Id; Id]
    w_d = (c * np.concatenate([Id, -Id], axis=1))[None]           # down c [Id, -Id]
    x = rng.standard_normal((4, H))
    dy = rng.standard_normal((4, H))
    y = _forward(x, np.zeros(4, int), w_gu, w_d)
    assert np.allclose(y, c * x * x, rtol=1e-12, atol=1e-12)      # the forward identity
    _, dx = orc.ffn_backward_values(x, np.zeros(4, int), w_gu, w_d, dy)
    assert np.allclose(dx, 2 * c * x * dy, rtol=1e-12, atol=1e-12)


def test_ffn_wgrad_finite_differences(orc):
    """dW_d and dW_gu against central differences of <dy, y> in the weights."""
    rng = np.random.default_rng(5)
    n, nl, H, I = 6, 2, 5, 3
    x = rng.standard_normal((n, H))
    w_gu = rng.standard_normal((nl, 2 * I, H)) * 0.5
    w_d = rng.standard_normal((nl, H, I)) * 0.5
    dy = rng.standard_normal((n, H))
    eor = np.array([0, 1, 1, 0, 1, 1])
    dh, _ = orc.ffn_backward_values(x, eor, w_gu, w_d, dy)
    dw_gu, dw_d = orc.ffn_wgrad_values(x, eor, w_gu, dy, dh, nl, H)
    eps = 1e-6
    f = lambda g, d: float(np.sum(dy * _forward(x, eor, g, d)))
    for e in range(nl):
        for i in range(H):
            for j in range(I):
                p_, m_ = w_d.copy(), w_d.copy()
                p_[e, i, j] += eps
                m_[e, i, j] -= eps
                assert abs(dw_d[e, i, j] - (f(w_gu, p_) - f(w_gu, m_)) / (2 * eps)) < 1e-6
        for i in range(2 * I):
            for j in range(H):
                p_, m_ = w_gu.copy(), w_gu.copy()
                p_[e, i, j] += eps
                m_[e, i, j] -= eps
                assert abs(dw_gu[e, i, j] - (f(p_, w_d) - f(m_, w_d)) / (2 * eps)) < 1e-6


def test_layer_backward_glue_finite_differences(orc):
    """The whole-layer backward of oracle.backward (merge backward: dy = w dout
    and dgate = <dout, y>; the dispatch backward: dx[t] = sum over t's local
    slots) against central differences of L = sum_t <dout[t], out[t]> through
    an unrounded fp64 forward written here from the layer's definition:
    out[t] = sum over t's local picks j of w_tj W_d[e_tj] (SiLU(g) u), with
    [g, u] = W_gu[e_tj] x[t].  A wrong pick <-> slot mapping, gate index or
    dispatch sum moves dx or dgate far outside the bars; tokens without a
    local pick must get no gradient."""
    import workloads as W
    wl = W.small_pool(91, n_partitions=2, part_rows=7, H=32, I=16, E=7, k=3, expert_base=2,
                      counts=[5, 0, 6, 3])
    val = lambda b: orc.bf16_value(b).astype(np.float64)
    x, w_gu, w_d = val(wl.x), val(wl.w_gu) * 20.0, val(wl.w_d) * 20.0  # O(1) activations
    wl.w_gu = orc.bf16_round(w_gu).reshape(w_gu.shape)
    wl.w_d = orc.bf16_round(w_d).reshape(w_d.shape)
    w_gu, w_d = val(wl.w_gu), val(wl.w_d)
    gates = wl.topk_gate.astype(np.float64)
    idx = wl.topk_idx - wl.expert_base
    rng = np.random.default_rng(92)
    dout = orc.bf16_round(rng.standard_normal((wl.T, wl.H))).reshape(wl.T, wl.H)
    dv = val(dout)
    I = wl.I

    def loss(xx, gg):
        total = 0.0
        for t in range(wl.T):
            for j in range(wl.k):
                e = idx[t, j]
                if 0 <= e < wl.n_local:
                    h = w_gu[e] @ xx[t]
                    y = w_d[e] @ (h[:I] / (1.0 + np.exp(-h[:I])) * h[I:])
                    total += gg[t, j] * float(dv[t] @ y)
        return total

    ref = orc.backward(wl, dout)
    local = (idx >= 0) & (idx < wl.n_local)
    written = local.any(1)
    assert np.array_equal(ref["written"], written) and 0 < written.sum() < wl.T
    eps = 1e-6
    # dx: every element of a few tokens with 0, 1 and several local picks
    for t in [int(np.argmin(local.sum(1))), int(np.argmax(local.sum(1)))] + \
            [int(v) for v in np.nonzero(local.sum(1) == 1)[0][:2]]:
        for h in range(wl.H):
            xp, xm = x.copy(), x.copy()
            xp[t, h] += eps
            xm[t, h] -= eps
            fd = (loss(xp, gates) - loss(xm, gates)) / (2 * eps)
            assert abs(ref["dx"][t, h] - fd) <= 1e-6 * (1.0 + abs(fd)), (t, h)
    # dgate of every local pick; the oracle's uses the stored bf16 y, so the bar
    # is the rounding of y: 2^-8 sum_h |dout y|
    for t, j in zip(*np.nonzero(local)):
        gp, gm = gates.copy(), gates.copy()
        gp[t, j] += eps
        gm[t, j] -= eps
        fd = (loss(x, gp) - loss(x, gm)) / (2 * eps)
        e = idx[t, j]
        h = w_gu[e] @ x[t]
        mag = float(np.abs(dv[t]) @ np.abs(w_d[e] @ (h[:I] / (1.0 + np.exp(-h[:I])) * h[I:])))
        assert abs(ref["dgate"][t, j] - fd) <= 2.0 ** -8 * mag + 1e-9, (t, j)
    assert np.all(np.isnan(ref["dgate"][~local]))
    # dy = w dout of each slot's own pick
    aos = orc.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)["assign_of_slot"]
    assert np.array_equal(ref["dy"], gates.reshape(-1)[aos][:, None] * dv[aos // wl.k])


# ---------------------------------------------------------------- MXFP8 backward
def _e4m3_table():
    """Non-negative finite OCP E4M3FN values by code 0..126 (0x7f is NaN),
    from the format's fields: 4 exponent bits (bias 7), 3 mantissa bits,
    subnormals at exponent field 0."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


def _mx_brute(v):
    """MXFP8 of rows [n, K] along K by exhaustive search: per block of 32 the
    E8M0 scale 2^E with E = floor(log2 amax) - 8 (the exponent of E4M3's
    largest power of two, 2^8), clipped to [-127, 127] (-127 for an all-zero
    block); each value v / 2^E saturated at 448 and rounded to the nearest
    code value, ties to the even code; the sign kept, also for zero."""
    tab = _e4m3_table()
    v = np.asarray(v, np.float64)
    n, K = v.shape
    codes = np.zeros((n, K), np.uint8)
    scales = np.zeros((n, K // 32), np.uint8)
    for i in range(n):
        for b in range(K // 32):
            blk = v[i, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            E = -127 if amax == 0 else int(np.clip(np.frexp(amax)[1] - 1 - 8, -127, 127))
            scales[i, b] = E + 127
            for j, x in enumerate(blk):
                d = np.abs(tab - min(abs(x) / 2.0 ** E, 448.0))
                best = np.nonzero(d == d.min())[0]
                c = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
                codes[i, 32 * b + j] = c | (0x80 if np.signbit(x) else 0)
    return codes, scales


def _mx_vals(codes, scales):
    tab = _e4m3_table()
    mag = tab[codes & 0x7f] * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    return np.where(codes & 0x80, -mag, mag)


def _mx_case(orc, seed=31, wfmt=0):
    import workloads as W
    wl = W.small_pool(seed, n_partitions=2, part_rows=20, H=64, I=32, E=8, k=3, expert_base=1,
                      counts=[17, 0, 9, 6], act_format=W.ACT_MXFP8)
    val = lambda b: orc.bf16_value(b).astype(np.float64)
    wl.w_gu = orc.bf16_round(val(wl.w_gu) * 20.0).reshape(wl.w_gu.shape)  # O(1) activations
    wl.w_d = orc.bf16_round(val(wl.w_d) * 20.0).reshape(wl.w_d.shape)
    wl.weight_format = wfmt
    rng = np.random.default_rng(seed + 1)
    dout = orc.bf16_round(rng.standard_normal((wl.T, wl.H))).reshape(wl.T, wl.H)
    return wl, dout


@pytest.mark.parametrize("wfmt", [0, 1])
def test_mx_backward_storage_points(orc, wfmt):
    """Every MXFP8 buffer of oracle.backward_mx against a brute-force search
    written from the E4M3 and E8M0 definitions (the quantisation axis and
    block alignment, the scale rule, ties, saturation), each from the inputs
    the path stores: dy from the fp32 w dout; h bf16 of W_gu x_q with x_q the
    ring's values; dh from the stored h and dy_q through the SwiGLU backward
    pinned above by finite differences; dx_s, dx and the weight gradients from
    the quantised operands.  wfmt = 1: MXFP8 weights, each GEMM's along its own
    contraction dimension (W_gu along H for h, W_d along H for da, W_gu along
    2I for dx_s), by the same search."""
    import bars
    wl, dout = _mx_case(orc, wfmt=wfmt)
    r = orc.backward_mx(wl, dout)
    R, I, H = r["R"], wl.I, wl.H
    eos, t_of = r["expert_of_slot"], r["token_of_slot"]
    aos = orc.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)["assign_of_slot"][:R]
    # the ring: MXFP8 of the gathered bf16 rows along H
    xc, xs = _mx_brute(orc.bf16_value(wl.x).astype(np.float64)[t_of])
    assert np.array_equal(xc, r["x_codes"]) and np.array_equal(xs, r["x_scales"])
    xq = _mx_vals(xc, xs)
    # dy = MXFP8 of the fp32 product w * dout along H
    w32 = wl.topk_gate.astype(np.float32).reshape(-1)[aos]
    prod = (w32[:, None] * orc.bf16_value(dout)[t_of]).astype(np.float64)
    dyc, dys = _mx_brute(prod)
    assert np.array_equal(dyc, r["dy_codes"]) and np.array_equal(dys, r["dy_scales"])
    dyq = _mx_vals(dyc, dys)
    wgu, wd = orc.bf16_value(wl.w_gu).astype(np.float64), orc.bf16_value(wl.w_d).astype(np.float64)
    wgu_h, wd_da, wgu_dx = wgu, wd, wgu
    if wfmt:
        q_rows = lambda w: _mx_vals(*_mx_brute(w.reshape(-1, w.shape[-1]))).reshape(w.shape)
        wgu_h = q_rows(wgu)                                           # along H
        wd_da = np.swapaxes(q_rows(np.swapaxes(wd, 1, 2)), 1, 2)      # along H (columns)
        wgu_dx = np.swapaxes(q_rows(np.swapaxes(wgu, 1, 2)), 1, 2)    # along 2I (columns)
    hv = np.zeros((R, 2 * I))
    dh = np.zeros((R, 2 * I))
    for e in np.unique(eos):
        rr = np.nonzero(eos == e)[0]
        hv[rr] = bars.bf16_rne(xq[rr] @ wgu_h[e].T)
    assert np.array_equal(hv, orc.bf16_value(r["h"]).astype(np.float64))
    for e in np.unique(eos):
        rr = np.nonzero(eos == e)[0]
        dh[rr] = orc.swiglu_backward_values(hv[rr], dyq[rr] @ wd_da[e])
    dhc, dhs = _mx_brute(dh)
    assert np.array_equal(dhc, r["dh_codes"]) and np.array_equal(dhs, r["dh_scales"])
    dhq = _mx_vals(dhc, dhs)
    dxs = np.zeros((R, H))
    for e in np.unique(eos):
        rr = np.nonzero(eos == e)[0]
        dxs[rr] = bars.bf16_rne(dhq[rr] @ wgu_dx[e])
    assert np.array_equal(dxs, orc.bf16_value(r["dx_slots"]))
    dx = np.zeros((wl.T, H))
    np.add.at(dx, t_of, dxs)
    assert np.array_equal(bars.bf16_rne(dx), orc.bf16_value(r["dx"]))
    ac, asc = _mx_brute(r["a_exact"])
    aq = _mx_vals(ac, asc)
    for e in range(wl.n_local):
        rr = np.nonzero(eos == e)[0]
        assert np.array_equal(bars.bf16_rne(dyq[rr].T @ aq[rr]), orc.bf16_value(r["dw_d"][e]))
        assert np.array_equal(bars.bf16_rne(dhq[rr].T @ xq[rr]), orc.bf16_value(r["dw_gu"][e]))
    # the cases the search covers are really present: several scales, ties
    # of neither kind missing from dh, negative zeros in dy
    assert len(np.unique(dhs)) > 4 and len(np.unique(dys)) > 4


def test_mx_backward_near_the_unquantised_chain(orc):
    """The MXFP8 chain stays within the size of its quantisation errors of
    the unquantised fp64 chain (ffn_backward_values / ffn_wgrad_values, pinned
    by finite differences, on the same x_q and the exact dy = w dout): each
    E4M3 rounding moves a value by at most 2^-4 of it, so the RMS difference
    is a few per cent -- and it is not zero (the quantisation is applied),
    while a transposed weight or a dropped SiLU' term moves dx by tens of per
    cent."""
    wl, dout = _mx_case(orc, seed=43)
    r = orc.backward_mx(wl, dout)
    R, H = r["R"], wl.H
    eos, t_of = r["expert_of_slot"], r["token_of_slot"]
    aos = orc.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)["assign_of_slot"][:R]
    xq = orc.mx_values(r["x_codes"], r["x_scales"])
    wgu, wd = orc.bf16_value(wl.w_gu).astype(np.float64), orc.bf16_value(wl.w_d).astype(np.float64)
    dy = wl.topk_gate.astype(np.float64).reshape(-1)[aos][:, None] * \
        orc.bf16_value(dout).astype(np.float64)[t_of]
    dh, dxs = orc.ffn_backward_values(xq, eos, wgu, wd, dy)
    dx = np.zeros((wl.T, H))
    np.add.at(dx, t_of, dxs)
    dw_gu, dw_d = orc.ffn_wgrad_values(xq, eos, wgu, dy, dh, wl.n_local, H)
    rel = lambda got, ref: float(np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2)))
    wr = r["written"]
    for name, got, ref in (("dx", orc.bf16_value(r["dx"])[wr], dx[wr]),
                           ("dw_d", orc.bf16_value(r["dw_d"]), dw_d),
                           ("dw_gu", orc.bf16_value(r["dw_gu"]), dw_gu),
                           ("dh", orc.mx_values(r["dh_codes"], r["dh_scales"]), dh)):
        d = rel(got.astype(np.float64), ref)
        assert 1e-3 < d < 0.06, (name, d)
