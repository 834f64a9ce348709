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
