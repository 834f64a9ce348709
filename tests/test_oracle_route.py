"""Pins for the oracle's top-k route (tahou.com MoK article, routing paragraph).

The pages give no k, tie rule or gate form; the reading pinned here: the k
largest logits per token, equal logits resolved to the lower expert id,
picks ordered by descending logit, gates = softmax over the k picks.
Pins: brute force by a full lexicographic sort, k = 1 against np.argmax,
the closed forms of the gates (renormalised full softmax, k = 1 gives 1).
"""
import numpy as np
import pytest


def _brute_topk(logits, k):
    T, E = logits.shape
    out = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("E", [2, 3, 5, 8, 384])
@pytest.mark.parametrize("alphabet", [None, 2, 3])
def test_topk_matches_brute_force(orc, E, alphabet):
    rng = np.random.default_rng(E * 10 + (alphabet or 0))
    T = 64
    if alphabet is None:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    else:
        logits = rng.integers(0, alphabet, (T, E)).astype(np.float32)
    for k in sorted({1, 2, min(E, 3), min(E, 8), E if E <= 8 else 8}):
        idx, _ = orc.route_topk(logits, k)
        assert np.array_equal(idx, _brute_topk(logits, k)), (E, k)


def test_k1_is_argmax_first_occurrence(orc):
    rng = np.random.default_rng(7)
    logits = rng.integers(-2, 3, (500, 16)).astype(np.float32)
    idx, gate = orc.route_topk(logits, 1)
    assert np.array_equal(idx[:, 0], np.argmax(logits, axis=1))
    assert np.all(gate == 1.0)


def test_signed_zero_ties_go_to_lower_id(orc):
    logits = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    idx, _ = orc.route_topk(logits, 2)
    assert idx.tolist() == [[0, 1], [0, 1]]


@pytest.mark.parametrize("E,k", [(8, 2), (384, 8), (16, 16)])
def test_gates_are_renormalised_softmax(orc, E, k):
    rng = np.random.default_rng(E + k)
    logits = (rng.standard_normal((200, E)) * 3).astype(np.float32)
    idx, gate = orc.route_topk(logits, k)
    l64 = logits.astype(np.float64)
    full = np.exp(l64 - l64.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    picked = np.take_along_axis(full, idx.astype(np.int64), 1)
    ref = picked / picked.sum(1, keepdims=True)
    # each gate is the fp64 value rounded once to fp32
    assert np.all(np.abs(gate - ref) <= 2.0 ** -24 * np.maximum(ref, 2.0 ** -126) * 1.01)
    assert np.all(np.abs(gate.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)
    assert np.all(np.diff(gate, axis=1) <= 0)
    # selected logits are non-increasing along j
    assert np.all(np.diff(np.take_along_axis(logits, idx.astype(np.int64), 1), axis=1) <= 0)


def test_rejects_k_above_e(orc):
    with pytest.raises(ValueError):
        orc.route_topk(np.zeros((2, 3), np.float32), 4)


def test_router_logits_against_exact_sums(orc):
    """router_logits (x . w_router^T over bf16 values) against exactly rounded
    sums of the products, term by term in pure Python, on a shape with
    T != E != H so a transposed or swapped operand cannot pass."""
    import math
    rng = np.random.default_rng(11)
    T, E, H = 3, 5, 7
    x = orc.bf16_round(rng.standard_normal((T, H))).reshape(T, H)
    w = orc.bf16_round(rng.standard_normal((E, H)) * 0.3).reshape(E, H)
    got = orc.router_logits(x, w)
    assert got.shape == (T, E)
    xv, wv = orc.bf16_value(x).astype(float), orc.bf16_value(w).astype(float)
    for t in range(T):
        for e in range(E):
            exact = math.fsum(float(xv[t, h]) * float(wv[e, h]) for h in range(H))
            assert abs(got[t, e] - exact) <= 1e-15 * (1.0 + abs(exact)), (t, e)


def test_router_logits_small_integers_exact(orc):
    """Integer-valued bf16 inputs give integer logits, exactly: the case the
    device's fp32 sums also get exactly (used by the GPU tie test)."""
    rng = np.random.default_rng(12)
    x = orc.bf16_round(rng.integers(-2, 3, (4, 64)).astype(np.float64)).reshape(4, 64)
    w = orc.bf16_round(rng.integers(-2, 3, (6, 64)).astype(np.float64)).reshape(6, 64)
    got = orc.router_logits(x, w)
    ref = np.zeros((4, 6), np.int64)
    xi = orc.bf16_value(x).astype(np.int64)
    wi = orc.bf16_value(w).astype(np.int64)
    for t in range(4):
        for e in range(6):
            ref[t, e] = sum(int(xi[t, h]) * int(wi[e, h]) for h in range(64))
    assert np.array_equal(got, ref.astype(np.float64))
