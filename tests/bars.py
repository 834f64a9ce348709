"""Parity bars for the layer's floating-point results, derived from where the
kernels round (numpy only: no GPU, no torch).

Forward (bf16 activations and weights).  Every stored value is a bf16
rounding (round to nearest even) of a sum the device forms in fp32 and the
oracle in fp64.  The two roundings agree unless the oracle's exact value lies
within the device's error of a rounding boundary; there either neighbour is a
correct result.  So instead of a tolerance, each element gets the interval of
bf16 values the device may legitimately store, built from the oracle's fp64
values before rounding:

  a = SiLU(g) u: the device's g, u carry fp32 accumulation error.  Each
      MFMA instruction adds a 16-product slice of K to the fp32 accumulator,
      so a K-term sum takes K/16 roundings of the running sum S, modelled as
      independent and uniform within +-2^-24 |S| (the RMS of S over the sum
      is estimated from prefix sums at block boundaries):
      sigma = 2^-24 sqrt(K/16/3) RMS(S).  (tests/test_bars_host.py checks
      that the bands also hold an fp32 evaluation that rounds after every
      product.)  The band on a is 6 sigma (propagated through SiLU(g) u) plus
      (|g| + 8) 2^-23 |a| for the exp / reciprocal / products of the
      epilogue.  Roundings of a to either side of that band are the
      candidate flips.
  y = W_d a: the device's exact sum differs from the oracle's by
      sum_i W_d[h,i] (a_dev_i - a_orc_i) over the candidate flips: an interval
      [lo, hi], taking each flip or not; plus 6 sigma of its own fp32
      accumulation over I terms (the same model).  Allowed y = bf16 roundings of
      [y_exact + lo - band, y_exact + hi + band].
  out = sum_j w_j y_j (fp32 fma, ascending j): the sum over the allowed y
      intervals (w_j > 0), plus k 2^-24 sum |w y| for the fp32 sums and, when
      the device computes its own gates, their bar 2^-19 w per gate.

MXFP8 activations: the stored a is the MX quantisation (E4M3 codes, one
power-of-two scale per 32); the candidate moves are the neighbouring codes
within the band and, for a block whose largest magnitude lies within the
band of a power of two, the whole block under the neighbouring scale.  MXFP8
weights: the block-scaled FP8 MFMA's own sum error, 2^-12 of the magnitudes
of each 64-product step, joins the fp32 model.

Outside the flagged elements the interval is one value, the oracle's
rounding: bit-exact.  The statistic of the stated bar, max|got - ref| /
RMS(ref), is reported beside it (``band_stats``).

Backward: the device stores dy, h = [g, u], dh, dx_s and dx in bf16 (each a
rounding within 2^-8 of its value, standard deviation at most 2^-8 / sqrt 3
of it) and sums in fp32.  The bars are 6 standard deviations of the
propagated rounding errors, summed as independent terms (root-sum-square),
element by element; dgate gets the interval of <dout, y> over the forward's
allowed y.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24            # unit roundoff of fp32
U16 = 2.0 ** -8             # unit roundoff of bf16 (8 significant bits)
RHO16 = U16 / np.sqrt(3.0)  # std of one bf16 rounding, relative (uniform error)
C_SIGMA = 6.0               # statistical bands: 6 standard deviations


# ------------------------------------------------------------------ bf16
def bf16_values(bits) -> np.ndarray:
    """bf16 bit patterns -> values (float64)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_rne(v) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), as float64; finite
    inputs in the normal and subnormal range."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                          # a = m 2^e, m in [0.5, 1)
    e = np.maximum(e, -125)                     # subnormals: fixed spacing 2^-133
    q = np.ldexp(1.0, e - 8)                    # spacing of bf16 at a
    return np.copysign(np.rint(a / q) * q, v)


def bf16_bits(v) -> np.ndarray:
    """Values already on the bf16 grid (bf16_rne's output) -> bf16 bit patterns."""
    b = np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)
    return b.astype(np.uint16)


# ------------------------------------------------------------------ forward
def _prefix_rms(W: np.ndarray, X: np.ndarray, bs: int) -> tuple:
    """For rows X [n, K] against W [N, K]: RMS over block boundaries of the
    running sums of W[o] * X[r] along K, and the final sums.  -> ([n, N], [n, N])"""
    N, K = W.shape
    n = X.shape[0]
    nb = K // bs
    Wt = np.ascontiguousarray(W.reshape(N, nb, bs).transpose(1, 0, 2), np.float32)
    Xt = np.ascontiguousarray(X.reshape(n, nb, bs).transpose(1, 2, 0), np.float32)
    P = np.matmul(Wt, Xt).astype(np.float64)       # [nb, N, n] block sums
    S = np.cumsum(P, axis=0)
    return np.sqrt(np.mean(S * S, axis=0)).T, S[-1].T


def _block(K: int) -> int:
    """Block length of the prefix sums: at least 16 block boundaries, so that
    the running sum's RMS is seen even where the final sum cancels."""
    for bs in (256, 128, 64, 32, 16, 8, 4, 2):
        if K % bs == 0 and K // bs >= 16:
            return bs
    return 1


def e4m3_rne(v) -> np.ndarray:
    """float64 -> nearest OCP E4M3FN value (ties to even, saturating at
    +-448, subnormal spacing 2^-9), as float64."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    e = np.maximum(e, -5)                       # below 2^-6: fixed spacing 2^-9
    q = np.ldexp(1.0, e - 4)
    return np.copysign(np.minimum(np.rint(a / q) * q, 448.0), v)


def _mx_blocks(a: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Quantise-dequantise rows a [n, I] in blocks of 32 with the block
    exponents exps [n, I/32]: e4m3(a / 2^E) 2^E."""
    n, I = a.shape
    sc = np.ldexp(1.0, np.repeat(exps, 32, axis=1))
    return e4m3_rne(a / sc) * sc


def _mx_exps(a: np.ndarray) -> np.ndarray:
    """OCP MX scale exponent per block of 32: floor(log2 amax) - 8 in
    [-127, 127]; -127 for an all-zero block."""
    amax = np.abs(a).reshape(a.shape[0], -1, 32).max(2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    return np.where(amax > 0, np.clip(e - 1 - 8, -127, 127), -127)


def _mx_moves(center: np.ndarray, lo: np.ndarray, hi: np.ndarray):
    """MX quantisation of rows [n, K] (blocks of 32 along K) whose values the
    device knows only within [lo, hi] around the oracle's center: returns the
    oracle's quantised values q0 and the largest moves up (dp >= 0) and down
    (dm <= 0) the device's quantised values can take from them.  Inside one
    block the codes move with the value; a block whose largest magnitude may
    lie in the neighbouring binade may take the neighbouring scale, and then
    every element of it moves."""
    E = _mx_exps(center)
    q0 = _mx_blocks(center, E)
    moves = [_mx_blocks(hi, E) - q0, _mx_blocks(lo, E) - q0]
    n = center.shape[0]
    amax_hi = np.maximum(np.abs(lo), np.abs(hi)).reshape(n, -1, 32).max(2)
    low_mag = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    amax_lo = low_mag.reshape(n, -1, 32).max(2)
    for dE in (-1, 1):
        E2 = np.clip(E + dE, -127, 127)
        b_lo, b_hi = np.ldexp(1.0, E2 + 8), np.ldexp(1.0, E2 + 9)   # amax range of exponent E2
        reach = (amax_hi >= b_lo) & (amax_lo < b_hi) & (E2 != E)
        if reach.any():
            m = np.repeat(reach, 32, axis=1)
            for v in (center, lo, hi):
                moves.append(np.where(m, _mx_blocks(v, E2) - q0, 0.0))
    st = np.stack(moves)
    return q0, np.maximum(st, 0.0).max(0), np.minimum(st, 0.0).min(0)


def _candidates(ae: np.ndarray, band: np.ndarray, act_mx: bool):
    """The oracle's stored a (a0) and the largest moves up (dp >= 0) and down
    (dm <= 0) a device value within +-band of a_exact can make it take."""
    if not act_mx:
        a0 = bf16_rne(ae)
        return a0, bf16_rne(ae + band) - a0, bf16_rne(ae - band) - a0
    return _mx_moves(ae, ae - band, ae + band)


# Sum error of one step of gfx950's block-scaled FP8 MFMA (64 products of E4M3
# codes with their block scales, added to an fp32 accumulator), relative to the
# sum of the magnitudes of the step's products: a GPU probe over random codes
# and scales measured about 2e-4 of the exact 64-term sum; 2^-12 of the
# magnitudes bounds that with room to spare.
MX_MFMA_REL = 2.0 ** -12


def ffn_y_band(x_vals: np.ndarray, expert_of_row, w_gu_vals: np.ndarray, w_d_vals: np.ndarray,
               a_exact: np.ndarray, y_exact: np.ndarray, act_mx: bool = False,
               w_mx: bool = False, return_a: bool = False):
    """Allowed bf16 values of y per element for dispatched rows (values
    [n, H], as the GEMM reads them) of experts expert_of_row, given the
    oracle's fp64 a and y before their rounding (or MX quantisation of a when
    act_mx).  Weights as values ([n_local, 2I, H], [n_local, H, I]); w_mx:
    MXFP8 weights, multiplied by the block-scaled FP8 MFMA.  Returns (y_lo,
    y_hi) as float64 values [n, H] and the number of activation elements whose
    stored value may move; with return_a also (a0, dp, dm) [n, I]: the
    oracle's stored a and the largest moves of the device's from it."""
    x = np.asarray(x_vals, np.float64)
    eor = np.asarray(expert_of_row, np.int64).reshape(-1)
    n, H = x.shape
    I = a_exact.shape[1]
    y_lo = np.empty((n, H))
    y_hi = np.empty((n, H))
    a_all = np.zeros((3, n, I))
    n_aflag = 0

    def acc_sigma(W, X, K):
        """std of the device's sum error per output (rows X against W [N, K])"""
        rms, fin = _prefix_rms(W, X, _block(K))
        var = (U32 * rms) ** 2 * (K / 16) / 3.0
        if w_mx:
            step = np.abs(W).reshape(W.shape[0], K // 64, 64)
            # sum over steps of (rel * A_s)^2, A_s = sum of |products| of step s
            A = np.einsum("okj,nkj->nok", step, np.abs(X).reshape(X.shape[0], K // 64, 64),
                          optimize=True)
            var = var + (MX_MFMA_REL ** 2 / 3.0) * np.sum(A * A, axis=2)
        return np.sqrt(var), fin

    for e in np.unique(eor):
        r = np.nonzero(eor == e)[0]
        wgu = np.asarray(w_gu_vals[e], np.float32)                    # [2I, H]
        sig, gu = acc_sigma(wgu, x[r], H)                             # [n_e, 2I]
        g, u = gu[:, :I], gu[:, I:]
        sg, su = sig[:, :I], sig[:, I:]
        s = 1.0 / (1.0 + np.exp(-g))
        silu, dsilu = g * s, s * (1.0 + g * (1.0 - s))
        ae = a_exact[r]
        band_a = (C_SIGMA * np.sqrt((dsilu * u * sg) ** 2 + (silu * su) ** 2) +
                  (np.abs(g) + 8.0) * 2.0 ** -23 * np.abs(ae) + 1e-38)
        a0, dp, dm = _candidates(ae, band_a, act_mx)
        a_all[0, r], a_all[1, r], a_all[2, r] = a0, dp, dm
        n_aflag += int(np.count_nonzero(dp) + np.count_nonzero(dm))
        wd = np.asarray(w_d_vals[e], np.float64)                      # [H, I]
        wp, wm = np.maximum(wd, 0.0), np.minimum(wd, 0.0)
        lo = dm @ wp.T + dp @ wm.T
        hi = dp @ wp.T + dm @ wm.T
        sig_y, _ = acc_sigma(wd.astype(np.float32), a0, I)
        band_y = C_SIGMA * sig_y + 1e-38
        ye = y_exact[r]
        y_lo[r] = bf16_rne(ye + lo - band_y)
        y_hi[r] = bf16_rne(ye + hi + band_y)
    if return_a:
        return y_lo, y_hi, n_aflag, (a_all[0], a_all[1], a_all[2])
    return y_lo, y_hi, n_aflag


def out_band(y_lo: np.ndarray, y_hi: np.ndarray, row_of_slot: np.ndarray,
             slot_of_assign: np.ndarray, gates: np.ndarray, tokens, k: int,
             gate_rel: float = 0.0):
    """Allowed bf16 values of the merged rows of `tokens` (ascending j over
    their local slots, fp32 fma from 0) when slot s's y may be any value in
    [y_lo, y_hi][row_of_slot[s]].  gate_rel: relative bar of the device's
    gates against the oracle's (0 when both use the same gates)."""
    tokens = np.asarray(tokens, np.int64)
    soa = np.asarray(slot_of_assign).reshape(-1, k)[tokens]
    w = np.asarray(gates, np.float64).reshape(-1, k)[tokens]
    n, H = tokens.size, y_lo.shape[1]
    lo = np.zeros((n, H))
    hi = np.zeros((n, H))
    mag = np.zeros((n, H))
    for j in range(k):
        s = soa[:, j]
        m = s >= 0
        if not m.any():
            continue
        rr = np.asarray(row_of_slot)[s[m]]
        wl, wh = w[m, j, None] * y_lo[rr], w[m, j, None] * y_hi[rr]
        lo[m] += np.minimum(wl, wh)
        hi[m] += np.maximum(wl, wh)
        mag[m] += np.maximum(np.abs(wl), np.abs(wh))
    err = (k * U32 + gate_rel) * mag
    return bf16_rne(lo - err), bf16_rne(hi + err)


def band_stats(got_bits, ref_bits, lo, hi, tol: float, what: str) -> dict:
    """Asserts lo <= got <= hi element by element (bit-exact where lo == hi)
    and that the oracle's own rounding lies in its band; returns the stated
    bar's statistic max|got - ref| / RMS(ref) and counts: elements, flagged
    (band wider than one value), differing from the oracle, above
    tol * RMS(ref) (each of them inside its band)."""
    g, r = bf16_values(got_bits), bf16_values(ref_bits)
    lo, hi = np.asarray(lo), np.asarray(hi)
    assert g.shape == r.shape == lo.shape, (what, g.shape, r.shape, lo.shape)
    assert np.all((r >= lo) & (r <= hi)), f"{what}: the oracle's rounding is outside its own band"
    fin = np.isfinite(g)
    assert fin.all(), f"{what}: {int((~fin).sum())} non-finite values"
    bad = (g < lo) | (g > hi)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    d = np.abs(g - r)
    if bad.any():
        i = np.argmax(np.where(bad, d, -1.0))
        idx = np.unravel_index(i, g.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {g.size} elements outside their rounding band; e.g. "
            f"at {tuple(int(v) for v in idx)} got {g[idx]!r}, oracle {r[idx]!r}, band "
            f"[{lo[idx]!r}, {hi[idx]!r}]")
    st = dict(what=what, n=int(g.size), flagged=int(np.count_nonzero(lo != hi)),
              differ=int(np.count_nonzero(g != r)),
              strict=float(d.max() / rms) if rms > 0 and d.size else 0.0,
              over_strict=int(np.count_nonzero(d > tol * rms)), tol=tol)
    print(f"[parity] {what}: max|d|/RMS = {st['strict']:.3e} (bar {tol:g}); {st['differ']} of "
          f"{st['n']} elements differ from the oracle, {st['flagged']} in a tie band, "
          f"{st['over_strict']} above the bar (each a tie-band neighbour)", flush=True)
    return st


def strict_stats(got_bits, ref_bits, tol: float, what: str, check: bool = True) -> float:
    """max|got - ref| <= tol * RMS(ref) over every element (the stated bar,
    no allowance; check=False only prints it); returns max|got - ref| / RMS(ref)."""
    g, r = bf16_values(got_bits), bf16_values(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    if g.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    d = np.abs(g - r)
    rel = float(d.max()) / rms if rms > 0 else 0.0
    print(f"[parity] {what}: max|d|/RMS = {rel:.3e} (bar {tol:g}, no allowance"
          f"{'' if check else ', reported'})", flush=True)
    assert rel <= tol or not check, f"{what}: max|d|/RMS = {rel:.4g} > {tol}"
    return rel


def layer_values(wl, x_rows):
    """What the device's GEMMs multiply, as values: the dispatched rows (bf16
    bits, or MXFP8 (codes, scales)) and the weights (bf16, or their MXFP8
    quantisation per row when the workload has MXFP8 weights)."""
    import oracle
    if wl.act_format == 1:
        codes, scales = x_rows
        n, H = codes.shape
        xv = oracle.mx_dequantize(codes.reshape(-1), scales.reshape(-1)).reshape(n, H)
    else:
        xv = bf16_values(x_rows)
    if getattr(wl, "weight_format", 0) == 1:
        deq = lambda w: oracle.mx_dequantize(*(q.reshape(-1) for q in oracle.mx_quantize_rows(w))) \
            .reshape(w.shape)
        return xv, deq(wl.w_gu), deq(wl.w_d)
    return xv, bf16_values(wl.w_gu), bf16_values(wl.w_d)


def layer_y_band(wl, x_rows, expert_of_row, a_exact, y_exact):
    """ffn_y_band for a workload's formats."""
    xv, wgu, wd = layer_values(wl, x_rows)
    return ffn_y_band(xv, expert_of_row, wgu, wd, a_exact, y_exact, act_mx=wl.act_format == 1,
                      w_mx=getattr(wl, "weight_format", 0) == 1)


def forward_band(wl, r: dict, gate_rel: float = 0.0):
    """Bands of the oracle's forward result r (oracle.forward, with its exact
    values): (y_lo, y_hi) per computed slot (rows of r['y']) and (out_lo,
    out_hi) per listed token."""
    y_lo, y_hi, _ = layer_y_band(wl, r["x_rows"], r["expert_of_slot"], r["a_exact"],
                                 r["y_exact"])
    row_of_slot = np.full(max(int(r["R"]), 1), -1, np.int64)
    row_of_slot[r["slots"]] = np.arange(r["slots"].size)
    o_lo, o_hi = out_band(y_lo, y_hi, row_of_slot, r["slot_of_assign"], r["topk_gate"],
                          r["tokens"], wl.k, gate_rel)
    return y_lo, y_hi, o_lo, o_hi


# ------------------------------------------------------------------ backward
def dgate_band(dout_vals: np.ndarray, y_lo: np.ndarray, y_hi: np.ndarray):
    """Interval of <dout, y> (fp32 sums over H) when y may be any value of
    [y_lo, y_hi]; rows aligned.  -> (lo, hi) per row."""
    a, b = dout_vals * y_lo, dout_vals * y_hi
    lo, hi = np.minimum(a, b).sum(1), np.maximum(a, b).sum(1)
    err = dout_vals.shape[1] * U32 * np.maximum(np.abs(a), np.abs(b)).sum(1)
    return lo - err, hi + err


def ffn_backward_sigma(x_vals, expert_of_row, w_gu_vals, w_d_vals, dy, h, dh):
    """Standard deviation of the device's dh and dx_s per element (rows of
    the oracle's fp64 values: dy, h = [g, u], dh) from the bf16 roundings of
    dy, g, u, dh and dx_s, propagated to first order, independent terms.
    Returns (sigma_dh [n, 2I], sigma_dxs [n, H])."""
    eor = np.asarray(expert_of_row, np.int64).reshape(-1)
    n, H = x_vals.shape
    I = h.shape[1] // 2
    s_dh = np.zeros((n, 2 * I))
    s_dx = np.zeros((n, H))
    for e in np.unique(eor):
        r = np.nonzero(eor == e)[0]
        wd, wgu = w_d_vals[e], w_gu_vals[e]
        g, u = h[r, :I], h[r, I:]
        s = 1.0 / (1.0 + np.exp(-g))
        silu, d1 = g * s, s * (1.0 + g * (1.0 - s))
        d2 = s * (1.0 - s) * (2.0 + g * (1.0 - 2.0 * s))
        da = dy[r] @ wd                                           # [n_e, I]
        s_da = np.sqrt((RHO16 * dy[r]) ** 2 @ (wd * wd))          # from the dy roundings
        sg, su = RHO16 * np.abs(g), RHO16 * np.abs(u)
        dg, du = dh[r, :I], dh[r, I:]
        v_dg = (u * d1 * s_da) ** 2 + (da * d1 * su) ** 2 + (da * u * d2 * sg) ** 2 + (RHO16 * dg) ** 2
        v_du = (silu * s_da) ** 2 + (da * d1 * sg) ** 2 + (RHO16 * du) ** 2
        s_dh[r] = np.sqrt(np.concatenate([v_dg, v_du], 1))
        dxs = dh[r] @ wgu
        s_dx[r] = np.sqrt(s_dh[r] ** 2 @ (wgu * wgu) + (RHO16 * dxs) ** 2)
    return s_dh, s_dx


def dx_bar(sigma_dxs: np.ndarray, token_of_row: np.ndarray, dx_ref: np.ndarray):
    """Bar of the device's dx per token (sum of its slots' dx_s in fp32, then
    bf16): 6 sigma of the slots' errors and the final rounding."""
    var = np.zeros_like(dx_ref)
    np.add.at(var, np.asarray(token_of_row, np.int64), sigma_dxs ** 2)
    return C_SIGMA * np.sqrt(var + (RHO16 * dx_ref) ** 2) + 1e-30


def wgrad_bars(expert_of_row, n_local: int, x_vals, a_vals, dy, dh, s_dh, dw_d, dw_gu):
    """Bars of the weight gradients dW_d[e] = sum_s dy a^T (device: bf16 dy and
    bf16 act) and dW_gu[e] = sum_s dh x^T (device: bf16 dh, exact x), 6 sigma
    of the operands' roundings summed over the expert's slots plus the
    result's own rounding.  a_vals: the oracle's fp64 a."""
    eor = np.asarray(expert_of_row, np.int64).reshape(-1)
    bd = np.zeros_like(dw_d)
    bg = np.zeros_like(dw_gu)
    for e in range(n_local):
        r = np.nonzero(eor == e)[0]
        v_d = (RHO16 * dy[r]).T ** 2 @ a_vals[r] ** 2 + (dy[r] ** 2).T @ (RHO16 * a_vals[r]) ** 2 \
            if r.size else 0.0
        v_g = (s_dh[r] ** 2).T @ (x_vals[r] ** 2) if r.size else 0.0
        bd[e] = C_SIGMA * np.sqrt(v_d + (RHO16 * dw_d[e]) ** 2) + 1e-30
        bg[e] = C_SIGMA * np.sqrt(v_g + (RHO16 * dw_gu[e]) ** 2) + 1e-30
    return bd, bg


# ------------------------------------------------------------------ MXFP8 backward
def _acc_sigma_padded(W: np.ndarray, X: np.ndarray, w_mx: bool = False) -> np.ndarray:
    """std of the device's fp32 sum error of X [n, K] against W [N, K] (the
    K/16-roundings model of the forward), for any K: the sums are zero-padded
    to a multiple of 16 block boundaries.  w_mx: the block-scaled FP8 MFMA's
    own error too, MX_MFMA_REL of each 64-product step's magnitudes (K a
    multiple of 64)."""
    N, K = W.shape
    n = X.shape[0]
    if K == 0:
        return np.zeros((n, N))
    bs = max(1, -(-K // 16))
    Kp = bs * 16
    Wp = np.zeros((N, Kp), np.float32)
    Xp = np.zeros((n, Kp), np.float32)
    Wp[:, :K], Xp[:, :K] = W, X
    rms, _ = _prefix_rms(Wp, Xp, bs)
    var = (U32 * rms) ** 2 * max(K / 16.0, 1.0) / 3.0
    if w_mx:
        A = np.einsum("okj,nkj->nok", np.abs(W).reshape(N, K // 64, 64),
                      np.abs(X).reshape(n, K // 64, 64), optimize=True)
        var = var + (MX_MFMA_REL ** 2 / 3.0) * np.sum(A * A, axis=2)
    return np.sqrt(var)


def swiglu_bwd_values(g, u, da):
    """[da u SiLU'(g), da SiLU(g)] (numpy, any float type)."""
    s = 1.0 / (1.0 + np.exp(-g))
    return np.concatenate([da * u * s * (1.0 + g * (1.0 - s)), da * g * s], axis=1)


def mx_backward_bands(wl, r: dict, dout_bits) -> dict:
    """Bands of the MXFP8 backward for the oracle's result r
    (oracle.backward_mx), built like the forward's: from where the device
    rounds and what it decides.
      dy      the device takes the same decisions on the same fp32 products:
              bit-exact (no band).
      dgate   the interval of <dout, y> over the forward's y bands.
      h       bf16 roundings within 6 sigma of the fp32 sum over H.
      dh      the device's value before quantisation lies within the SwiGLU
              backward evaluated at the corners of its inputs' bands (h, and
              da within 6 sigma of its fp32 sum over H) plus the epilogue's
              fp32 arithmetic; the band is the quantisations of that interval
              (neighbouring codes, and the neighbouring scale for a block whose
              amax may cross a power of two).
      dx_s    the oracle's sum over the dh_q moves (interval per weight sign)
              plus 6 sigma of the fp32 sum over 2I, rounded to bf16.
      dx      the fp32 sum of the slots' dx_s bands, rounded to bf16.
      dW_d    sum_s dy_q a^T over the forward's a moves; dW_gu: sum_s dh x_q^T
              over the dh moves; each plus 6 sigma of its fp32 sum over the
              expert's slots, rounded to bf16.
    Returns a dict of (lo, hi) pairs of values ('a' and 'dh' as intervals of
    the device's dequantised values, 'a_q0' and 'dh_q0' the oracle's), plus
    'dh_flagged'."""
    import oracle
    I, H = wl.I, wl.H
    eos, t_of, R = r["expert_of_slot"], r["token_of_slot"], r["R"]
    w_mx = getattr(wl, "weight_format", 0) == 1
    xq, wgu_f, wd_f = layer_values(wl, (r["x_codes"], r["x_scales"]))   # the forward's weights
    wgu, wd, wgu_dx = r["w_gu_h"], r["w_d_da"], r["w_gu_dx"]            # h, da, dx_s
    y_lo, y_hi, _, (a0, a_dp, a_dm) = ffn_y_band(xq, eos, wgu_f, wd_f, r["a_exact"], r["y_exact"],
                                                 act_mx=True, w_mx=w_mx, return_a=True)
    out = {"y": (y_lo, y_hi), "a": (a0 + a_dm, a0 + a_dp), "a_q0": a0}
    out["dgate"] = dgate_band(bf16_values(dout_bits)[t_of], y_lo, y_hi)
    dyq = oracle.mx_values(r["dy_codes"], r["dy_scales"])
    h_ex = r["h_exact"]
    h_lo, h_hi = np.empty_like(h_ex), np.empty_like(h_ex)
    d_lo, d_hi = np.empty((R, 2 * I)), np.empty((R, 2 * I))
    for e in np.unique(eos):
        rr = np.nonzero(eos == e)[0]
        sig_h = _acc_sigma_padded(np.asarray(wgu[e], np.float32), xq[rr], w_mx)
        h_lo[rr] = bf16_rne(h_ex[rr] - C_SIGMA * sig_h)
        h_hi[rr] = bf16_rne(h_ex[rr] + C_SIGMA * sig_h)
        da = dyq[rr] @ wd[e]
        sig_da = _acc_sigma_padded(np.asarray(wd[e].T, np.float32), dyq[rr], w_mx)
        corners = []
        for g in (h_lo[rr, :I], h_hi[rr, :I]):
            for u in (h_lo[rr, I:], h_hi[rr, I:]):
                for dd in (da - C_SIGMA * sig_da, da + C_SIGMA * sig_da):
                    corners.append(swiglu_bwd_values(g, u, dd))
        st = np.stack(corners)
        g_abs = np.concatenate([np.abs(h_ex[rr, :I])] * 2, axis=1)
        err = (g_abs + 8.0) * 2.0 ** -23 * np.abs(st).max(0) + 1e-38
        d_lo[rr], d_hi[rr] = st.min(0) - err, st.max(0) + err
    out["h"] = (h_lo, h_hi)
    q0, dp, dm = _mx_moves(r["dh_exact"], d_lo, d_hi)
    out["dh"] = (q0 + dm, q0 + dp)
    out["dh_q0"] = q0
    out["dh_flagged"] = int(np.count_nonzero(dp) + np.count_nonzero(dm))
    dxs_lo, dxs_hi = np.empty((R, H)), np.empty((R, H))
    for e in np.unique(eos):
        rr = np.nonzero(eos == e)[0]
        W = wgu_dx[e]                                                 # [2I, H]
        wp, wm = np.maximum(W, 0.0), np.minimum(W, 0.0)
        lo = dm[rr] @ wp + dp[rr] @ wm
        hi = dp[rr] @ wp + dm[rr] @ wm
        band = C_SIGMA * _acc_sigma_padded(np.asarray(W.T, np.float32), q0[rr], w_mx) + 1e-38
        ce = r["dx_slots_exact"][rr]
        dxs_lo[rr], dxs_hi[rr] = bf16_rne(ce + lo - band), bf16_rne(ce + hi + band)
    out["dx_slots"] = (dxs_lo, dxs_hi)
    soa = r["slot_of_assign"]
    out["dx"] = out_band(dxs_lo, dxs_hi, np.arange(max(R, 1)), soa,
                         np.ones(soa.size), np.arange(wl.T), wl.k)
    dwd_lo, dwd_hi = np.empty_like(r["dw_d_exact"]), np.empty_like(r["dw_d_exact"])
    dwg_lo, dwg_hi = np.empty_like(r["dw_gu_exact"]), np.empty_like(r["dw_gu_exact"])
    for e in range(wl.n_local):
        rr = np.nonzero(eos == e)[0]
        dy = dyq[rr]                                                   # [n_e, H]
        yp, ym = np.maximum(dy, 0.0), np.minimum(dy, 0.0)
        lo = yp.T @ a_dm[rr] + ym.T @ a_dp[rr]
        hi = yp.T @ a_dp[rr] + ym.T @ a_dm[rr]
        band = C_SIGMA * _acc_sigma_padded(np.asarray(a0[rr].T, np.float32), dy.T) + 1e-38
        ce = r["dw_d_exact"][e]
        dwd_lo[e], dwd_hi[e] = bf16_rne(ce + lo - band), bf16_rne(ce + hi + band)
        x = xq[rr]
        xp_, xm_ = np.maximum(x, 0.0), np.minimum(x, 0.0)
        lo = dm[rr].T @ xp_ + dp[rr].T @ xm_
        hi = dp[rr].T @ xp_ + dm[rr].T @ xm_
        band = C_SIGMA * _acc_sigma_padded(np.asarray(x.T, np.float32), q0[rr].T) + 1e-38
        ce = r["dw_gu_exact"][e]
        dwg_lo[e], dwg_hi[e] = bf16_rne(ce + lo - band), bf16_rne(ce + hi + band)
    out["dw_d"] = (dwd_lo, dwd_hi)
    out["dw_gu"] = (dwg_lo, dwg_hi)
    return out


def interval_stats(got: np.ndarray, ref: np.ndarray, lo: np.ndarray, hi: np.ndarray,
                   what: str) -> dict:
    """lo <= got <= hi for values (not bf16 bits: the MXFP8 dh), the oracle's
    own value inside too; prints how many elements differ from the oracle."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all((ref >= lo) & (ref <= hi)), f"{what}: the oracle's value is outside its own band"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bad = (got < lo) | (got > hi)
    if bad.any():
        i = np.unravel_index(np.argmax(bad), got.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} elements outside their band; "
                             f"e.g. at {tuple(int(v) for v in i)} got {got[i]!r}, oracle {ref[i]!r}, "
                             f"band [{lo[i]!r}, {hi[i]!r}]")
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    st = dict(n=int(got.size), differ=int(np.count_nonzero(got != ref)),
              flagged=int(np.count_nonzero(lo != hi)),
              strict=float(np.abs(got - ref).max() / rms) if rms > 0 else 0.0)
    print(f"[parity] {what}: {st['differ']} of {st['n']} elements differ from the oracle, "
          f"{st['flagged']} in a band, max|d|/RMS = {st['strict']:.3e}", flush=True)
    return st


def mx_stage_bands(wl, r: dict, dh_vals: np.ndarray, act_vals: np.ndarray) -> dict:
    """Bands of the MXFP8 backward's later stages given the device's own stored
    inputs to them (its dh and act values, each checked against its own band
    by mx_backward_bands): dx_s = bf16(dh W_gu) per slot, dW_d[e] = bf16(sum_s
    dy a^T) and dW_gu[e] = bf16(sum_s dh x_q^T), each the interval of its fp32
    sum (6 sigma, with the block-scaled MFMA's error for MXFP8 weights) around
    the exact product of those inputs, rounded to bf16.  With MXFP8 weights the
    error model of that MFMA leaves many dh elements a code away from the
    oracle's, and an interval over all of them would say little about dx_s;
    given the device's dh, what remains is the GEMM's own rounding.  Returns
    (lo, hi, center) per key; dx: pass the device's dx_s to out_band."""
    import oracle
    I, H, R = wl.I, wl.H, r["R"]
    eos = r["expert_of_slot"]
    w_mx = getattr(wl, "weight_format", 0) == 1
    xq = oracle.mx_values(r["x_codes"], r["x_scales"])
    dyq = oracle.mx_values(r["dy_codes"], r["dy_scales"])
    out = {}
    lo, hi, ce = np.empty((R, H)), np.empty((R, H)), np.empty((R, H))
    for e in np.unique(eos):
        rr = np.nonzero(eos == e)[0]
        W = r["w_gu_dx"][e]                                           # [2I, H]
        c = dh_vals[rr] @ W
        band = C_SIGMA * _acc_sigma_padded(np.asarray(W.T, np.float32), dh_vals[rr], w_mx) + 1e-38
        lo[rr], hi[rr], ce[rr] = bf16_rne(c - band), bf16_rne(c + band), bf16_rne(c)
    out["dx_slots"] = (lo, hi, ce)
    n_local = wl.n_local
    shp_d, shp_g = (n_local, H, I), (n_local, 2 * I, H)
    dl, dhh, dc = np.empty(shp_d), np.empty(shp_d), np.empty(shp_d)
    gl, gh, gc = np.empty(shp_g), np.empty(shp_g), np.empty(shp_g)
    for e in range(n_local):
        rr = np.nonzero(eos == e)[0]
        c = dyq[rr].T @ act_vals[rr]
        band = C_SIGMA * _acc_sigma_padded(np.asarray(act_vals[rr].T, np.float32), dyq[rr].T) + 1e-38
        dl[e], dhh[e], dc[e] = bf16_rne(c - band), bf16_rne(c + band), bf16_rne(c)
        c = dh_vals[rr].T @ xq[rr]
        band = C_SIGMA * _acc_sigma_padded(np.asarray(xq[rr].T, np.float32), dh_vals[rr].T) + 1e-38
        gl[e], gh[e], gc[e] = bf16_rne(c - band), bf16_rne(c + band), bf16_rne(c)
    out["dw_d"] = (dl, dhh, dc)
    out["dw_gu"] = (gl, gh, gc)
    return out
