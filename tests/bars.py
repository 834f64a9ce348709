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


def _candidates(ae: np.ndarray, band: np.ndarray, act_mx: bool):
    """The oracle's stored a (a0) and the largest moves up (dp >= 0) and down
    (dm <= 0) a device value within +-band of a_exact can make it take."""
    if not act_mx:
        a0 = bf16_rne(ae)
        return a0, bf16_rne(ae + band) - a0, bf16_rne(ae - band) - a0
    E = _mx_exps(ae)
    a0 = _mx_blocks(ae, E)
    moves = [_mx_blocks(ae + band, E) - a0, _mx_blocks(ae - band, E) - a0]
    # a block whose amax lies within the band of a power of two may take the
    # neighbouring scale: every element of it may then move
    n, I = ae.shape
    amax = np.abs(ae).reshape(n, -1, 32).max(2)
    bmax = band.reshape(n, -1, 32).max(2)
    for dE in (-1, 1):
        E2 = np.clip(E + dE, -127, 127)
        lo, hi = np.ldexp(1.0, E2 + 8), np.ldexp(1.0, E2 + 9)   # amax range of exponent E2
        reach = (amax + bmax >= lo) & (amax - bmax < hi) & (E2 != E)
        if reach.any():
            alt = np.where(np.repeat(reach, 32, axis=1), _mx_blocks(ae, E2) - a0, 0.0)
            moves += [alt]
    st = np.stack(moves)
    return a0, np.maximum(st, 0.0).max(0), np.minimum(st, 0.0).min(0)


# Sum error of one step of gfx950's block-scaled FP8 MFMA (64 products of E4M3
# codes with their block scales, added to an fp32 accumulator), relative to the
# sum of the magnitudes of the step's products: a GPU probe over random codes
# and scales measured about 2e-4 of the exact 64-term sum; 2^-12 of the
# magnitudes bounds that with room to spare.
MX_MFMA_REL = 2.0 ** -12


def ffn_y_band(x_vals: np.ndarray, expert_of_row, w_gu_vals: np.ndarray, w_d_vals: np.ndarray,
               a_exact: np.ndarray, y_exact: np.ndarray, act_mx: bool = False,
               w_mx: bool = False):
    """Allowed bf16 values of y per element for dispatched rows (values
    [n, H], as the GEMM reads them) of experts expert_of_row, given the
    oracle's fp64 a and y before their rounding (or MX quantisation of a when
    act_mx).  Weights as values ([n_local, 2I, H], [n_local, H, I]); w_mx:
    MXFP8 weights, multiplied by the block-scaled FP8 MFMA.  Returns (y_lo,
    y_hi) as float64 values [n, H] and the number of activation elements whose
    stored value may move."""
    x = np.asarray(x_vals, np.float64)
    eor = np.asarray(expert_of_row, np.int64).reshape(-1)
    n, H = x.shape
    I = a_exact.shape[1]
    y_lo = np.empty((n, H))
    y_hi = np.empty((n, H))
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


def strict_stats(got_bits, ref_bits, tol: float, what: str) -> float:
    """max|got - ref| <= tol * RMS(ref) over every element (the stated bar,
    no allowance); returns max|got - ref| / RMS(ref)."""
    g, r = bf16_values(got_bits), bf16_values(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    if g.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    d = np.abs(g - r)
    rel = float(d.max()) / rms if rms > 0 else 0.0
    print(f"[parity] {what}: max|d|/RMS = {rel:.3e} (bar {tol:g}, no allowance)", flush=True)
    assert rel <= tol, f"{what}: max|d|/RMS = {rel:.4g} > {tol}"
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
