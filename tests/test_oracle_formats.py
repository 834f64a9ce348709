"""Pins for the oracle's number formats: bf16 rounding, OCP E4M3 and MXFP8.

MXFP8 activations are fused into dispatch and SwiGLU on the pages (tahou.com
MoK article, state-machine paragraph); the format itself is the OCP
Microscaling v1.0 MXFP8 E4M3 one: 32-element blocks, an E8M0 shared scale
2^(floor(log2 amax) - 8), elements rounded to nearest even and saturated at
448.  Pins: torch's bf16 and float8_e4m3fn conversions (library routines),
a brute-force nearest-code search over all 254 finite codes, and a second
scalar MX implementation below that finds the scale by search, not frexp.
"""
import math

import numpy as np
import pytest
import torch


def _all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().double().numpy()
    return codes, vals


def _nearest_code(v, codes, vals):
    """Nearest finite E4M3 value, ties to the even code, saturating at 448."""
    if v == 0.0:
        return 0x80 if math.copysign(1.0, v) < 0 else 0x00
    a = min(abs(v), 448.0)
    pos = codes[(codes & 0x80) == 0]
    pv = vals[(codes & 0x80) == 0]
    d = np.abs(pv - a)
    best = np.nonzero(d == d.min())[0]
    if best.size > 1:
        best = [b for b in best if pos[b] % 2 == 0]
    c = int(pos[best[0]])
    return c | (0x80 if v < 0 else 0)


def test_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_e4m3_encode_brute_force(orc):
    codes, vals = _all_finite_codes()
    pos = np.unique(vals[vals > 0])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    v = np.concatenate([pos, -pos, mids, -mids, [0.0, -0.0, 2.0 ** -11, -2.0 ** -11,
                                                   463.9, 464.0, 470.0, 1e6, -1e6],
                        rng.standard_normal(3000) * 50, rng.standard_normal(1000) * 0.01])
    got = orc.e4m3_encode(v)
    ref = np.array([_nearest_code(x, codes, vals) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 40, rng.uniform(-448, 448, 20000)])
    v = v.astype(np.float32)  # torch converts fp32 -> e4m3 with round-to-nearest-even
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(v.astype(np.float64)), ref)


def test_bf16_round_matches_torch(orc):
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(50000) * np.exp(rng.uniform(-60, 60, 50000))).astype(np.float32)
    # exact ties between neighbouring bf16 values, both parities
    b = rng.integers(0x0080, 0x7F00, 4000, dtype=np.uint32)  # finite patterns only
    ties = ((b << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.float32([0.0, -0.0, 3.0e38, 1e-40])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_round(f.astype(np.float64)), ref)


def _mx_block_by_search(v, codes, vals):
    """Second MXFP8 block quantiser: the scale exponent found by search."""
    amax = max(abs(x) for x in v)
    if amax == 0.0:
        E = -127
    else:
        E = -127
        while E < 127 and 2.0 ** (E + 9) <= amax:   # want 2^(E+8) <= amax < 2^(E+9)
            E += 1
    return [_nearest_code(x / 2.0 ** E, codes, vals) for x in v], E + 127


def test_mx_block_vs_search(orc):
    codes, vals = _all_finite_codes()
    rng = np.random.default_rng(3)
    blocks = [rng.standard_normal(32) * s for s in (1e-3, 0.02, 1.0, 300.0)]
    blocks += [np.zeros(32), -np.zeros(32), np.full(32, 2.0 ** -120),
               np.linspace(-1, 1, 32), np.array([2.0 ** 8] + [1.0] * 31),
               np.array([511.0 / 512 * 2.0 ** 9] + [0.001] * 31)]
    for blk in blocks:
        c, s = orc.mx_quantize(blk)
        rc, rs = _mx_block_by_search(list(blk), codes, vals)
        assert s[0] == rs
        assert c.tolist() == rc


def test_mx_invariants(orc):
    rng = np.random.default_rng(4)
    v = rng.standard_normal(32 * 500) * np.repeat(np.exp(rng.uniform(-20, 20, 500)), 32)
    c, s = orc.mx_quantize(v)
    dq = orc.mx_dequantize(c, s)
    # scale: 2^(floor(log2 amax) - 8) per block
    amax = np.abs(v.reshape(-1, 32)).max(1)
    assert np.array_equal(s.astype(np.int64) - 127, np.floor(np.log2(amax)).astype(np.int64) - 8)
    # elements never exceed 448 in code units
    assert np.all(np.abs(orc.e4m3_decode(c)) <= 448)
    # idempotent
    c2, s2 = orc.mx_quantize(dq)
    assert np.array_equal(c2, c) and np.array_equal(s2, s)
    # relative error <= 2^-4 where the scaled element is a normal, unsaturated E4M3 value
    scaled = np.abs(v) / np.repeat(2.0 ** (s.astype(np.int64) - 127), 32)
    ok = (scaled >= 2.0 ** -6) & (scaled <= 448)
    assert np.all(np.abs(dq[ok] - v[ok]) <= 2.0 ** -4 * np.abs(v[ok]))
    # all-zero block: smallest scale, zero codes
    c0, s0 = orc.mx_quantize(np.zeros(32))
    assert s0[0] == 0 and np.all(c0 == 0)


def test_mx_exact_round_trip(orc):
    codes, vals = _all_finite_codes()
    rng = np.random.default_rng(5)
    for E in (-20, -8, 0, 5):
        pick = vals[rng.integers(0, vals.size, 32)]
        pick[0] = 288.0  # an E4M3 value with floor(log2) = 8: the scale is 2^E
        blk = pick * 2.0 ** E
        c, s = orc.mx_quantize(blk)
        assert s[0] == E + 127
        assert np.array_equal(orc.mx_dequantize(c, s), blk)
