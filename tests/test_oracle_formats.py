"""Pins for the oracle's element and scale codecs (CPU only).

Each test checks the oracle against something other than itself: a value the
pages print, a closed form, a brute-force search with exact rationals, or an
independent library conversion (torch's float8_e4m3fn cast).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def _f32_neighbors(values, k=48):
    """All float32 bit patterns within +-k ulps of each value (non-negative)."""
    out = []
    for v in values:
        b = np.float32(v).view(np.uint32).astype(np.int64)
        lo = max(0, b - k)
        out.append(np.arange(lo, b + k + 1, dtype=np.int64).astype(np.uint32).view(np.float32))
    return np.concatenate(out)


# --- E2M1 -----------------------------------------------------------------------

def test_e2m1_decode_matches_page_closed_form_and_value_list():
    # The E2M1 closed form on the page: e=0 -> (-1)^s * 0.5m * 2^0, e>0 -> (-1)^s (1+0.5m) 2^(e-1)
    for nib in range(16):
        s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
        expect = (0.5 * m) if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
        expect = -expect if s else expect
        got = oracle.e2m1_decode(nib)
        assert got == expect and np.signbit(got) == bool(s)
    distinct = sorted({oracle.e2m1_decode(n) for n in range(16)})
    assert distinct == GOLD["e2m1_values"]["value"]          # 15 values (+0 and -0 compare equal)
    assert max(distinct) * GOLD["e4m3_max"]["value"] == GOLD["nvfp4_max"]["value"]


def _brute_rtn(a: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude by exact rational distance, ties to the even code."""
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    out = np.zeros(a.size, dtype=np.uint8)
    for i, v in enumerate(a.tolist()):
        fv = Fraction(v)
        d = [abs(fv - g) for g in grid]
        m = min(d)
        cands = [c for c in range(8) if d[c] == m]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out[i] = c
    return out


def test_e2m1_rtn_brute_force_near_every_threshold_and_grid_point():
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0, 8.0]
    a = _f32_neighbors(pts, k=40)
    rng = np.random.default_rng(11)
    a = np.concatenate([a, rng.uniform(0, 9, 20000).astype(np.float32),
                        (np.arange(0, 9 * 4096) / 4096.0).astype(np.float32)])
    got = oracle.e2m1_rtn(a)
    assert np.array_equal(got & 7, _brute_rtn(a))
    assert np.all(got & 8 == 0)
    # sign is copied, including for values that round to zero and for -0
    neg = oracle.e2m1_rtn(-a)
    assert np.array_equal(neg & 7, got & 7) and np.all(neg & 8 == 8)
    assert oracle.e2m1_rtn(np.float32(-0.0))[0] == 0x8
    # saturation: anything beyond 6 is 6
    assert np.all(oracle.e2m1_rtn(np.array([5.0001, 7, 1e3, 3e38], np.float32)) == 7)


def test_e2m1_rtn_ties_go_to_even_code():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in ties.items():
        assert oracle.e2m1_rtn(np.float32(v))[0] == c, v


# --- stochastic rounding -----------------------------------------------------------

def _grid_bracket(a):
    g = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    lo = max(c for c in range(7) if g[c] <= a)
    return lo, Fraction(g[lo]), Fraction(g[lo + 1])


def test_sr_midpoint_is_fifty_fifty_as_the_page_says():
    r = np.arange(65536, dtype=np.uint32)
    codes = oracle.e2m1_sr(np.full(65536, 2.5, np.float32), r)
    up = np.count_nonzero(codes == 5)          # 3.0
    down = np.count_nonzero(codes == 4)        # 2.0
    assert up + down == 65536
    assert up / 65536 == GOLD["sr_midpoint_probability"]["value"]


def test_sr_expectation_closed_form_and_support():
    """Over all 2^16 draws: only the bracketing grid values occur, and the mean is
    lo + step * floor(frac * 2^16) / 2^16 exactly (frac on the local interval)."""
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.uniform(0, 6, 60).astype(np.float32),
                           np.array([0.0, 0.1, 0.5, 0.7, 1.0, 1.3, 2.0, 2.9, 4.0, 5.99, 6.0, 7.5,
                                     1e-30, 0.4999999], np.float32)])
    r = np.arange(65536, dtype=np.uint32)
    for v in vals.tolist():
        codes = oracle.e2m1_sr(np.full(65536, v, np.float32), r)
        mags = np.array([abs(oracle.e2m1_decode(int(c))) for c in range(8)])[codes & 7]
        if v >= 6:
            assert np.all(mags == 6.0)
            continue
        lo_c, lo, hi = _grid_bracket(v)
        assert set(np.unique(mags).tolist()) <= {float(lo), float(hi)}
        frac = (Fraction(v) - lo) / (hi - lo)
        expect = lo + (hi - lo) * Fraction(int(frac * 65536), 65536)
        mean = Fraction(int(np.count_nonzero(mags == float(hi)))) / 65536 * (hi - lo) + lo
        assert mean == expect, v
        assert abs(float(mean) - v) <= float(hi - lo) / 65536 + 1e-12
    # on a grid point the result is deterministic
    for g in [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]:
        codes = oracle.e2m1_sr(np.full(65536, g, np.float32), r)
        assert np.all(codes == codes[0])
    assert np.all(oracle.e2m1_sr(np.full(4, -2.5, np.float32), np.array([0, 1, 65535, 32768])) & 8 == 8)


# --- E4M3 ---------------------------------------------------------------------------

def _e4m3_values():
    return np.array([oracle.e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)


def test_e4m3_decode_is_the_fn_format_with_max_448():
    vals = _e4m3_values()
    assert np.all(np.diff(vals) > 0)
    assert vals[-1] == GOLD["e4m3_max"]["value"]
    t = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(vals, t)


def test_e4m3_encode_matches_torch_cast_below_464():
    vals = _e4m3_values()
    mids = (vals[1:] + vals[:-1]) / 2
    y = _f32_neighbors(np.concatenate([vals, mids]).astype(np.float32), k=24)
    rng = np.random.default_rng(3)
    y = np.concatenate([y, rng.uniform(0, 464, 200000).astype(np.float32),
                        np.exp(rng.uniform(-20, 6.1, 200000)).astype(np.float32)])
    y = y[(y >= 0) & (y < 464)]
    got = oracle.e4m3_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_at_448():
    y = np.array([448.0, 463.9, 464.0, 465.0, 1e4, 3e38], np.float32)
    assert np.all(oracle.e4m3_encode(y) == 0x7E)


# --- E8M0 ---------------------------------------------------------------------------

def test_e8m0_is_nearest_power_of_two_with_even_ties():
    ys = np.array([np.ldexp(m, e) for e in range(-140, 128)
                   for m in (1.0, 1.25, 1.5, 1.75, 1.9999999)], dtype=np.float64).astype(np.float32)
    ys = ys[np.isfinite(ys) & (ys > 0)]
    ys = np.concatenate([ys, _f32_neighbors(np.float32(1.5) * (2.0 ** np.arange(-120, 120)).astype(np.float32), k=2)])
    got = oracle.e8m0_encode(ys)
    for y, c in zip(ys.tolist(), got.tolist()):
        fy = Fraction(y)
        # candidates: every code 0..254, value 2^(code-127); nearest in value, ties to even code
        e = fy.numerator.bit_length() - fy.denominator.bit_length()
        cands = [k for k in range(max(0, e + 127 - 2), min(254, e + 127 + 2) + 1)]
        if not cands:
            cands = [0] if e < 0 else [254]
        d = {k: abs(fy - Fraction(2) ** (k - 127)) for k in cands}
        m = min(d.values())
        best = [k for k in cands if d[k] == m]
        expect = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
        if e + 127 < 0:
            expect = 0
        assert c == expect, (y, c, expect)
    assert oracle.e8m0_encode(np.float32(0.0))[0] == 0
    assert oracle.e8m0_decode(127) == 1.0 and oracle.e8m0_decode(0) == 2.0 ** -127
