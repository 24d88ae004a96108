"""Pins for the oracle's MX FP6 codec (CPU only): the values the FP6 page prints, an
exact-rational nearest-value search by bisection over the page-pinned grid, the
packing of four codes into three bytes, and the block round trip."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
FMTS = {oracle.E2M3: "e2m3", oracle.E3M2: "e3m2"}


def grid(fmt):
    return [oracle.fp6_decode(fmt, c) for c in range(32)]


@pytest.mark.parametrize("fmt", [oracle.E2M3, oracle.E3M2])
def test_fp6_grid_matches_the_page(fmt):
    g = grid(fmt)
    assert g == sorted(g) and len(set(g)) == 32 and g[0] == 0.0           # monotone codes, 32 magnitudes
    for c in range(32):
        neg = oracle.fp6_decode(fmt, c | 0x20)
        assert neg == -g[c] and np.signbit(neg)                            # the sign bit mirrors
    if fmt == oracle.E3M2:
        assert g[-1] == GOLD["fp6_e3m2_max"]["value"]
        run = GOLD["fp6_e3m2_run"]["value"]
        i = g.index(run[0])
        assert g[i:i + len(run)] == run                                    # consecutive representable values
        steps = np.diff(g)
        assert steps.min() == GOLD["fp6_e3m2_smallest_step"]["value"]
        assert steps.max() / steps.min() == GOLD["fp6_e3m2_step_ratio"]["value"]
    else:
        assert g[-1] == GOLD["fp6_e2m3_max"]["value"]
        # one exponent band: [1, 2) holds 8 values
        assert sum(1 for v in g if 1.0 <= v < 2.0) == GOLD["fp6_e2m3_values_per_binade"]["value"]


def test_fp6_page_rounding_examples():
    ex = GOLD["fp6_e3m2_examples"]["value"]
    got11 = oracle.fp6_decode(oracle.E3M2, oracle.fp6_rtn(oracle.E3M2, 11.0))
    assert got11 in ex["11"] and got11 == 12.0                             # our reading: ties to the even code
    assert oracle.fp6_decode(oracle.E3M2, oracle.fp6_rtn(oracle.E3M2, 0.1)) == ex["0.1"]
    assert oracle.fp6_rtn(oracle.E3M2, 1e30) == 31 and oracle.fp6_rtn(oracle.E2M3, 7.76) == 31   # saturate
    assert oracle.fp6_rtn(oracle.E3M2, -0.0) == 0x20 and oracle.fp6_rtn(oracle.E2M3, -1e-9) == 0x20


def _nearest_even(fmt, v):
    """Bisection over the grid's midpoints with exact rationals; ties to the even code."""
    g = [Fraction(x) for x in grid(fmt)]
    a = abs(Fraction(float(v)))
    lo, hi = 0, 31
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if a >= g[mid]:
            lo = mid
        else:
            hi = mid
    if a >= g[31]:
        return 31
    d_lo, d_hi = a - g[lo], g[hi] - a
    if d_lo < d_hi:
        return lo
    if d_hi < d_lo:
        return hi
    return lo if lo % 2 == 0 else hi


@pytest.mark.parametrize("fmt", [oracle.E2M3, oracle.E3M2])
def test_fp6_rtn_equals_exact_nearest_even_near_every_grid_point_and_midpoint(fmt):
    g = grid(fmt)
    pts = g + [(a + b) / 2 for a, b in zip(g, g[1:])] + [g[-1] * 1.2]
    vals = []
    for p in pts:
        b = np.float32(p).view(np.uint32).astype(np.int64)
        vals.extend(np.arange(max(0, b - 3), b + 4, dtype=np.int64).astype(np.uint32).view(np.float32).tolist())
    for v in vals:
        assert oracle.fp6_rtn(fmt, v) == _nearest_even(fmt, v), (fmt, v)


def test_fp6_packing_four_codes_in_three_bytes():
    # a block whose max is 28 gets scale 2^0 (E8M0 code 127); values on the grid
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :4] = [0.0625, 0.125, 0.1875, 0.25]            # E3M2 codes 1, 2, 3, 4
    x[0, 31] = 28.0
    codes, scales = oracle.quantize_mxfp6(x, oracle.E3M2)
    assert codes.shape == (1, 24) and scales[0, 0] == 127
    word = 1 | (2 << 6) | (3 << 12) | (4 << 18)         # code j at bits 6j of the little-endian 24-bit word
    assert codes[0, :3].tolist() == [word & 0xFF, (word >> 8) & 0xFF, word >> 16]
    assert np.array_equal(oracle.dequantize_mxfp6(oracle.E3M2, codes, scales, 1, 32), x)


@pytest.mark.parametrize("fmt", [oracle.E2M3, oracle.E3M2])
def test_mxfp6_round_trip_error_is_within_half_a_step(fmt):
    rng = np.random.default_rng(31 + fmt)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-4, 4, (16, 1)))).astype(np.float32)
    codes, scales = oracle.quantize_mxfp6(x, fmt)
    y = oracle.dequantize_mxfp6(fmt, codes, scales, 16, 256)
    g = np.array(grid(fmt))
    mb = 3 if fmt == oracle.E2M3 else 2
    for r in range(16):
        for b in range(8):
            s = 2.0 ** (int(scales[r, b]) - 127)
            blk, out = x[r, 32 * b:32 * b + 32].astype(np.float64), y[r, 32 * b:32 * b + 32].astype(np.float64)
            # E8M0 is the nearest power of two of amax / max: the block max lands within sqrt(2) of max
            assert np.abs(blk).max() / s <= g[-1] * 1.5
            inside = np.abs(blk) / s <= g[-1]
            step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(blk) / s, 1e-30))) - mb), g[1])
            assert np.all(np.abs(out - blk)[inside] <= 0.5 * step[inside] * s * (1 + 1e-6))
            assert np.all(np.sign(out[~inside]) * blk[~inside] >= 0) and np.all(np.abs(out[~inside]) == g[-1] * s)
