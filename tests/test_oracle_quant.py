"""Pins for the oracle's block quantizers (CPU only).

Pinned against: the glossary's printed mean absolute errors, the worked scale
example's 448, the IF4 explainer's Table 1, exact-rational brute force on tiny
blocks, and invariants the formats guarantee (amax -> 6, q(W^T) = q(W)^T, the
column-wise layout being the row-wise layout of X^T, exact round trips of
grid-aligned inputs).
"""
import json
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth_inputs as si

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
G = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _nibbles(codes):
    return np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


# --- the glossary's block-size comparison -----------------------------------------------

def test_glossary_block_mae_reproduces_page_values():
    x = si.tiny_reference()
    want = GOLD["glossary_block_mae"]["value"]
    for block in (4096, 32, 16):
        y = oracle.plain_block_roundtrip(x, block)
        mae = float(np.mean(np.abs(y.astype(np.float64) - x.astype(np.float64))))
        assert round(mae, 4) == want[str(block)], (block, mae)


def test_contract_formats_on_tiny_reference_order_like_the_page():
    """NVFP4 (16, E4M3 + FP32) beats MXFP4 (32, E8M0), and both beat one tensor scale."""
    x = si.tiny_reference().reshape(1, -1)
    c, s, gs = oracle.quantize_nvfp4(x)
    mae_nv = np.mean(np.abs(oracle.dequantize(oracle.FMT_NVFP4, c, s, gs, 1, 4096) - x))
    c, s = oracle.quantize_mxfp4(x)
    mae_mx = np.mean(np.abs(oracle.dequantize(oracle.FMT_MXFP4, c, s, 1.0, 1, 4096) - x))
    c, s, gs = oracle.quantize_if4(x)
    mae_if = np.mean(np.abs(oracle.dequantize(oracle.FMT_IF4, c, s, gs, 1, 4096) - x))
    mae_one = np.mean(np.abs(oracle.plain_block_roundtrip(x, 4096) - x))
    assert mae_if <= mae_nv < mae_mx < mae_one
    # Regression values computed independently of this oracle (a separate CPU
    # implementation of the same definitions), to four decimals: NVFP4 0.0779, MXFP4
    # 0.1094, IF4 0.0722 with 153 of the 256 blocks INT4, one plain tensor scale 0.7238.
    assert round(float(mae_nv), 4) == 0.0779 and round(float(mae_mx), 4) == 0.1094
    assert round(float(mae_if), 4) == 0.0722 and int(np.count_nonzero(s >= 0x80)) == 153
    assert round(float(mae_one), 4) == 0.7238


# --- NVFP4 --------------------------------------------------------------------------

def test_worked_scale_example_block_with_tensor_amax_gets_448():
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = (rng.standard_normal(64).astype(np.float32) * np.float32(100.0))
        x[0] = 10000
        _, s, gs = oracle.quantize_nvfp4(x.reshape(1, 64))
        assert oracle.e4m3_decode(int(s[0, 0])) == GOLD["scale_of_block_holding_tensor_amax"]["value"]
        assert np.all(s[0, 1:] < 0x7E)
        assert gs == np.float32(2688.0) / np.float32(10000.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nvfp4_block_max_maps_to_six(dtype):
    x = si.activation(64, 256, seed=1)
    if dtype == "f32":
        x = si.bf16_bits_to_f32(x) * np.float32(1.37)
    xf = si.bf16_bits_to_f32(x) if dtype == "bf16" else x
    codes, scales, gs = oracle.quantize_nvfp4(x)
    nib = _nibbles(codes)
    amax = np.max(np.abs(xf))
    for r in range(xf.shape[0]):
        for b in range(xf.shape[1] // 16):
            blk = np.abs(xf[r, b * 16:(b + 1) * 16])
            s = oracle.e4m3_decode(int(scales[r, b]))
            k = int(np.argmax(blk))
            if s >= 2.0 ** -6:                   # normal E4M3 scale
                assert nib[r, b * 16 + k] & 7 == 7
    # the largest reconstructed magnitude is the tensor amax up to the binary32 roundings
    y = oracle.dequantize(oracle.FMT_NVFP4, codes, scales, gs, *xf.shape)
    assert abs(np.max(np.abs(y)) - amax) <= 4 * np.spacing(np.float32(amax))


def test_nvfp4_colwise_is_rowwise_of_transpose():
    x = si.activation(48, 80, seed=9)
    c_col, s_col, gs = oracle.quantize_nvfp4(x, colwise=True)
    c_row, s_row, gs_t = oracle.quantize_nvfp4(np.ascontiguousarray(x.T))
    assert gs == gs_t
    assert np.array_equal(c_col, c_row) and np.array_equal(s_col, s_row)
    # SR uses a different stream for the column-wise output
    c_col_sr, _, _ = oracle.quantize_nvfp4(x, colwise=True, rnd=oracle.SR, seed=3)
    c_row_sr, _, _ = oracle.quantize_nvfp4(np.ascontiguousarray(x.T), rnd=oracle.SR, seed=3)
    assert not np.array_equal(c_col_sr, c_row_sr)


def test_nvfp4_sampled_rows_match_whole_matrix():
    x = si.activation(64, 96, seed=4)
    gs = oracle.tensor_scale(oracle.amax(x))
    for colwise in (False, True):
        for rnd in (oracle.RTN, oracle.SR):
            c, s, _ = oracle.quantize_nvfp4(x, colwise=colwise, gs=gs, rnd=rnd, seed=17)
            cr, sr = oracle.quantize_nvfp4_rows(x, 5, 7, colwise, gs, rnd=rnd, seed=17)
            assert np.array_equal(cr, c[5:12]) and np.array_equal(sr, s[5:12])


def test_nvfp4_zero_scale_block_gives_signed_zeros():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16:] = np.float32(1e-12) * np.array([1, -1] * 8, np.float32)
    codes, scales, _ = oracle.quantize_nvfp4(x)
    assert scales[0, 1] == 0
    nib = _nibbles(codes)[0, 16:]
    assert np.array_equal(nib, np.array([0, 8] * 8, np.uint8))


def test_dequant_of_grid_aligned_input_is_exact():
    """x = g * s / gs with a power-of-two s and gs = 1 (amax = 2688) round-trips exactly."""
    rng = np.random.default_rng(1)
    rows, cols = 8, 64
    g = rng.choice(np.concatenate([G, -G[1:]]), size=(rows, cols)).astype(np.float32)
    g[:, ::16] = 6.0                           # each block's max is on the grid top
    s = np.float32(2.0) ** rng.integers(-4, 7, size=(rows, cols // 16)).astype(np.float32)
    s[0, 0] = 448.0                            # this block's max 6*448 is the tensor amax -> gs = 1
    x = (g * np.repeat(s, 16, axis=1)).astype(np.float32)
    codes, scales, gs = oracle.quantize_nvfp4(x)
    assert gs == 1.0
    y = oracle.dequantize(oracle.FMT_NVFP4, codes, scales, gs, rows, cols)
    assert np.array_equal(y, x)


# --- NVFP4 16x16 -----------------------------------------------------------------------

def test_2d_quantization_commutes_with_transpose():
    w = si.weight(96, 160, seed=8)
    c, s, gs = oracle.quantize_nvfp4_2d(w)
    ct, st, gst = oracle.quantize_nvfp4_2d(np.ascontiguousarray(w.T))
    assert gs == gst
    assert np.array_equal(st, s.T)
    assert np.array_equal(_nibbles(ct), _nibbles(c).T)
    # one scale per 16x16 tile: the tile's max maps to 6
    nib = _nibbles(c)
    for br in range(6):
        for bc in range(10):
            tile = np.abs(w[br * 16:(br + 1) * 16, bc * 16:(bc + 1) * 16])
            i, j = np.unravel_index(np.argmax(tile), tile.shape)
            assert nib[br * 16 + i, bc * 16 + j] & 7 == 7


def test_2d_equals_1x16_when_every_tile_row_shares_the_max():
    """If each 16x16 tile's rows all have the same block amax, both schemes coincide."""
    rng = np.random.default_rng(2)
    w = rng.uniform(-1, 1, (32, 32)).astype(np.float32)
    w[:, ::16] = 1.0
    c2, s2, _ = oracle.quantize_nvfp4_2d(w)
    c1, s1, _ = oracle.quantize_nvfp4(w)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1[::16], s2)


def _e4m3_values_by_torch(codes: np.ndarray) -> np.ndarray:
    """E4M3 values decoded by torch's float8_e4m3fn cast (independent of the oracle)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _grid_aligned_2d(rows, cols, seed):
    """Codes, tile scales, gs and the exact values x = g * s / gs of a 2D quantization
    built by hand: every 16x16 tile holds a +-6, so quantizing x gives back the same
    codes and scales, and dequantizing them must give x exactly."""
    rng = np.random.default_rng(seed)
    nib = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    nib[::16, ::16] = 7 | (rng.integers(0, 2, size=(rows // 16, cols // 16)).astype(np.uint8) << 3)
    tiles = rng.integers(0x20, 0x77, size=(rows // 16, cols // 16)).astype(np.uint8)
    gs = np.float32(0.125)                                # a power of two: g*s/gs stays exact
    g = np.where(nib & 8, -1.0, 1.0) * G[nib & 7]         # the page's E2M1 values
    s = np.repeat(np.repeat(_e4m3_values_by_torch(tiles).astype(np.float64), 16, 0), 16, 1)
    x = (g * s / float(gs)).astype(np.float32)
    x[(nib == 8)] = np.float32(-0.0)
    assert np.array_equal(x.astype(np.float64), g * s / float(gs))
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, tiles, gs, x


def _check_2d_dequant_pins(dequantize, quantize_2d=None):
    """The 2D dequantization against hand-built tiles (non-square tile grid, a
    different scale per tile), and its transpose identity."""
    rows, cols = 48, 80
    codes, tiles, gs, x = _grid_aligned_2d(rows, cols, seed=31)
    y = dequantize(oracle.FMT_NVFP4_2D, codes, tiles, gs, rows, cols)
    ok = np.array_equal(y.view(np.uint32), x.view(np.uint32))
    if quantize_2d is not None:
        c, sc, _ = quantize_2d(x, gs=gs)
        ok = ok and np.array_equal(c, codes) and np.array_equal(sc, tiles)
    return ok


def test_2d_dequantize_of_grid_aligned_tiles_is_exact():
    assert _check_2d_dequant_pins(oracle.dequantize, oracle.quantize_nvfp4_2d)


def test_2d_dequantize_of_transpose_is_transpose_of_dequantize():
    w = si.weight(96, 160, seed=13)
    c, s, gs = oracle.quantize_nvfp4_2d(w)
    ct, st, gst = oracle.quantize_nvfp4_2d(np.ascontiguousarray(w.T))
    y = oracle.dequantize(oracle.FMT_NVFP4_2D, c, s, gs, 96, 160)
    yt = oracle.dequantize(oracle.FMT_NVFP4_2D, ct, st, gst, 160, 96)
    assert np.array_equal(yt.view(np.uint32), np.ascontiguousarray(y.T).view(np.uint32))
    # and each tile dequantizes with its own scale: x_hat = fl(fl(r * s) / gs)
    r = np.where(_nibbles(c) & 8, -1.0, 1.0) * G[_nibbles(c) & 7]
    sv = np.repeat(np.repeat(_e4m3_values_by_torch(s), 16, 0), 16, 1)
    want = ((r.astype(np.float32) * sv).astype(np.float32) / np.float32(gs)).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))


def test_2d_dequantize_pin_catches_a_wrong_tile_index(tmp_path):
    """Plant a transposed tile index in a copy of the oracle: the pin must fail."""
    import ctypes
    src = open(oracle.SRC).read()
    good = "scales[(r / 16) * (cols / 16) + c / 16]"
    assert src.count(good) == 1
    bad_src = tmp_path / "mutant.c"
    bad_src.write_text(src.replace(good, "scales[(c / 16) * (rows / 16) + r / 16]"))
    so = str(tmp_path / "libmutant.so")
    cmd = [a if a != oracle.LIB else so for a in oracle.BUILD_CMD]
    cmd = [a if a != oracle.SRC else str(bad_src) for a in cmd]
    subprocess.run(cmd + ["-I", oracle.HERE], check=True)
    m = ctypes.CDLL(so)
    m.ora_dequantize.restype = None
    m.ora_dequantize.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]

    def mutant_dequantize(fmt, codes, scales, gs, rows, cols):
        codes, scales = np.ascontiguousarray(codes), np.ascontiguousarray(scales)
        y = np.zeros((rows, cols), np.float32)
        m.ora_dequantize(fmt, codes.ctypes.data, scales.ctypes.data, gs, rows, cols, y.ctypes.data)
        return y

    assert _check_2d_dequant_pins(oracle.dequantize)
    assert not _check_2d_dequant_pins(mutant_dequantize)


# --- MXFP4 --------------------------------------------------------------------------

def test_mxfp4_scale_is_nearest_power_of_two_of_amax_over_6():
    x = si.weight(32, 256, seed=5) * np.float32(50)
    codes, scales = oracle.quantize_mxfp4(x)
    nib = _nibbles(codes)
    for r in range(32):
        for b in range(8):
            blk = x[r, b * 32:(b + 1) * 32]
            bamax = Fraction(float(np.max(np.abs(blk))))
            y = Fraction(float(np.float32(np.max(np.abs(blk))) / np.float32(6)))
            k = int(scales[r, b]) - 127
            # nearest power of two in value to y
            assert abs(y - Fraction(2) ** k) <= min(abs(y - Fraction(2) ** (k - 1)), abs(y - Fraction(2) ** (k + 1)))
            # block max lands on 6 (significand of y below 1.5) or 4 (above 1.5)
            j = int(np.argmax(np.abs(blk)))
            mag = G[nib[r, b * 32 + j] & 7]
            vmax = bamax / Fraction(2) ** k
            assert mag == (6.0 if vmax > 5 else 4.0)
    y = oracle.dequantize(oracle.FMT_MXFP4, codes, scales, 1.0, 32, 256)
    # dequantization is exact: each value is g * 2^k
    k = np.repeat(scales.astype(np.int32) - 127, 32, axis=1)
    assert np.array_equal(y, (np.array([oracle.e2m1_decode(int(n)) for n in range(16)], np.float32)[nib]
                              * np.ldexp(np.float32(1), k)).astype(np.float32))


# --- IF4 ----------------------------------------------------------------------------

def _brute_if4_choice(v):
    """Exact-rational SSE of both candidates for the block's scaled values v (float32)."""
    fv = [Fraction(float(a)) for a in v]
    c76, c67 = Fraction(float(np.float32(7) / np.float32(6))), Fraction(float(np.float32(6) / np.float32(7)))
    grid = [Fraction(g) for g in G]
    e_fp = e_int = Fraction(0)
    for a in fv:
        d = [abs(abs(a) - g) for g in grid]
        m = min(d)
        cs = [c for c in range(8) if d[c] == m]
        c = cs[0] if len(cs) == 1 else [c for c in cs if c % 2 == 0][0]
        r = grid[c] if a >= 0 else -grid[c]
        e_fp += (a - r) ** 2
        q = max(-7, min(7, round(a * c76)))     # Python round: nearest, ties to even
        e_int += (a - q * c67) ** 2
    return e_fp, e_int


def test_if4_choice_matches_exact_rational_brute_force():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal((40, 64)), rng.uniform(-1, 1, (40, 64)),
                        rng.laplace(0, 1, (40, 64))]).astype(np.float32)
    codes, scales, gs = oracle.quantize_if4(x)
    near_ties = 0
    for r in range(x.shape[0]):
        for b in range(4):
            blk = x[r, b * 16:(b + 1) * 16]
            s = np.float32(oracle.e4m3_decode(int(scales[r, b]) & 0x7F))
            v = ((blk * np.float32(gs)).astype(np.float32) / s).astype(np.float32)
            e_fp, e_int = _brute_if4_choice(v)
            flag = bool(scales[r, b] & 0x80)
            if abs(e_fp - e_int) <= Fraction(1, 2 ** 20) * max(e_fp, e_int):
                near_ties += 1
                continue
            assert flag == (e_int < e_fp), (r, b, float(e_fp), float(e_int))
    assert near_ties < 3


def test_if4_never_worse_than_nvfp4_per_block_and_flag_polarity():
    x = si.if4_mix(64, 128, seed=2)
    ci, si_, gs = oracle.quantize_if4(x)
    cn, sn, gsn = oracle.quantize_nvfp4(x)
    assert gs == gsn
    assert np.array_equal(si_ & 0x7F, sn)               # same E4M3 scale; flag only in bit 7
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    yi = oracle.dequantize(oracle.FMT_IF4, ci, si_, gs, *x.shape).astype(np.float64)
    yn = oracle.dequantize(oracle.FMT_NVFP4, cn, sn, gs, *x.shape).astype(np.float64)
    ei = ((yi - xf) ** 2).reshape(64, 8, 16).sum(-1)
    en = ((yn - xf) ** 2).reshape(64, 8, 16).sum(-1)
    assert np.all(ei <= en * (1 + 1e-5) + 1e-30)
    # blocks flagged FP4 are byte-identical to NVFP4
    fp_blocks = (si_ & 0x80) == 0
    cb_i = ci.reshape(64, 8, 8)
    cb_n = cn.reshape(64, 8, 8)
    assert np.array_equal(cb_i[fp_blocks], cb_n[fp_blocks])
    # INT4 nibbles never use -8
    int_blocks = ~fp_blocks
    assert np.all(_nibbles(ci).reshape(64, 8, 16)[int_blocks] != 8)


def test_if4_table1_mse_on_normal_data():
    """Table 1 of the IF4 explainer: MSE on normal data NVFP4 9.0 -> IF4 6.2 (x1e-3).

    The page prints one decimal; with 4M samples the sampling error is about 0.01,
    so the check allows the printed value +-0.1."""
    x = si.normal_f32(1 << 22, seed=12).reshape(4096, 1024)
    want = GOLD["if4_table1_mse_normal"]["value"]
    cn, sn, gs = oracle.quantize_nvfp4(x)
    ci, sc, gsi = oracle.quantize_if4(x)
    mse_n = np.mean((oracle.dequantize(oracle.FMT_NVFP4, cn, sn, gs, *x.shape) - x).astype(np.float64) ** 2)
    mse_i = np.mean((oracle.dequantize(oracle.FMT_IF4, ci, sc, gsi, *x.shape) - x).astype(np.float64) ** 2)
    assert abs(mse_n * 1e3 - want["nvfp4"]) < 0.1
    assert abs(mse_i * 1e3 - want["if4"]) < 0.1


def test_if4_int4_rate_per_distribution():
    """Share of blocks that take INT4 on the IF4 workload's three row groups: about
    0.63 for N(0,1), 0.93 for U(-1,1) and 0.42 for Laplace(0,1) (regression values
    computed independently of this oracle; uniform data has no large values for FP4's
    coarse top step, heavy tails favour it)."""
    x = si.if4_mix(2048, 1024, seed=5)
    _, s, _ = oracle.quantize_if4(x)
    f = s >= 0x80
    rates = [f[:1024].mean(), f[1024:1536].mean(), f[1536:].mean()]
    for got, want in zip(rates, (0.63, 0.93, 0.42)):
        assert abs(got - want) < 0.02, rates
