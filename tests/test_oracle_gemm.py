"""Pins for the oracle's MXFP4 GEMM (CPU only).

C = A B^T over two row-wise MXFP4 operands.  The pins do not re-call the oracle's own
decode: element values come from the E2M1 bit layout the pages give (sign, two exponent
bits, one mantissa bit), summed with exact rationals; a one-hot operand must select
single entries of the other; the product must equal numpy's matmul of the separately
pinned dequantization; and quantized Gaussian operands must track the float product.
"""
from fractions import Fraction

import numpy as np

import oracle
import synth_inputs as si


def _e2m1_exact(nib: int) -> Fraction:
    # The page's closed form: e = 0 -> 0.5 m; e > 0 -> (1 + 0.5 m) 2^(e-1); sign bit mirrors.
    s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
    v = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -v if s else v


def _random_operand(rng, rows, k, lo=118, hi=136):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, k // 32), dtype=np.uint8)
    return codes, scales


def _exact_matrix(codes, scales):
    rows, k = codes.shape[0], codes.shape[1] * 2
    out = [[Fraction(0)] * k for _ in range(rows)]
    for r in range(rows):
        for t in range(k):
            byte = int(codes[r, t // 2])
            nib = (byte >> 4) if (t & 1) else (byte & 15)       # element 2i in the low nibble
            out[r][t] = _e2m1_exact(nib) * Fraction(2) ** (int(scales[r, t // 32]) - 127)
    return out


def test_gemm_brute_force_with_exact_rationals():
    rng = np.random.default_rng(11)
    m, n, k = 3, 4, 96
    ac, as_ = _random_operand(rng, m, k)
    bc, bs = _random_operand(rng, n, k)
    c, cabs = oracle.gemm_mxfp4(ac, as_, bc, bs)
    A, B = _exact_matrix(ac, as_), _exact_matrix(bc, bs)
    for i in range(m):
        for j in range(n):
            exact = sum(A[i][t] * B[j][t] for t in range(k))
            mag = sum(abs(A[i][t] * B[j][t]) for t in range(k))
            assert c[i, j] == float(exact) and Fraction(c[i, j]) == exact
            assert cabs[i, j] == float(mag)


def test_gemm_one_hot_rows_select_entries_of_the_other_operand():
    rng = np.random.default_rng(12)
    m, n, k = 64, 5, 64
    bc, bs = _random_operand(rng, n, k)
    ac = np.zeros((m, k // 2), dtype=np.uint8)
    for i in range(m):
        ac[i, i // 2] = 0x2 << (4 * (i & 1))                    # +1.0 at column i
    as_ = np.full((m, k // 32), 127, dtype=np.uint8)          # 2^0
    c, _ = oracle.gemm_mxfp4(ac, as_, bc, bs)
    bdq = oracle.dequantize(2, bc, bs, 1.0, n, k)
    assert np.array_equal(c, bdq[:, :m].T.astype(np.float64))


def test_gemm_equals_matmul_of_the_dequantized_operands():
    rng = np.random.default_rng(13)
    m, n, k = 37, 29, 320
    ac, as_ = _random_operand(rng, m, k)
    bc, bs = _random_operand(rng, n, k)
    c, cabs = oracle.gemm_mxfp4(ac, as_, bc, bs)
    a = oracle.dequantize(2, ac, as_, 1.0, m, k).astype(np.float64)
    b = oracle.dequantize(2, bc, bs, 1.0, n, k).astype(np.float64)
    assert np.array_equal(c, a @ b.T)                          # every partial sum is exact
    assert np.array_equal(cabs, np.abs(a) @ np.abs(b).T)


def test_gemm_of_quantized_gaussians_tracks_the_float_product():
    m, n, k = 48, 40, 1024
    x = si.weight(m, k, seed=21, std=1.0)
    w = si.weight(n, k, seed=22, std=0.02)
    ac, as_ = oracle.quantize_mxfp4(x)
    bc, bs = oracle.quantize_mxfp4(w)
    c, _ = oracle.gemm_mxfp4(ac, as_, bc, bs)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    # E2M1 with a per-32 power-of-two scale keeps each element within about 1/6 of its
    # block maximum; two independently quantized operands give roughly 0.1 relative error.
    assert 0.02 < rel < 0.2


# --- NVFP4 1x16 operands ------------------------------------------------------------

def _nv_operand(rng, rows, k):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(1, 127, size=(rows, k // 16), dtype=np.uint8)   # positive, finite e4m3fn codes
    return codes, scales


def _e4m3_exact(code: int) -> Fraction:
    # independent decode: torch's own float8_e4m3fn interpretation of the byte
    import torch
    v = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
    return Fraction(v)


def test_nvfp4_gemm_brute_force_with_exact_rationals():
    rng = np.random.default_rng(14)
    m, n, k = 2, 3, 64
    ac, as_ = _nv_operand(rng, m, k)
    bc, bs = _nv_operand(rng, n, k)
    gs_a, gs_b = np.float32(37.25), np.float32(1234.5678)
    c, cabs = oracle.gemm_nvfp4(ac, as_, gs_a, bc, bs, gs_b)

    def val(codes, scales, r, t):
        byte = int(codes[r, t // 2])
        nib = (byte >> 4) if (t & 1) else (byte & 15)
        return _e2m1_exact(nib) * _e4m3_exact(int(scales[r, t // 16]))

    g = Fraction(float(gs_a)) * Fraction(float(gs_b))
    for i in range(m):
        for j in range(n):
            exact = sum(val(ac, as_, i, t) * val(bc, bs, j, t) for t in range(k)) / g
            assert abs(Fraction(c[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 52)   # one binary64 rounding
            mag = sum(abs(val(ac, as_, i, t) * val(bc, bs, j, t)) for t in range(k)) / g
            assert abs(Fraction(cabs[i, j]) - mag) <= mag * Fraction(1, 2 ** 52)


def test_nvfp4_gemm_equals_matmul_of_the_dequantized_operands_at_unit_tensor_scale():
    rng = np.random.default_rng(15)
    m, n, k = 19, 23, 256
    ac, as_ = _nv_operand(rng, m, k)
    bc, bs = _nv_operand(rng, n, k)
    c, _ = oracle.gemm_nvfp4(ac, as_, 1.0, bc, bs, 1.0)
    a = oracle.dequantize(0, ac, as_, 1.0, m, k).astype(np.float64)   # r * s, exact at gs = 1
    b = oracle.dequantize(0, bc, bs, 1.0, n, k).astype(np.float64)
    assert np.array_equal(c, a @ b.T)


def test_nvfp4_gemm_of_quantized_gaussians_tracks_the_float_product():
    m, n, k = 40, 48, 1024
    x = si.weight(m, k, seed=23, std=1.0)
    w = si.weight(n, k, seed=24, std=0.02)
    ac, as_, gsa = oracle.quantize_nvfp4(x)
    bc, bs, gsb = oracle.quantize_nvfp4(w)
    c, _ = oracle.gemm_nvfp4(ac, as_, gsa, bc, bs, gsb)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    assert 0.01 < rel < 0.15      # 16-element blocks with E4M3 scales: tighter than MXFP4


# --- NVFP4 16x16 (2D) operands --------------------------------------------------------

def _nv_tiled_operand(rng, rows, k):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(1, 127, size=(rows // 16, k // 16), dtype=np.uint8)
    return codes, scales


def test_nvfp4_gemm_with_tiled_operands_brute_force_with_exact_rationals():
    """A with 16x16 tiles, B with 1x16 blocks and the reverse: element (r, t) of a tiled
    operand carries the scale of tile (r // 16, t // 16)."""
    rng = np.random.default_rng(31)
    m, n, k = 32, 16, 48

    def val(codes, scales, r, t, tiled):
        byte = int(codes[r, t // 2])
        nib = (byte >> 4) if (t & 1) else (byte & 15)
        return _e2m1_exact(nib) * _e4m3_exact(int(scales[r // 16 if tiled else r, t // 16]))

    for tiles in (1, 2, 3):
        ac, as_ = (_nv_tiled_operand if tiles & 1 else _nv_operand)(rng, m, k)
        bc, bs = (_nv_tiled_operand if tiles & 2 else _nv_operand)(rng, n, k)
        gs_a, gs_b = np.float32(3.5), np.float32(0.75)
        c, _ = oracle.gemm_nvfp4(ac, as_, gs_a, bc, bs, gs_b, flags=tiles)
        g = Fraction(float(gs_a)) * Fraction(float(gs_b))
        for i in (0, 15, 16, 31):
            for j in (0, 7, 15):
                exact = sum(val(ac, as_, i, t, tiles & 1) * val(bc, bs, j, t, tiles & 2) for t in range(k)) / g
                assert abs(Fraction(c[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 52), (tiles, i, j)


def test_nvfp4_gemm_tiled_equals_row_blocks_with_replicated_tile_scales():
    """A tiled operand is the same matrix as a 1x16 operand whose row r holds the scales
    of tile row r // 16."""
    rng = np.random.default_rng(32)
    m, n, k = 48, 32, 128
    ac, ast = _nv_tiled_operand(rng, m, k)
    bc, bst = _nv_tiled_operand(rng, n, k)
    c2, cabs2 = oracle.gemm_nvfp4(ac, ast, 2.0, bc, bst, 5.0, flags=3)
    c1, cabs1 = oracle.gemm_nvfp4(ac, np.repeat(ast, 16, axis=0), 2.0, bc, np.repeat(bst, 16, axis=0), 5.0)
    assert np.array_equal(c2, c1) and np.array_equal(cabs2, cabs1)
    c3, _ = oracle.gemm_nvfp4(ac, ast, 2.0, bc, np.repeat(bst, 16, axis=0), 5.0, flags=1)
    assert np.array_equal(c3, c1)


def test_nvfp4_gemm_tiled_equals_matmul_of_the_2d_dequantization():
    rng = np.random.default_rng(33)
    m, n, k = 32, 64, 256
    ac, as_ = _nv_operand(rng, m, k)
    bc, bs = _nv_tiled_operand(rng, n, k)
    c, _ = oracle.gemm_nvfp4(ac, as_, 1.0, bc, bs, 1.0, flags=2)
    a = oracle.dequantize(0, ac, as_, 1.0, m, k).astype(np.float64)
    b = oracle.dequantize(1, bc, bs, 1.0, n, k).astype(np.float64)
    assert np.array_equal(c, a @ b.T)


def test_nvfp4_forward_and_dgrad_with_one_2d_weight_quantization():
    """Y = X W^T uses W quantized in 16x16 tiles; dX = dY W uses W^T, whose 16x16
    quantization is the transposed tile array, so both products track the float ones."""
    m, n, k = 64, 96, 512
    x = si.weight(m, k, seed=41, std=1.0)
    w = si.weight(n, k, seed=42, std=0.02)
    dy = si.weight(m, n, seed=43, std=1.0)
    xc, xs, gx = oracle.quantize_nvfp4(x)
    wc, ws, gw = oracle.quantize_nvfp4_2d(w)
    y, _ = oracle.gemm_nvfp4(xc, xs, gx, wc, ws, gw, flags=2)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert 0.01 < np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.15
    wtc, wts, gwt = oracle.quantize_nvfp4_2d(np.ascontiguousarray(w.T))
    assert np.array_equal(wts, ws.T) and gwt == gw
    dc, ds, gd = oracle.quantize_nvfp4(dy)
    dx, _ = oracle.gemm_nvfp4(dc, ds, gd, wtc, wts, gwt, flags=2)
    ref = dy.astype(np.float64) @ w.astype(np.float64)
    assert 0.01 < np.linalg.norm(dx - ref) / np.linalg.norm(ref) < 0.15


# --- IF4 operands -------------------------------------------------------------------

def _if4_operand(rng, rows, k, int_share=0.5):
    """Random codes and E4M3 scales with the INT4 flag (bit 7) on about int_share of the blocks."""
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(1, 127, size=(rows, k // 16), dtype=np.uint8)
    flags = (rng.random(size=scales.shape) < int_share).astype(np.uint8) << 7
    return codes, scales | flags


def _if4_exact(codes, scales, r, t):
    """Element (r, t) of an IF4 operand as an exact rational, computed apart from the C:
    an INT4 block restores q as the float32 product fl(q * fl(6/7)) (numpy's float32
    multiply), scaled by the E4M3 value of the scale byte without its flag bit."""
    byte = int(codes[r, t // 2])
    nib = (byte >> 4) if (t & 1) else (byte & 15)
    sc = int(scales[r, t // 16])
    if sc & 0x80:
        q = nib - 16 if nib >= 8 else nib
        u = np.float32(q) * np.float32(6.0 / 7.0)
        return Fraction(float(u)) * _e4m3_exact(sc & 0x7F)
    return _e2m1_exact(nib) * _e4m3_exact(sc)


def test_if4_gemm_brute_force_with_exact_rationals():
    """IF4 x NVFP4, NVFP4 x IF4 and IF4 x IF4 (flags 4, 8, 12): every product is exact in
    binary64 (at most 24 + 4 bits times 6 or 28 bits), but with INT4 restores the running
    sum no longer fits 53 bits, so C is the exact rational sum within the summation bound
    (k + 1) 2^-53 sum |products| (k additions and the division by gs_a gs_b); negative
    INT4 codes (nibbles 8..15) and both block kinds occur in every row."""
    rng = np.random.default_rng(61)
    m, n, k = 3, 4, 96
    for flags in (4, 8, 12):
        ac, as_ = (_if4_operand if flags & 4 else _nv_operand)(rng, m, k)
        bc, bs = (_if4_operand if flags & 8 else _nv_operand)(rng, n, k)
        gs_a, gs_b = np.float32(11.5), np.float32(0.3125)
        c, cabs = oracle.gemm_nvfp4(ac, as_, gs_a, bc, bs, gs_b, flags=flags)
        va = (lambda r, t: _if4_exact(ac, as_, r, t)) if flags & 4 else \
            (lambda r, t: _e2m1_exact(((int(ac[r, t // 2]) >> 4) if t & 1 else int(ac[r, t // 2]) & 15)) *
             _e4m3_exact(int(as_[r, t // 16])))
        vb = (lambda r, t: _if4_exact(bc, bs, r, t)) if flags & 8 else \
            (lambda r, t: _e2m1_exact(((int(bc[r, t // 2]) >> 4) if t & 1 else int(bc[r, t // 2]) & 15)) *
             _e4m3_exact(int(bs[r, t // 16])))
        g = Fraction(float(gs_a)) * Fraction(float(gs_b))
        for i in range(m):
            for j in range(n):
                exact = sum(va(i, t) * vb(j, t) for t in range(k)) / g
                mag = sum(abs(va(i, t) * vb(j, t)) for t in range(k)) / g
                bound = (k + 1) * mag * Fraction(1, 2 ** 53)
                assert abs(Fraction(c[i, j]) - exact) <= bound, (flags, i, j)
                assert abs(Fraction(cabs[i, j]) - mag) <= bound


def test_if4_gemm_without_int4_blocks_is_the_nvfp4_product():
    rng = np.random.default_rng(62)
    m, n, k = 17, 21, 256
    ac, as_ = _if4_operand(rng, m, k, int_share=0.0)
    bc, bs = _if4_operand(rng, n, k, int_share=0.0)
    ref, ref_abs = oracle.gemm_nvfp4(ac, as_, 3.0, bc, bs, 7.0)
    for flags in (4, 8, 12):
        c, cabs = oracle.gemm_nvfp4(ac, as_, 3.0, bc, bs, 7.0, flags=flags)
        assert np.array_equal(c, ref) and np.array_equal(cabs, ref_abs)


def test_if4_gemm_of_quantized_gaussians_tracks_the_float_product():
    """Y = X W^T on the oracle's IF4 quantization of both operands tracks the float
    product at least as closely as NVFP4 does (IF4 picks the smaller block error)."""
    m, n, k = 40, 48, 1024
    x = si.weight(m, k, seed=63, std=1.0)
    w = si.weight(n, k, seed=64, std=0.02)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    xc, xs, gx = oracle.quantize_if4(x)
    wc, ws, gw = oracle.quantize_if4(w)
    assert (xs & 0x80).any() and (ws & 0x80).any()
    c, _ = oracle.gemm_nvfp4(xc, xs, gx, wc, ws, gw, flags=12)
    rel_if4 = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    nc, ns, gn = oracle.quantize_nvfp4(x)
    vc, vs, gv = oracle.quantize_nvfp4(w)
    c_nv, _ = oracle.gemm_nvfp4(nc, ns, gn, vc, vs, gv)
    rel_nv = np.linalg.norm(c_nv - ref) / np.linalg.norm(ref)
    assert 0.005 < rel_if4 < 0.15 and rel_if4 <= rel_nv * 1.02, (rel_if4, rel_nv)
