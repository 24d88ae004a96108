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
