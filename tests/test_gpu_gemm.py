"""GPU parity of the MXFP4 GEMM (fp4q_gemm_mxfp4, through the C ABI) against the oracle.

The oracle's C is exact (binary64).  Every product of two MXFP4 values is exact in
fp32, so the kernel's only error is its fp32 summation: whatever order the block-scaled
MFMA uses inside one instruction (64 products) and across the k/64 instructions, a
summation tree of depth at most 6 + k/64 bounds it by (6 + k/64) u sum|a b| with
u = 2^-24; the tolerance doubles that to allow either rounding inside the instruction.
A bf16 output adds its rounding error, at most half an ulp of an 8-bit significand,
2^-8 |C|.  A wrong scale byte, K
block or lane mapping misses this by orders of magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from block_scaled_fp4_05_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _operand(rng, rows, k, lo=118, hi=136):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, k // 32), dtype=np.uint8)
    return codes, scales


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _gemm(ac, as_, bc, bs, out_dtype=torch.float32) -> np.ndarray:
    m, n, k = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    c = torch.full((m, n), float("nan"), dtype=out_dtype, device=DEV)
    B.fp4q_gemm_mxfp4(_dev(ac), _dev(as_), _dev(bc), _dev(bs), m, n, k, B._dt(c), c)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def _check(got, exact, cabs, k, bf16=False):
    tol = 2.0 * (6 + k / 64) * 2.0 ** -24 * cabs
    if bf16:
        tol = tol + 2.0 ** -8 * (np.abs(exact) + tol)
    err = np.abs(got - exact)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, (f"{len(bad)} of {err.size} outside the bound; first {bad[:4].tolist()}, "
                           f"err {err[tuple(bad[0])]:.3e} tol {tol[tuple(bad[0])]:.3e}")


@pytest.mark.parametrize("shape", [(256, 256, 128), (300, 520, 384), (1, 1, 128), (257, 129, 256),
                                   (64, 2048, 1024), (1000, 333, 640), (513, 768, 2048)])
def test_gemm_random_codes_fp32_out(shape):
    m, n, k = shape
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    ac, as_ = _operand(rng, m, k)
    bc, bs = _operand(rng, n, k)
    print(f"gemm m={m} n={n} k={k}", flush=True)
    got = _gemm(ac, as_, bc, bs)
    exact, cabs = oracle.gemm_mxfp4(ac, as_, bc, bs)
    _check(got, exact, cabs, k)


@pytest.mark.parametrize("shape", [(256, 256, 256), (390, 200, 512), (257, 130, 256), (600, 1000, 384)])
def test_gemm_random_codes_bf16_out(shape):
    m, n, k = shape
    rng = np.random.default_rng(99 + m + n + k)
    ac, as_ = _operand(rng, m, k)
    bc, bs = _operand(rng, n, k)
    got = _gemm(ac, as_, bc, bs, torch.bfloat16)
    exact, cabs = oracle.gemm_mxfp4(ac, as_, bc, bs)
    _check(got, exact, cabs, k, bf16=True)


def test_gemm_of_quantizer_outputs():
    """Y = X W^T on what fp4q_quantize_mxfp4 writes for a bf16 activation and an fp32 weight."""
    m, n, k = 384, 320, 1024
    x = si.activation(m, k, seed=31)
    w = si.weight(n, k, seed=32)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    qa = B.quantize_mxfp4(xd)
    qb = B.quantize_mxfp4(torch.from_numpy(w).to(DEV))
    c = B.gemm_mxfp4(qa, qb).cpu().numpy().astype(np.float64)
    ac, as_, bc, bs = (t.cpu().numpy() for t in (qa["codes"], qa["scales"], qb["codes"], qb["scales"]))
    exact, cabs = oracle.gemm_mxfp4(ac, as_, bc, bs)
    _check(c, exact, cabs, k)


def test_gemm_zero_operand_gives_exact_zeros():
    rng = np.random.default_rng(5)
    ac = np.zeros((130, 64), dtype=np.uint8)
    as_ = rng.integers(100, 150, size=(130, 4), dtype=np.uint8)
    bc, bs = _operand(rng, 70, 128)
    got = _gemm(ac, as_, bc, bs)
    assert np.array_equal(got, np.zeros_like(got))


def test_gemm_repeated_calls_agree_bitwise():
    rng = np.random.default_rng(6)
    ac, as_ = _operand(rng, 512, 1024)
    bc, bs = _operand(rng, 512, 1024)
    first = _gemm(ac, as_, bc, bs)
    for _ in range(3):
        assert np.array_equal(_gemm(ac, as_, bc, bs), first)


def test_gemm_full_size_sampled():
    """The 8192 x 8192 x 8192 product, bf16 out, launched as the benchmark launches it;
    sampled rows and columns (tile edges included) against the oracle."""
    m = n = k = 8192
    rng = np.random.default_rng(8)
    ac, as_ = _operand(rng, m, k, 120, 134)
    bc, bs = _operand(rng, n, k, 120, 134)
    print("gemm full size", flush=True)
    c = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    B.fp4q_gemm_mxfp4(_dev(ac), _dev(as_), _dev(bc), _dev(bs), m, n, k, B.BF16, c)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 256, 4095, 4100, 8064, 8190, 8191])
    cols = np.array([0, 31, 32, 255, 256, 1000, 4096, 8000, 8191])
    exact, cabs = oracle.gemm_mxfp4(ac[rows], as_[rows], bc[cols], bs[cols])
    got = c[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy()
    _check(got.astype(np.float64), exact, cabs, k, bf16=True)
