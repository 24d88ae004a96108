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


# ---------------------------------------------------------------------------------------
# NVFP4 operands (f16 MFMA after an exact decode; bf16 with IF4 operands).  Each product of two decoded values
# r s has at most twelve significant bits, exact in fp32; an instruction sums 16, so the
# summation depth is at most 4 + k/16.  The tensor scales add three roundings
# (fl(gs_a gs_b), its reciprocal, the product): 3 u |C|.
# ---------------------------------------------------------------------------------------

def _nv_operand(rng, rows, k):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(1, 127, size=(rows, k // 16), dtype=np.uint8)   # positive finite e4m3fn codes
    return codes, scales


def _nv_check(got, exact, cabs, k, bf16=False):
    tol = 2.0 * (4 + k / 16) * 2.0 ** -24 * cabs + 3.0 * 2.0 ** -24 * np.abs(exact)
    if bf16:
        tol = tol + 2.0 ** -8 * (np.abs(exact) + tol)
    err = np.abs(got - exact)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, (f"{len(bad)} of {err.size} outside the bound; first {bad[:4].tolist()}, "
                           f"err {err[tuple(bad[0])]:.3e} tol {tol[tuple(bad[0])]:.3e}")


def _nv_gemm(ac, as_, ga, bc, bs, gb, out_dtype=torch.float32, flags=0):
    m, n, k = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    c = torch.full((m, n), float("nan"), dtype=out_dtype, device=DEV)
    ta = torch.tensor([ga], dtype=torch.float32, device=DEV)
    tb = torch.tensor([gb], dtype=torch.float32, device=DEV)
    B.fp4q_gemm_nvfp4(_dev(ac), _dev(as_), ta, _dev(bc), _dev(bs), tb, m, n, k, flags, B._dt(c), c)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("shape,bf16", [((256, 256, 128), False), ((300, 520, 384), False), ((1, 1, 128), False),
                                        ((257, 129, 256), False), ((513, 768, 1024), False),
                                        ((256, 256, 256), True), ((390, 200, 512), True), ((257, 130, 256), True)])
def test_nvfp4_gemm_random_codes(shape, bf16):
    m, n, k = shape
    rng = np.random.default_rng(m * 5 + n * 11 + k)
    ac, as_ = _nv_operand(rng, m, k)
    bc, bs = _nv_operand(rng, n, k)
    ga, gb = np.float32(173.25), np.float32(0.8125)
    print(f"nvfp4 gemm m={m} n={n} k={k} bf16={bf16}", flush=True)
    got = _nv_gemm(ac, as_, ga, bc, bs, gb, torch.bfloat16 if bf16 else torch.float32)
    exact, cabs = oracle.gemm_nvfp4(ac, as_, ga, bc, bs, gb)
    _nv_check(got, exact, cabs, k, bf16)


def test_nvfp4_gemm_decode_range_edges():
    """The largest and smallest decoded magnitudes, 6 * 448 = 2688 and 0.5 * 2^-9 = 2^-10
    (E4M3 codes 126 and 1), in every combination and both signs: the decode keeps them
    exact, so each output is an exact sum that the oracle reproduces."""
    m, n, k = 256, 256, 256
    rng = np.random.default_rng(77)
    big, small = 0x7, 0x1                                   # E2M1 codes of 6 and 0.5
    def operand(rows):
        nib = np.where(rng.random((rows, k)) < 0.5, big, small).astype(np.uint8)
        nib |= (rng.random((rows, k)) < 0.5).astype(np.uint8) << 3          # sign bit
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales = np.where(rng.random((rows, k // 16)) < 0.5, 126, 1).astype(np.uint8)
        return codes, scales
    ac, as_ = operand(m)
    bc, bs = operand(n)
    ga, gb = np.float32(1.0), np.float32(1.0)
    print(f"nvfp4 gemm decode range edges m={m} n={n} k={k}", flush=True)
    got = _nv_gemm(ac, as_, ga, bc, bs, gb)
    exact, cabs = oracle.gemm_nvfp4(ac, as_, ga, bc, bs, gb)
    _nv_check(got, exact, cabs, k)


def test_nvfp4_gemm_wgrad_after_rht_end_to_end():
    """Wgrad = dY^T X from the column-wise NVFP4 operands after the 128-token RHT
    (SR for the gradient, RTN for the activation): the product matches the oracle on the
    library's own codes, and tracks the exact dY^T X, as H H^T = I promises."""
    tokens, nout, nin = 1024, 256, 384
    g_bits = si.wgrad_gradient(tokens, nout, seed=4)
    x_bits = si.activation(tokens, nin, seed=5)
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(DEV)
    signs = B.fp4q_rht_signs_from_seed(4)
    qg = B.quantize_nvfp4(to_dev(g_bits), B.COLWISE, rnd=B.SR, sr_seed=40, rht_signs=signs)
    qx = B.quantize_nvfp4(to_dev(x_bits), B.COLWISE, rnd=B.RTN, rht_signs=signs)
    w = B.gemm_nvfp4(qg["col_codes"], qg["col_scales"], qg["tensor_scale"],
                     qx["col_codes"], qx["col_scales"], qx["tensor_scale"]).cpu().numpy().astype(np.float64)
    h = lambda t: t.cpu().numpy()
    exact, cabs = oracle.gemm_nvfp4(h(qg["col_codes"]), h(qg["col_scales"]), float(h(qg["tensor_scale"])[0]),
                                    h(qx["col_codes"]), h(qx["col_scales"]), float(h(qx["tensor_scale"])[0]))
    _nv_check(w, exact, cabs, tokens)
    f32 = lambda b: (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = f32(g_bits).T @ f32(x_bits)
    rel = np.linalg.norm(w - ref) / np.linalg.norm(ref)
    assert rel < 0.2, rel


@pytest.mark.parametrize("shape,tiles,bf16", [((256, 256, 128), 2, False), ((304, 528, 384), 1, False),
                                              ((256, 256, 256), 3, True), ((272, 160, 512), 2, True),
                                              ((16, 16, 128), 3, False), ((257, 144, 256), 2, False)])
def test_nvfp4_gemm_with_16x16_scale_tiles(shape, tiles, bf16):
    """Operands carrying one E4M3 scale per 16x16 tile, [rows/16][k/16]: the kernel reads
    tile row r // 16 for row r, across ragged M/N edges and several K tiles."""
    m, n, k = shape
    rng = np.random.default_rng(m * 3 + n * 7 + k + tiles)
    ac, as_ = _nv_operand(rng, m, k)
    bc, bs = _nv_operand(rng, n, k)
    if tiles & 1:
        as_ = as_[: m // 16].copy()
    if tiles & 2:
        bs = bs[: n // 16].copy()
    ga, gb = np.float32(3.0), np.float32(0.375)
    print(f"nvfp4 gemm tiles={tiles} m={m} n={n} k={k} bf16={bf16}", flush=True)
    got = _nv_gemm(ac, as_, ga, bc, bs, gb, torch.bfloat16 if bf16 else torch.float32, tiles)
    exact, cabs = oracle.gemm_nvfp4(ac, as_, ga, bc, bs, gb, flags=tiles)
    _nv_check(got, exact, cabs, k, bf16)


def test_nvfp4_forward_and_dgrad_with_2d_weight_end_to_end():
    """Y = X W^T with W quantized in 16x16 tiles by the library, and dX = dY W with the
    library's 16x16 quantization of W^T: both products match the oracle on the library's
    own operands, and W^T's tiles are the transposed tile array of W."""
    m, n, k = 256, 384, 512
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(DEV)
    x_bits = si.activation(m, k, seed=51)
    w = torch.from_numpy(si.weight(n, k, seed=52, std=0.02)).to(DEV)
    dy_bits = si.activation(m, n, seed=53)
    qx = B.quantize_nvfp4(to_dev(x_bits), B.ROWWISE)
    qw = B.quantize_nvfp4_2d(w, transposed=True)
    qwt = B.quantize_nvfp4_2d(w.t().contiguous())
    qd = B.quantize_nvfp4(to_dev(dy_bits), B.ROWWISE)
    h = lambda t: t.cpu().numpy()
    # one quantization of W serves both products: W^T's codes and tiles are W's transposed
    assert np.array_equal(h(qwt["scales"]), h(qw["scales"]).T)
    assert np.array_equal(h(qwt["codes"]), h(qw["codes_t"]))
    y = B.gemm_nvfp4(qx["row_codes"], qx["row_scales"], qx["tensor_scale"], qw["codes"], qw["scales"],
                     qw["tensor_scale"], operand_flags=B.TILES_B)
    dx = B.gemm_nvfp4(qd["row_codes"], qd["row_scales"], qd["tensor_scale"], qwt["codes"], qwt["scales"],
                      qwt["tensor_scale"], operand_flags=B.TILES_B)
    for got, (a, b) in ((y, (qx, qw)), (dx, (qd, qwt))):
        exact, cabs = oracle.gemm_nvfp4(h(a["row_codes"]), h(a["row_scales"]), float(h(a["tensor_scale"])[0]),
                                        h(b["codes"]), h(b["scales"]), float(h(b["tensor_scale"])[0]), flags=2)
        _nv_check(got.cpu().numpy().astype(np.float64), exact, cabs, a["row_codes"].shape[1] * 2)


def test_nvfp4_gemm_full_size_sampled():
    m = n = k = 8192
    rng = np.random.default_rng(9)
    ac, as_ = _nv_operand(rng, m, k)
    bc, bs = _nv_operand(rng, n, k)
    ga, gb = np.float32(50.0), np.float32(3.0)
    print("nvfp4 gemm full size", flush=True)
    c = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    ta = torch.tensor([ga], device=DEV)
    tb = torch.tensor([gb], device=DEV)
    B.fp4q_gemm_nvfp4(_dev(ac), _dev(as_), ta, _dev(bc), _dev(bs), tb, m, n, k, 0, B.BF16, c)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 256, 4095, 8190, 8191])
    cols = np.array([0, 31, 32, 255, 256, 4096, 8191])
    exact, cabs = oracle.gemm_nvfp4(ac[rows], as_[rows], ga, bc[cols], bs[cols], gb)
    got = c[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy()
    _nv_check(got.astype(np.float64), exact, cabs, k, bf16=True)


# --- output amax from the GEMM epilogue ---------------------------------------------

def _run_with_amax(kind, m, n, k, bf16, rng, amax):
    dt = torch.bfloat16 if bf16 else torch.float32
    c = torch.full((m, n), float("nan"), dtype=dt, device=DEV)
    if kind == "mx":
        ac, as_ = _operand(rng, m, k)
        bc, bs = _operand(rng, n, k)
        args = (_dev(ac), _dev(as_), _dev(bc), _dev(bs), m, n, k, B._dt(c), c)
        B.fp4q_gemm_mxfp4(*args, amax)
        exact, cabs = oracle.gemm_mxfp4(ac, as_, bc, bs)
    else:
        ac, as_ = _nv_operand(rng, m, k)
        bc, bs = _nv_operand(rng, n, k)
        ta = torch.tensor([37.5], device=DEV)
        tb = torch.tensor([2.25], device=DEV)
        args = (_dev(ac), _dev(as_), ta, _dev(bc), _dev(bs), tb, m, n, k, 0, B._dt(c), c)
        B.fp4q_gemm_nvfp4(*args, amax)
        exact, cabs = oracle.gemm_nvfp4(ac, as_, np.float32(37.5), bc, bs, np.float32(2.25))
    torch.cuda.synchronize()
    # the same call without amax stores the same C
    c2 = torch.full_like(c, float("nan"))
    (B.fp4q_gemm_mxfp4 if kind == "mx" else B.fp4q_gemm_nvfp4)(*args[:-1], c2)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16 if bf16 else torch.int32), c2.view(torch.int16 if bf16 else torch.int32))
    got = c.float().cpu().numpy().astype(np.float64)
    (_check if kind == "mx" else _nv_check)(got, exact, cabs, k, bf16)
    return got


@pytest.mark.parametrize("kind", ["mx", "nv"])
@pytest.mark.parametrize("bf16", [False, True])
def test_gemm_amax_is_max_abs_of_the_stored_output(kind, bf16):
    """The amax the epilogue posts equals max |C| over exactly the stored m x n outputs
    (after the bf16 rounding); a second call on the same word, with a smaller product,
    starts again from zero."""
    rng = np.random.default_rng(71 + bf16 + 2 * (kind == "nv"))
    amax = torch.full((1,), 1e30, dtype=torch.float32, device=DEV)
    for m, n, k in [(300, 520, 384), (257, 130, 256), (1, 1, 128)]:
        print(f"gemm amax {kind} bf16={bf16} m={m} n={n} k={k}", flush=True)
        got = _run_with_amax(kind, m, n, k, bf16, rng, amax)
        assert amax.item() == np.abs(got).max(), (amax.item(), np.abs(got).max())


def test_gemm_amax_feeds_the_nvfp4_quantization_of_its_output():
    """C from the MXFP4 GEMM with its epilogue amax, quantized to NVFP4 with that amax
    given, is bit-identical to the quantization that computes the amax from C, and to the
    oracle's quantization of C."""
    m, n, k = 512, 384, 512
    x = si.weight(m, k, seed=31, std=1.0)
    w = si.weight(n, k, seed=32, std=0.05)
    qa = B.quantize_mxfp4(torch.from_numpy(x).to(DEV))
    qb = B.quantize_mxfp4(torch.from_numpy(w).to(DEV))
    amax = torch.empty(1, dtype=torch.float32, device=DEV)
    print("gemm amax -> nvfp4 quantize", flush=True)
    c = B.gemm_mxfp4(qa, qb, out_dtype=torch.bfloat16, amax=amax)
    given = B.quantize_nvfp4(c, B.ROWWISE | B.COLWISE, amax=amax)
    computed = B.quantize_nvfp4(c, B.ROWWISE | B.COLWISE)
    torch.cuda.synchronize()
    assert given["amax"].item() == computed["amax"].item()
    for key in ("tensor_scale", "row_codes", "row_scales", "col_codes", "col_scales"):
        assert torch.equal(given[key], computed[key]), key
    rc, rs, gs = oracle.quantize_nvfp4(c.float().cpu().numpy())
    assert np.array_equal(given["row_codes"].cpu().numpy(), rc)
    assert np.array_equal(given["row_scales"].cpu().numpy(), rs)
    assert given["tensor_scale"].item() == float(gs)


def test_gemm_amax_full_size_launch():
    """At 8192^3 with bf16 output (the measured launch), the epilogue amax equals the
    largest magnitude of the stored product (a property that holds at any size)."""
    m = n = k = 8192
    rng = np.random.default_rng(5)
    ac, as_ = _operand(rng, m, k)
    bc, bs = _operand(rng, n, k)
    c = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    amax = torch.full((1,), -1.0, device=DEV)
    print("gemm amax full size", flush=True)
    B.fp4q_gemm_mxfp4(_dev(ac), _dev(as_), _dev(bc), _dev(bs), m, n, k, B.BF16, c, amax)
    torch.cuda.synchronize()
    assert amax.item() == c.float().abs().max().item()


# --- IF4 operands -------------------------------------------------------------------
# An IF4 operand's INT4 element e = fl(fl(q fl(6/7)) s) reaches the bf16 MFMA as
# hi + lo (hi = bf16(e), lo = bf16(e - hi)): two bf16 roundings of at most 2^-8 each
# after e's fp32 rounding put hi + lo within d = 2^-16 + 2^-23 of the exact element
# (2^-23 also covering the product of the small terms).  One IF4 operand: each product
# term within d |a b|.  Both: (1 + d)^2 - 1 plus the omitted lo x lo (at most about
# 2^-16 |a b|), below 3 d.  Each K block then takes 1 + (IF4 operands) MFMAs, which
# lengthens the fp32 accumulation chain by that factor.

def _if4_operand(rng, rows, k, int_share=0.5):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(1, 127, size=(rows, k // 16), dtype=np.uint8)
    flags = (rng.random(size=scales.shape) < int_share).astype(np.uint8) << 7
    return codes, scales | flags


def _if4_check(got, exact, cabs, k, nif4, bf16=False):
    d = 2.0 ** -16 + 2.0 ** -23
    split = d if nif4 == 1 else 3.0 * d
    tol = (2.0 * (4 + (1 + nif4) * k / 16) * 2.0 ** -24 + split) * cabs + 3.0 * 2.0 ** -24 * np.abs(exact)
    if bf16:
        tol = tol + 2.0 ** -8 * (np.abs(exact) + tol)
    err = np.abs(got - exact)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, (f"{len(bad)} of {err.size} outside the bound; first {bad[:4].tolist()}, "
                           f"err {err[tuple(bad[0])]:.3e} tol {tol[tuple(bad[0])]:.3e}")


@pytest.mark.parametrize("shape,flags,bf16", [((256, 256, 128), 4, False), ((300, 520, 384), 8, False),
                                              ((257, 129, 256), 12, False), ((1, 1, 128), 12, False),
                                              ((390, 200, 512), 4, True), ((513, 768, 1024), 12, True),
                                              ((64, 2048, 2048), 8, True), ((272, 160, 512), 1 | 8, False),
                                              ((256, 304, 384), 4 | 2, True)])
def test_if4_gemm_random_codes(shape, flags, bf16):
    """IF4 x NVFP4, NVFP4 x IF4 and IF4 x IF4 on random codes with about half the blocks
    flagged INT4, across ragged M/N edges and several K steps; also an IF4 operand against
    a 16x16-tiled NVFP4 one (flags 9 and 6)."""
    m, n, k = shape
    rng = np.random.default_rng(m * 13 + n * 5 + k + flags)
    ac, as_ = (_if4_operand if flags & 4 else _nv_operand)(rng, m, k)
    bc, bs = (_if4_operand if flags & 8 else _nv_operand)(rng, n, k)
    if flags & 1:
        as_ = as_[: m // 16].copy()
    if flags & 2:
        bs = bs[: n // 16].copy()
    ga, gb = np.float32(41.75), np.float32(0.6875)
    print(f"if4 gemm flags={flags} m={m} n={n} k={k} bf16={bf16}", flush=True)
    got = _nv_gemm(ac, as_, ga, bc, bs, gb, torch.bfloat16 if bf16 else torch.float32, flags)
    exact, cabs = oracle.gemm_nvfp4(ac, as_, ga, bc, bs, gb, flags=flags)
    _if4_check(got, exact, cabs, k, bin(flags >> 2).count("1"), bf16)


def test_if4_gemm_without_int4_blocks_is_the_nvfp4_product():
    """With no block flagged the IF4 path stores bit-identical outputs to the NVFP4 path."""
    m, n, k = 320, 288, 512
    rng = np.random.default_rng(77)
    ac, as_ = _if4_operand(rng, m, k, int_share=0.0)
    bc, bs = _if4_operand(rng, n, k, int_share=0.0)
    ref = _nv_gemm(ac, as_, 5.0, bc, bs, 0.5)
    for flags in (4, 8, 12):
        assert np.array_equal(_nv_gemm(ac, as_, 5.0, bc, bs, 0.5, flags=flags), ref), flags


def test_if4_gemm_of_quantizer_outputs_end_to_end():
    """Y = X W^T from fp4q_quantize_if4 of a bf16 activation and an fp32 weight: the product
    matches the oracle on the library's own codes and tracks the float product."""
    m, n, k = 256, 320, 1024
    x_bits = si.activation(m, k, seed=81)
    w = si.weight(n, k, seed=82, std=0.02)
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(DEV)
    qx = B.quantize_if4(to_dev(x_bits))
    qw = B.quantize_if4(torch.from_numpy(w).to(DEV))
    h = lambda t: t.cpu().numpy()
    assert (h(qx["scales"]) & 0x80).any() and (h(qw["scales"]) & 0x80).any()
    y = B.gemm_nvfp4(qx["codes"], qx["scales"], qx["tensor_scale"], qw["codes"], qw["scales"], qw["tensor_scale"],
                     operand_flags=B.IF4_A | B.IF4_B).cpu().numpy().astype(np.float64)
    exact, cabs = oracle.gemm_nvfp4(h(qx["codes"]), h(qx["scales"]), float(h(qx["tensor_scale"])[0]),
                                    h(qw["codes"]), h(qw["scales"]), float(h(qw["tensor_scale"])[0]), flags=12)
    _if4_check(y, exact, cabs, k, 2)
    f32 = lambda b: (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = f32(x_bits) @ w.astype(np.float64).T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.15


@pytest.mark.parametrize("bf16", [False, True])
def test_if4_gemm_amax_is_max_abs_of_the_stored_output(bf16):
    """The epilogue amax with IF4 operands (their own kernel instances): it equals max |C|
    over the stored outputs, and C is the same with and without it."""
    m, n, k = 288, 352, 640
    rng = np.random.default_rng(91 + bf16)
    ac, as_ = _if4_operand(rng, m, k)
    bc, bs = _if4_operand(rng, n, k)
    dt = torch.bfloat16 if bf16 else torch.float32
    ta = torch.tensor([7.5], device=DEV)
    tb = torch.tensor([0.25], device=DEV)
    amax = torch.full((1,), float("nan"), device=DEV)
    c = torch.full((m, n), float("nan"), dtype=dt, device=DEV)
    c2 = torch.full_like(c, float("nan"))
    args = (_dev(ac), _dev(as_), ta, _dev(bc), _dev(bs), tb, m, n, k, B.IF4_A | B.IF4_B, B._dt(c))
    B.fp4q_gemm_nvfp4(*args, c, amax)
    B.fp4q_gemm_nvfp4(*args, c2)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16 if bf16 else torch.int32), c2.view(torch.int16 if bf16 else torch.int32))
    assert amax.item() == c.float().abs().max().item()
    exact, cabs = oracle.gemm_nvfp4(ac, as_, np.float32(7.5), bc, bs, np.float32(0.25), flags=12)
    _if4_check(c.float().cpu().numpy().astype(np.float64), exact, cabs, k, 2, bf16)
