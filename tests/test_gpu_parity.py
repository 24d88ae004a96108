"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer outputs (codes, scales, IF4 flags) must match bit for bit; amax and the
tensor scale exactly; dequantized values at 0 ULP.  The random Hadamard transform
runs on MFMA with fp32 accumulation, so its values are held to a 1e-5 relative
tolerance (per 128-value chunk column, relative to the column's RMS), while the
quantization that follows must match the oracle bit for bit when the oracle is fed
the library's own transform output (two-stage check).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from block_scaled_fp4_05_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def make_input(kind: str, rows: int, cols: int, seed: int = 0):
    """Returns (host array for the oracle, device tensor)."""
    if kind == "bf16":
        bits = si.activation(rows, cols, seed=seed)
        return bits, dev_bf16(bits)
    x = si.weight(rows, cols, seed=seed, std=1.0)
    x[:, ::7] *= np.float32(25.0)
    return x, dev_f32(x)


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------------------------------
# NVFP4 1x16
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(256, 512), (272, 400), (16, 16), (1040, 144)])
def test_nvfp4_row_and_col_rtn(kind, shape):
    rows, cols = shape
    xh, xd = make_input(kind, rows, cols, seed=rows + cols)
    out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE)
    rc, rs, gs = oracle.quantize_nvfp4(xh)
    cc, cs, _ = oracle.quantize_nvfp4(xh, colwise=True)
    assert host(out["amax"])[0] == np.float32(oracle.amax(xh))
    assert host(out["tensor_scale"])[0] == gs
    assert np.array_equal(host(out["row_codes"]), rc)
    assert np.array_equal(host(out["row_scales"]), rs)
    assert np.array_equal(host(out["col_codes"]), cc)
    assert np.array_equal(host(out["col_scales"]), cs)


@pytest.mark.parametrize("shape", [(37, 96), (1, 16), (129, 272)])
def test_nvfp4_rowwise_ragged_rows(shape):
    rows, cols = shape
    xh, xd = make_input("bf16", rows, cols, seed=3)
    out = B.quantize_nvfp4(xd, B.ROWWISE)
    rc, rs, gs = oracle.quantize_nvfp4(xh)
    assert np.array_equal(host(out["row_codes"]), rc)
    assert np.array_equal(host(out["row_scales"]), rs)


@pytest.mark.parametrize("shape", [(64, 40), (160, 8), (48, 136)])
def test_nvfp4_colwise_only(shape):
    rows, cols = shape
    xh, xd = make_input("f32", rows, cols, seed=5)
    out = B.quantize_nvfp4(xd, B.COLWISE)
    cc, cs, gs = oracle.quantize_nvfp4(xh, colwise=True)
    assert host(out["tensor_scale"])[0] == gs
    assert np.array_equal(host(out["col_codes"]), cc)
    assert np.array_equal(host(out["col_scales"]), cs)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_nvfp4_stochastic_rounding_matches_philox_oracle(kind):
    rows, cols = 272, 384
    xh, xd = make_input(kind, rows, cols, seed=11)
    seed = 0x1234_5678_9ABC
    out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, rnd=B.SR, sr_seed=seed)
    rc, rs, gs = oracle.quantize_nvfp4(xh, rnd=oracle.SR, seed=seed)
    cc, cs, _ = oracle.quantize_nvfp4(xh, colwise=True, rnd=oracle.SR, seed=seed)
    assert np.array_equal(host(out["row_codes"]), rc)
    assert np.array_equal(host(out["row_scales"]), rs)
    assert np.array_equal(host(out["col_codes"]), cc)
    assert np.array_equal(host(out["col_scales"]), cs)
    # same seed -> same bits; another seed -> different draws
    again = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, rnd=B.SR, sr_seed=seed)
    assert torch.equal(again["row_codes"], out["row_codes"])
    # another seed: among the elements whose SR code differs from the nearest code
    # (where the draw decided), about 2/3 change again under an independent draw
    # (E[1 - f] over f uniform on (0, 1/2), and symmetrically above); at least 40 %
    other = B.quantize_nvfp4(xd, B.ROWWISE, rnd=B.SR, sr_seed=seed + 1)
    rn, _, _ = oracle.quantize_nvfp4(xh)

    def nib(c):
        return np.stack([c & 15, c >> 4], -1).reshape(-1)
    affected = nib(rc) != nib(rn)
    changed = nib(host(other["row_codes"])) != nib(rc)
    assert affected.sum() > 1000
    assert changed[affected].mean() >= 0.40, changed[affected].mean()


def test_nvfp4_amax_given():
    rows, cols = 64, 128
    xh, xd = make_input("bf16", rows, cols, seed=2)
    given = torch.tensor([4.0 * oracle.amax(xh)], dtype=torch.float32, device=DEV)
    out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, amax=given)
    gs = oracle.tensor_scale(float(host(given)[0]))
    rc, rs, _ = oracle.quantize_nvfp4(xh, gs=gs)
    cc, cs, _ = oracle.quantize_nvfp4(xh, colwise=True, gs=gs)
    assert host(out["tensor_scale"])[0] == np.float32(gs)
    assert np.array_equal(host(out["row_codes"]), rc) and np.array_equal(host(out["row_scales"]), rs)
    assert np.array_equal(host(out["col_codes"]), cc) and np.array_equal(host(out["col_scales"]), cs)


def test_nvfp4_degenerate_inputs():
    # all zeros: amax 0 -> gs 1, every code and scale 0
    z = np.zeros((32, 32), np.float32)
    out = B.quantize_nvfp4(dev_f32(z), B.ROWWISE | B.COLWISE)
    assert host(out["tensor_scale"])[0] == 1.0
    assert not host(out["row_codes"]).any() and not host(out["col_codes"]).any()
    # signed zeros, zero-scale blocks (tiny values next to a large one) and huge values
    x = np.zeros((32, 64), np.float32)
    x[0, 0] = 3.0e38
    x[1, :] = -0.0
    x[2, 16:32] = np.float32(1e-30) * np.tile([1, -1], 8)
    x[3, 32:48] = -np.float32(1e-3)
    x[5:, :] = si.weight(27, 64, seed=1)
    for lay, colwise in ((B.ROWWISE, False), (B.COLWISE, True)):
        out = B.quantize_nvfp4(dev_f32(x), lay)
        c, s, gs = oracle.quantize_nvfp4(x, colwise=colwise)
        key = "col" if colwise else "row"
        assert np.array_equal(host(out[key + "_codes"]), c)
        assert np.array_equal(host(out[key + "_scales"]), s)


def _exact_given_amax(xh):
    return torch.tensor([oracle.amax(xh)], dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(256, 512), (272, 400), (1040, 144), (16, 16)])
@pytest.mark.parametrize("rnd", [0, 1])
def test_nvfp4_two_pass_streaming_kernel(kind, shape, rnd):
    """AMAX_GIVEN skips the one-pass kernel: the streaming tile kernel alone, ragged tiles included."""
    rows, cols = shape
    xh, xd = make_input(kind, rows, cols, seed=rows * 3 + cols)
    seed = 0xBEEF + rows
    out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, rnd=rnd, sr_seed=seed, amax=_exact_given_amax(xh))
    rc, rs, gs = oracle.quantize_nvfp4(xh, rnd=rnd, seed=seed)
    cc, cs, _ = oracle.quantize_nvfp4(xh, colwise=True, rnd=rnd, seed=seed)
    assert host(out["tensor_scale"])[0] == gs
    assert np.array_equal(host(out["row_codes"]), rc) and np.array_equal(host(out["row_scales"]), rs)
    assert np.array_equal(host(out["col_codes"]), cc) and np.array_equal(host(out["col_scales"]), cs)


@pytest.mark.parametrize("layouts", [3, 1, 2])
def test_nvfp4_one_pass_mid_size(layouts):
    """4000 x 2608 bf16 (32 x 21 tiles, ragged on both edges): more tiles than one per workgroup."""
    rows, cols = 4000, 2608
    xh, xd = make_input("bf16", rows, cols, seed=17)
    out = B.quantize_nvfp4(xd, layouts)
    if layouts & B.ROWWISE:
        rc, rs, gs = oracle.quantize_nvfp4(xh)
        assert np.array_equal(host(out["row_codes"]), rc) and np.array_equal(host(out["row_scales"]), rs)
    if layouts & B.COLWISE:
        cc, cs, gs = oracle.quantize_nvfp4(xh, colwise=True)
        assert np.array_equal(host(out["col_codes"]), cc) and np.array_equal(host(out["col_scales"]), cs)
    assert host(out["amax"])[0] == np.float32(oracle.amax(xh))
    assert host(out["tensor_scale"])[0] == gs


def test_nvfp4_one_pass_repeated_launches_agree():
    """The grid barrier is reused launch after launch; results must not depend on it."""
    rows, cols = 1024, 2048
    xh, xd = make_input("bf16", rows, cols, seed=23)
    first = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE)
    for _ in range(5):
        again = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE)
        for k in ("row_codes", "row_scales", "col_codes", "col_scales", "amax", "tensor_scale"):
            assert torch.equal(again[k], first[k])
    rc, rs, gs = oracle.quantize_nvfp4(xh)
    assert np.array_equal(host(first["row_codes"]), rc)


@pytest.mark.parametrize("shape", [(1024, 2048), (4000, 2608), (8192, 4096)])
def test_nvfp4_one_pass_grid_resident_no_fallback(shape):
    """At the default wait limit the sized-to-fit grid is resident: no workgroup reads x twice."""
    rows, cols = shape
    xh, xd = make_input("bf16", rows, cols, seed=31)
    s = torch.cuda.Stream()
    ws = B.Workspace()
    with torch.cuda.stream(s):
        before = B.fp4q_workspace_fallbacks(ws, stream=s)
        out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, ws=ws, stream=s)
        after = B.fp4q_workspace_fallbacks(ws, stream=s)
    s.synchronize()
    ws.close()
    assert after == before
    assert host(out["amax"])[0] == np.float32(oracle.amax(xh))


@pytest.mark.parametrize("shape", [(1024, 2048), (2048, 4096)])
def test_nvfp4_one_pass_forced_fallback_is_exact(shape):
    """Wait limit 0: every wait gives up at once and the workgroup reads the missing part of
    x itself; codes, scales and amax must still match the oracle bit for bit."""
    rows, cols = shape
    xh, xd = make_input("bf16", rows, cols, seed=37)
    s = torch.cuda.Stream()
    ws = B.Workspace()
    B.fp4q_workspace_set_wait(ws, 0)
    with torch.cuda.stream(s):
        before = B.fp4q_workspace_fallbacks(ws, stream=s)
        out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, ws=ws, stream=s)
        after = B.fp4q_workspace_fallbacks(ws, stream=s)
    s.synchronize()
    ws.close()
    assert after > before
    rc, rs, gs = oracle.quantize_nvfp4(xh)
    cc, cs, _ = oracle.quantize_nvfp4(xh, colwise=True)
    assert host(out["amax"])[0] == np.float32(oracle.amax(xh))
    assert host(out["tensor_scale"])[0] == gs
    assert np.array_equal(host(out["row_codes"]), rc) and np.array_equal(host(out["row_scales"]), rs)
    assert np.array_equal(host(out["col_codes"]), cc) and np.array_equal(host(out["col_scales"]), cs)


def test_nvfp4_beyond_one_grid_falls_back_sampled():
    """bf16 [16384 x 4096] has more tiles than one co-resident grid holds: amax pass + streaming pass."""
    bits = si.activation(16384, 4096, seed=29)
    xd = dev_bf16(bits)
    out = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE)
    amax = oracle.amax(bits)
    gs = oracle.tensor_scale(amax)
    assert host(out["amax"])[0] == np.float32(amax)
    assert host(out["tensor_scale"])[0] == np.float32(gs)
    rcg, rsg = host(out["row_codes"]), host(out["row_scales"])
    ccg, csg = host(out["col_codes"]), host(out["col_scales"])
    for r0 in (0, 8192, 16368):
        c, s = oracle.quantize_nvfp4_rows(bits, r0, 16, False, gs)
        assert np.array_equal(rcg[r0:r0 + 16], c) and np.array_equal(rsg[r0:r0 + 16], s)
    for j0 in (0, 2056, 4088):
        c, s = oracle.quantize_nvfp4_rows(bits, j0, 8, True, gs)
        assert np.array_equal(ccg[j0:j0 + 8], c) and np.array_equal(csg[j0:j0 + 8], s)


@pytest.mark.parametrize("kind,shape", [("f32", (8193, 4099)), ("bf16", (16385, 4097)), ("bf16", (37, 61)),
                                        ("f32", (3, 5))])
def test_amax_entry_point_small_and_wide_with_tails(kind, shape):
    """fp4q_amax on sizes below and above the wide-kernel threshold (128 MB), with element
    counts that leave a tail after the 16-byte vectors; the largest magnitude is planted
    in the tail, in the body, and compared with the oracle's exact amax."""
    rows, cols = shape
    rng = np.random.default_rng(rows)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x.reshape(-1)[-1] = -37.5          # tail element
    x.reshape(-1)[rows * cols // 3] = 41.25 if rows * cols > 64 else x.reshape(-1)[0]
    if kind == "bf16":
        bits = si.f32_to_bf16_bits(x)
        xh, xd = bits, dev_bf16(bits)
    else:
        xh, xd = x, dev_f32(x)
    a = B.amax(xd)
    assert host(a)[0] == np.float32(oracle.amax(xh))


# ---------------------------------------------------------------------------------------
# NVFP4 16x16
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(96, 160), (16, 16), (528, 272)])
def test_nvfp4_2d_and_transposed_codes(kind, shape):
    rows, cols = shape
    xh, xd = make_input(kind, rows, cols, seed=7)
    out = B.quantize_nvfp4_2d(xd, transposed=True)
    c, s, gs = oracle.quantize_nvfp4_2d(xh)
    ct, st, _ = oracle.quantize_nvfp4_2d(np.ascontiguousarray(xh.T))
    assert host(out["tensor_scale"])[0] == gs
    assert np.array_equal(host(out["codes"]), c)
    assert np.array_equal(host(out["scales"]), s)
    assert np.array_equal(host(out["codes_t"]), ct)
    assert np.array_equal(st, s.T)


# ---------------------------------------------------------------------------------------
# MXFP4
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("rnd", [0, 1])
def test_mxfp4(kind, rnd):
    rows, cols = 96, 320
    xh, xd = make_input(kind, rows, cols, seed=13)
    out = B.quantize_mxfp4(xd, rnd=rnd, sr_seed=99)
    c, s = oracle.quantize_mxfp4(xh, rnd=rnd, seed=99)
    assert np.array_equal(host(out["codes"]), c)
    assert np.array_equal(host(out["scales"]), s)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 32), (96, 320), (1000, 1024), (4100, 4096)])
def test_mxfp4_reports_tensor_amax(kind, shape):
    # from 1 workgroup to about 4 K (128 spread lines, up to 33 posts each); the amax
    # equals the oracle's and the codes do not change when it is requested
    rows, cols = shape
    xh, xd = make_input(kind, rows, cols, seed=17)
    out = B.quantize_mxfp4(xd, with_amax=True)
    assert host(out["amax"])[0] == np.float32(oracle.amax(xh))
    if rows * cols <= 96 * 320:
        c, s = oracle.quantize_mxfp4(xh)
        assert np.array_equal(host(out["codes"]), c) and np.array_equal(host(out["scales"]), s)
    plain = B.quantize_mxfp4(xd)
    assert torch.equal(plain["codes"], out["codes"]) and torch.equal(plain["scales"], out["scales"])


def test_mxfp4_amax_does_not_leak_between_calls():
    # a later call with a smaller maximum, and one over fewer workgroups than spread
    # lines, must not see the earlier call's posts
    big = si.weight(2048, 2048, seed=21)
    big[77, 5] = np.float32(123.0)
    small = si.weight(16, 64, seed=22)
    assert B.quantize_mxfp4(dev_f32(big), with_amax=True)["amax"].item() == np.float32(123.0)
    got = B.quantize_mxfp4(dev_f32(small), with_amax=True)["amax"].item()
    assert got == np.float32(oracle.amax(small))
    z = np.zeros((8, 64), np.float32)
    assert B.quantize_mxfp4(dev_f32(z), with_amax=True)["amax"].item() == 0.0


def test_mxfp4_extreme_blocks():
    x = np.zeros((4, 128), np.float32)
    x[0, :32] = np.float32(1e-39) * np.arange(1, 33, dtype=np.float32)   # subnormal block -> code 0 region
    x[1, :32] = 3.0e38
    x[1, 32:64] = 1.5 * 6.0                                                 # bamax/6 = 1.5 exactly: tie
    x[2, 64:96] = -0.0
    x[3, :] = si.weight(1, 128, seed=4)
    out = B.quantize_mxfp4(dev_f32(x))
    c, s = oracle.quantize_mxfp4(x)
    assert np.array_equal(host(out["scales"]), s)
    assert np.array_equal(host(out["codes"]), c)


# ---------------------------------------------------------------------------------------
# IF4
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(128, 256), (40, 48)])
def test_if4(shape):
    bits = si.if4_mix(*shape, seed=6)
    out = B.quantize_if4(dev_bf16(bits))
    c, s, gs = oracle.quantize_if4(bits)
    assert host(out["tensor_scale"])[0] == gs
    assert np.array_equal(host(out["scales"]), s)
    assert np.array_equal(host(out["codes"]), c)
    assert 0 < np.count_nonzero(s & 0x80) < s.size       # both block types occur


def test_if4_subnormal_scale_blocks():
    # Blocks whose E4M3 scale is subnormal (codes 1..7) can round far below bamax/6, so
    # their INT4 candidate needs the clamp to [-7, 7]; the kernel drops the clamp only in
    # waves without such blocks.  Rows 0..31 (workgroup 0) are all normal, rows 32..63
    # mix normal blocks with tiny ones placed to round their scale down.
    rng = np.random.default_rng(41)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[0, 0] = 100.0                                  # amax: gs = 26.88
    gs = np.float32(oracle.tensor_scale(100.0))
    for r in (33, 40, 47, 58):
        for cb in (0, 5, 17, 31):
            for k, y in enumerate((1.4, 1.9, 2.45, 5.3)):   # fl(bamax*gs)/6 = y * 2^-9
                if (cb + k) % 4 == 0:
                    m = np.float32(6.0 * y * 2.0 ** -9) / gs
                    blk = rng.uniform(-1.0, 1.0, 16).astype(np.float32) * m
                    blk[rng.integers(16)] = m
                    x[r, cb * 16:cb * 16 + 16] = blk
    bits = si.f32_to_bf16_bits(x)
    out = B.quantize_if4(dev_bf16(bits))
    c, s, g = oracle.quantize_if4(bits)
    assert host(out["tensor_scale"])[0] == g
    assert np.array_equal(host(out["scales"]), s)
    assert np.array_equal(host(out["codes"]), c)
    codes = s & 0x7F
    assert np.count_nonzero((codes >= 1) & (codes <= 7)) >= 8      # subnormal scales occur
    assert not np.any((codes[:32] >= 1) & (codes[:32] <= 7))       # workgroup 0 has none


# ---------------------------------------------------------------------------------------
# Dequantization
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["nvfp4", "nvfp4_2d", "mxfp4", "if4", "nvfp4_col"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_zero_ulp(fmt, out_dtype):
    rows, cols = 96, 256
    bits = si.if4_mix(rows, cols, seed=8)
    xd = dev_bf16(bits)
    if fmt == "nvfp4":
        q = B.quantize_nvfp4(xd, B.ROWWISE)
        args = (B.FMT_NVFP4, q["row_codes"], q["row_scales"], q["tensor_scale"], rows, cols)
    elif fmt == "nvfp4_col":
        q = B.quantize_nvfp4(xd, B.COLWISE)
        args = (B.FMT_NVFP4, q["col_codes"], q["col_scales"], q["tensor_scale"], cols, rows)
    elif fmt == "nvfp4_2d":
        q = B.quantize_nvfp4_2d(xd)
        args = (B.FMT_NVFP4_2D, q["codes"], q["scales"], q["tensor_scale"], rows, cols)
    elif fmt == "mxfp4":
        q = B.quantize_mxfp4(xd)
        args = (B.FMT_MXFP4, q["codes"], q["scales"], None, rows, cols)
    else:
        q = B.quantize_if4(xd)
        args = (B.FMT_IF4, q["codes"], q["scales"], q["tensor_scale"], rows, cols)
    f, codes, scales, ts, r, c = args
    gs = float(host(ts)[0]) if ts is not None else 1.0
    ref = oracle.dequantize(f, host(codes), host(scales), gs, r, c)
    if out_dtype == torch.float32:
        y = host(B.dequantize(*args))
        assert np.array_equal(f32_bits(y), f32_bits(ref))
    else:
        yb = host(B.dequantize(*args, out_dtype=torch.bfloat16).view(torch.int16)).view(np.uint16)
        assert np.array_equal(yb, si.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gs", [1.0, 3.7e-3, 0.6180339, 7.1e25, 2.3e-28, -2.5, 1.0e-40])
@pytest.mark.parametrize("fmt", ["nvfp4", "nvfp4_2d", "mxfp4", "if4"])
def test_dequantize_arbitrary_codes_and_tensor_scales(fmt, gs, out_dtype):
    """Every code byte, every finite E4M3 scale code (with and without the INT4 flag for
    IF4), every E8M0 code for MXFP4 (2^-127 and overflow included), and tensor scales
    that send blocks down both division paths: in range, so large or small that
    quotients leave the normal range, negative, subnormal.  Shapes include element
    counts that end inside a wave's span."""
    f = {"nvfp4": B.FMT_NVFP4, "nvfp4_2d": B.FMT_NVFP4_2D, "mxfp4": B.FMT_MXFP4, "if4": B.FMT_IF4}[fmt]
    shapes = {"nvfp4_2d": [(64, 512), (16, 272), (48, 80)],
              "mxfp4": [(64, 512), (16, 288), (3, 96)]}.get(fmt, [(64, 512), (16, 272), (3, 96)])
    rng = np.random.default_rng(97)
    gs32 = np.float32(gs)
    for rows, cols in shapes:
        codes = rng.integers(0, 256, size=rows * cols // 2, dtype=np.uint8)
        if fmt == "mxfp4":
            scales = rng.integers(0, 256, size=rows * cols // 32, dtype=np.uint8)
        elif fmt == "nvfp4_2d":
            scales = rng.integers(0, 0x7F, size=rows * cols // 256, dtype=np.uint8)  # 0x7F is NaN
        else:
            scales = rng.integers(0, 0x7F, size=rows * cols // 16, dtype=np.uint8)
        if fmt == "if4":
            scales |= (rng.integers(0, 2, size=scales.size, dtype=np.uint8) << 7).astype(np.uint8)
        ts = None if fmt == "mxfp4" else torch.tensor([gs32], dtype=torch.float32, device="cuda")
        ref = oracle.dequantize(f, codes, scales, float(gs32) if ts is not None else 1.0, rows, cols)
        args = (f, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), ts, rows, cols)
        if out_dtype == torch.float32:
            y = host(B.dequantize(*args))
            assert np.array_equal(f32_bits(y), f32_bits(ref)), (rows, cols)
        else:
            yb = host(B.dequantize(*args, out_dtype=torch.bfloat16).view(torch.int16)).view(np.uint16)
            assert np.array_equal(yb, si.f32_to_bf16_bits(ref)), (rows, cols)


# ---------------------------------------------------------------------------------------
# Random Hadamard transform
# ---------------------------------------------------------------------------------------

def rht_close(y: np.ndarray, ref: np.ndarray, tol: float = 1e-5) -> bool:
    """Per (128-row chunk, column): max |y - ref| <= tol * RMS(ref column chunk)."""
    rows, cols = ref.shape
    r = ref.reshape(rows // 128, 128, cols).astype(np.float64)
    d = np.abs(y.reshape(rows // 128, 128, cols).astype(np.float64) - r).max(axis=1)
    rms = np.sqrt((r ** 2).mean(axis=1))
    return bool(np.all(d <= tol * rms + 1e-30))


@pytest.mark.parametrize("kind", ["grad", "act"])
def test_rht_standalone_within_tolerance(kind):
    rows, cols = 384, 192
    bits = si.wgrad_gradient(rows, cols, seed=1) if kind == "grad" else si.wgrad_activation(rows, cols, seed=1)
    signs = oracle.rht_signs(4)
    y = host(B.rht(dev_bf16(bits), signs.tolist()))
    ref = oracle.rht(bits, signs)
    assert rht_close(y, ref)
    # inverse (bf16 MFMA path) and the f32 VALU path
    back = host(B.rht(dev_f32(ref), signs.tolist(), inverse=True))
    assert rht_close(back, si.bf16_bits_to_f32(bits))
    yf = host(B.rht(dev_f32(si.bf16_bits_to_f32(bits)), signs.tolist()))
    assert rht_close(yf, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(512, 256), (256, 200), (128, 72)])
@pytest.mark.parametrize("rnd", [0, 1])
def test_rht_fused_two_stage_exact(rnd, shape, dtype):
    """The fused RHT + column-wise NVFP4 equals the oracle quantizer fed with the
    library's own transform output (of the same dtype), bit for bit; against the
    all-oracle pipeline the codes may differ only at rounding ties.  Widths that are
    not a multiple of 64 leave a partial last column slab (bf16) or a partial last
    workgroup (fp32)."""
    rows, cols = shape
    if dtype == "bf16":
        bits = si.wgrad_gradient(rows, cols, seed=3)
        xd = dev_bf16(bits)
    else:
        bits = si.weight(rows, cols, seed=3, std=1e-3)
        xd = dev_f32(bits)
    signs = oracle.rht_signs(4)
    out = B.quantize_nvfp4(xd, B.COLWISE, rnd=rnd, sr_seed=40, rht_signs=signs.tolist())
    y = host(B.rht(xd, signs.tolist()))
    amax_g, gs_g = host(out["amax"])[0], host(out["tensor_scale"])[0]
    assert amax_g == np.max(np.abs(y))
    assert gs_g == np.float32(oracle.tensor_scale(float(amax_g)))
    c2, s2, _ = oracle.quantize_nvfp4(y, colwise=True, gs=float(gs_g), rnd=rnd, seed=40)
    assert np.array_equal(host(out["col_codes"]), c2)
    assert np.array_equal(host(out["col_scales"]), s2)
    # all-oracle pipeline
    yo = oracle.rht(bits, signs)
    assert rht_close(y, yo)
    c3, s3, _ = oracle.quantize_nvfp4(yo, colwise=True, rnd=rnd, seed=40)
    mism = np.count_nonzero(host(out["col_codes"]) != c3)
    assert mism <= max(1, int(c3.size * 2 * 1e-6))


# ---------------------------------------------------------------------------------------
# Two-pass calls: amax computed by a separate pass, or given by the caller
# ---------------------------------------------------------------------------------------

def _same_outputs(a: dict, b: dict):
    for k, v in a.items():
        if v is None or k == "amax":
            continue
        assert np.array_equal(host(v), host(b[k])), k


def test_given_amax_reproduces_computed_amax():
    """Each two-pass entry point, called with the amax its compute mode reported,
    produces the same tensor scale, codes and scales; the compute mode's amax is the
    exact maximum."""
    bits = si.if4_mix(256, 512, seed=31)
    xd = dev_bf16(bits)
    xf = dev_f32(si.bf16_bits_to_f32(bits))
    ref_amax = np.float32(np.max(np.abs(si.bf16_bits_to_f32(bits))))
    # 16x16 2D (fp32 and bf16) and IF4
    for fn, args in ((B.quantize_nvfp4_2d, (xf,)), (B.quantize_nvfp4_2d, (xd,)), (B.quantize_if4, (xd,))):
        c = fn(*args)
        assert host(c["amax"])[0] == ref_amax
        g = fn(*args, amax=c["amax"].clone())
        _same_outputs(c, g)
    # RHT + column-wise NVFP4 (SR)
    signs = oracle.rht_signs(4).tolist()
    c = B.quantize_nvfp4(xd, B.COLWISE, rnd=1, sr_seed=9, rht_signs=signs)
    assert host(c["amax"])[0] == host(B.rht(xd, signs).abs().max().reshape(1))[0]
    g = B.quantize_nvfp4(xd, B.COLWISE, rnd=1, sr_seed=9, rht_signs=signs, amax=c["amax"].clone())
    _same_outputs(c, g)


def test_two_pass_amax_does_not_leak_between_calls():
    """Two-pass calls on one stream share a workspace word: a call on a tensor with a
    small amax right after one with a large amax, through different entry points,
    still reports and uses its own amax."""
    big = si.if4_mix(256, 512, seed=32)
    small = si.f32_to_bf16_bits(si.bf16_bits_to_f32(big) * np.float32(1.0 / 1024.0))
    amax_big = np.float32(np.max(np.abs(si.bf16_bits_to_f32(big))))
    amax_small = np.float32(np.max(np.abs(si.bf16_bits_to_f32(small))))
    assert amax_small < amax_big
    signs = oracle.rht_signs(4).tolist()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(2):
            a = B.quantize_if4(dev_bf16(big), stream=s)
            b = B.quantize_nvfp4_2d(dev_bf16(small), stream=s)
            c = B.quantize_if4(dev_bf16(small), stream=s)
            d = B.quantize_nvfp4(dev_bf16(big), B.COLWISE, rht_signs=signs, stream=s)
            e = B.quantize_nvfp4(dev_bf16(small), B.COLWISE, rht_signs=signs, stream=s)
    s.synchronize()
    assert host(a["amax"])[0] == amax_big
    assert host(b["amax"])[0] == amax_small and host(c["amax"])[0] == amax_small
    assert host(e["amax"])[0] < host(d["amax"])[0]
    assert host(b["tensor_scale"])[0] == np.float32(oracle.tensor_scale(float(amax_small)))
    c_ref, s_ref, _ = oracle.quantize_if4(small)
    assert np.array_equal(host(c["codes"]), c_ref) and np.array_equal(host(c["scales"]), s_ref)


# ---------------------------------------------------------------------------------------
# Streams, determinism, guard bytes
# ---------------------------------------------------------------------------------------

def test_non_default_stream_and_guard_bytes():
    rows, cols = 128, 256
    xh, xd = make_input("bf16", rows, cols, seed=21)
    pad = 4096
    guard = lambda n: torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    rc, rs = guard(rows * cols // 2), guard(rows * cols // 16)
    cc, cs = guard(rows * cols // 2), guard(rows * cols // 16)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    ts = torch.zeros(1, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        B.fp4q_quantize_nvfp4(xd, B.BF16, rows, cols, B.ROWWISE | B.COLWISE, B.RTN, 0, None, B.AMAX_COMPUTE,
                              amax, ts, rc[pad:], rs[pad:], cc[pad:], cs[pad:], stream=s)
    s.synchronize()
    for t, n in ((rc, rows * cols // 2), (rs, rows * cols // 16), (cc, rows * cols // 2), (cs, rows * cols // 16)):
        h = host(t)
        assert np.all(h[:pad] == 0xA5) and np.all(h[pad + n:] == 0xA5)
    r_o, s_o, _ = oracle.quantize_nvfp4(xh)
    assert np.array_equal(host(rc)[pad:pad + rows * cols // 2].reshape(rows, cols // 2), r_o)
