"""GPU parity of MX FP6 (fp4q_quantize_mxfp6, fp4q_dequantize with the FP6 formats)
against the oracle: codes and scales bit for bit, dequantized values bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from block_scaled_fp4_05_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = [B.FP6_E2M3, B.FP6_E3M2]


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _input(kind, rows, cols, seed):
    if kind == "bf16":
        bits = si.activation(rows, cols, seed=seed)
        return bits, _dev_bf16(bits)
    x = si.weight(rows, cols, seed=seed, std=1.0)
    x[:, ::5] *= np.float32(40.0)
    return x, torch.from_numpy(x).to(DEV)


def _check(xh, xd, fmt):
    out = B.quantize_mxfp6(xd, fmt)
    torch.cuda.synchronize()
    c, s = oracle.quantize_mxfp6(xh, fmt)
    assert np.array_equal(out["scales"].cpu().numpy(), s)
    assert np.array_equal(out["codes"].cpu().numpy(), c)
    return c, s


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(256, 512), (272, 416), (1, 32), (1040, 160), (3, 96)])
def test_mxfp6_quantize_matches_oracle(fmt, kind, shape):
    rows, cols = shape
    xh, xd = _input(kind, rows, cols, seed=rows + cols)
    print(f"mxfp6 fmt={fmt} {kind} {shape}", flush=True)
    _check(xh, xd, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_mxfp6_edge_values(fmt):
    x = np.zeros((4, 128), dtype=np.float32)
    x[0, :32] = -0.0                                   # signed zeros, zero block
    x[1, :32] = np.linspace(-3e38, 3e38, 32)           # huge block: saturation and the top scale
    x[2, :32] = np.float32(1e-38) * np.arange(32)      # tiny block: subnormal inputs and low scales
    x[3] = np.random.default_rng(3).standard_normal(128).astype(np.float32) * np.float32(1e-30)
    x[0, 32:64] = np.float32(7.5) * np.arange(32) / 31  # on-grid and between-grid values
    x[1, 64:96] = np.float32(28.0) * (np.arange(32) - 16) / 16
    _check(x, torch.from_numpy(x).to(DEV), fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mxfp6_dequantize_matches_oracle(fmt, out_dtype):
    xh, xd = _input("f32", 300, 640, seed=7)
    c, s = _check(xh, xd, fmt)
    y = torch.empty(300, 640, dtype=out_dtype, device=DEV)
    B.fp4q_dequantize(B.FMT_MXFP6[fmt], torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV), None, 300, 640,
                      B._dt(y), y)
    torch.cuda.synchronize()
    ref = torch.from_numpy(oracle.dequantize_mxfp6(fmt, c, s, 300, 640))
    if out_dtype == torch.bfloat16:
        ref = ref.to(torch.bfloat16)
    assert torch.equal(y.cpu(), ref)


def test_mxfp6_full_weight_sampled():
    """fp32 [8192 x 8192] N(0, 0.02^2), both formats; sampled rows against the oracle."""
    w = si.weight(8192, 8192, seed=3)
    wd = torch.from_numpy(w).to(DEV)
    for fmt in FMTS:
        out = B.quantize_mxfp6(wd, fmt)
        torch.cuda.synchronize()
        codes, scales = out["codes"].cpu().numpy(), out["scales"].cpu().numpy()
        for r0 in (0, 4095, 8180):
            c, s = oracle.quantize_mxfp6(np.ascontiguousarray(w[r0:r0 + 12]), fmt)
            assert np.array_equal(codes[r0:r0 + 12], c) and np.array_equal(scales[r0:r0 + 12], s)
