"""CPU oracle for block-scaled FP4 quantization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never loads it and shares
no code with it.  The arithmetic lives in ``fp4q_oracle.c`` (plain C99, IEEE
binary32, no FMA contraction); this module only compiles it with gcc and
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4q_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
RTN, SR = 0, 1
FMT_NVFP4, FMT_NVFP4_2D, FMT_MXFP4, FMT_IF4 = 0, 1, 2, 3

BUILD_CMD = ["gcc", "-std=c99", "-O1", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]


def build() -> str:
    """Compile liboracle.so next to its source (always recompiles)."""
    subprocess.run(BUILD_CMD, check=True)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32
_F = ctypes.c_float
_I = ctypes.c_int


def _declare(L: ctypes.CDLL) -> None:
    sig = {
        "ora_philox4x32_10": (None, [_P, _P, _P]),
        "ora_sr_bits16": (_U32, [_U64, _U32, _U64]),
        "ora_rht_signs": (None, [_U64, _P]),
        "ora_e2m1_decode": (_F, [ctypes.c_uint8]),
        "ora_e2m1_rtn": (ctypes.c_uint8, [_F]),
        "ora_e2m1_sr": (ctypes.c_uint8, [_F, _U32]),
        "ora_e4m3_decode": (_F, [ctypes.c_uint8]),
        "ora_e4m3_encode": (ctypes.c_uint8, [_F]),
        "ora_e8m0_decode": (_F, [ctypes.c_uint8]),
        "ora_e8m0_encode": (ctypes.c_uint8, [_F]),
        "ora_int4_decode": (_F, [ctypes.c_uint8]),
        "ora_amax": (_F, [_P, _I, _I64]),
        "ora_tensor_scale": (_F, [_F]),
        "ora_quantize_nvfp4": (None, [_P, _I, _I64, _I64, _I, _F, _I, _U64, _P, _P]),
        "ora_quantize_nvfp4_strided": (None, [_P, _I, _I64, _I64, _I64, _I64, _F, _I, _U64, _U32, _I64, _P, _P]),
        "ora_quantize_nvfp4_2d": (None, [_P, _I, _I64, _I64, _F, _P, _P]),
        "ora_quantize_mxfp4": (None, [_P, _I, _I64, _I64, _I, _U64, _P, _P]),
        "ora_quantize_if4": (None, [_P, _I, _I64, _I64, _F, _P, _P]),
        "ora_dequantize": (None, [_I, _P, _P, _F, _I64, _I64, _P]),
        "ora_gemm_mxfp4": (None, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
        "ora_gemm_nvfp4": (None, [_P, _P, _F, _P, _P, _F, _I64, _I64, _I64, _I, _P, _P]),
        "ora_fp6_decode": (_F, [_I, ctypes.c_uint8]),
        "ora_fp6_rtn": (ctypes.c_uint8, [_I, _F]),
        "ora_quantize_mxfp6": (None, [_P, _I, _I64, _I64, _I, _P, _P]),
        "ora_dequantize_mxfp6": (None, [_I, _P, _P, _I64, _I64, _P]),
        "ora_hadamard_entry": (_I, [_I, _I]),
        "ora_rht": (None, [_P, _I, _I64, _I64, _P, _I, _P]),
        "ora_rht_column": (None, [_P, _I, _I64, _I64, _I64, _P, _P]),
        "ora_plain_block_roundtrip": (None, [_P, _I64, _I64, _P]),
        "ora_e2m1_rtn_array": (None, [_P, _I64, _P]),
        "ora_e2m1_sr_array": (None, [_P, _P, _I64, _P]),
        "ora_e4m3_encode_array": (None, [_P, _I64, _P]),
        "ora_e8m0_encode_array": (None, [_P, _I64, _P]),
        "ora_sr_bits16_array": (None, [_U64, _U32, _P, _I64, _P]),
        "ora_fp3_decode": (_F, [ctypes.c_uint8]),
        "ora_fp3_rtn": (ctypes.c_uint8, [_F]),
        "ora_variant_row_bytes": (_I64, [_I, _I64]),
        "ora_variant_tensor_scale": (_F, [_I, _F]),
        "ora_quantize_variant": (None, [_P, _I, _I64, _I64, _I, _F, _P, _P]),
        "ora_dequantize_variant": (None, [_I, _P, _P, _F, _I64, _I64, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:          # raw bfloat16 bits
        return BF16
    raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {x.dtype}")


# --- primitives ----------------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    lib().ora_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits16(seed: int, stream: int, idx) -> np.ndarray:
    i = np.ascontiguousarray(np.asarray(idx, dtype=np.uint64).reshape(-1))
    out = np.zeros(i.size, dtype=np.uint32)
    lib().ora_sr_bits16_array(seed, stream, _ptr(i), i.size, _ptr(out))
    return out


def rht_signs(seed: int) -> np.ndarray:
    out = np.zeros(4, dtype=np.uint32)
    lib().ora_rht_signs(seed, _ptr(out))
    return out


def e2m1_decode(nib: int) -> float:
    return lib().ora_e2m1_decode(nib)


def e2m1_rtn(v) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(-1))
    out = np.zeros(a.size, dtype=np.uint8)
    lib().ora_e2m1_rtn_array(_ptr(a), a.size, _ptr(out))
    return out


def e2m1_sr(v, r16) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(-1))
    r = np.ascontiguousarray(np.broadcast_to(np.asarray(r16, dtype=np.uint32), a.shape))
    out = np.zeros(a.size, dtype=np.uint8)
    lib().ora_e2m1_sr_array(_ptr(a), _ptr(r), a.size, _ptr(out))
    return out


def e4m3_encode(y) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(y, dtype=np.float32).reshape(-1))
    out = np.zeros(a.size, dtype=np.uint8)
    lib().ora_e4m3_encode_array(_ptr(a), a.size, _ptr(out))
    return out


def e4m3_decode(code: int) -> float:
    return lib().ora_e4m3_decode(code)


def e8m0_encode(y) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(y, dtype=np.float32).reshape(-1))
    out = np.zeros(a.size, dtype=np.uint8)
    lib().ora_e8m0_encode_array(_ptr(a), a.size, _ptr(out))
    return out


def e8m0_decode(code: int) -> float:
    return lib().ora_e8m0_decode(code)


def int4_decode(nib: int) -> float:
    return lib().ora_int4_decode(nib)


def amax(x: np.ndarray) -> float:
    x = np.ascontiguousarray(x)
    return lib().ora_amax(_ptr(x), _dtype_code(x), x.size)


def tensor_scale(amax_value: float) -> float:
    return lib().ora_tensor_scale(amax_value)


# --- whole-tensor quantizers -----------------------------------------------------

def quantize_nvfp4(x: np.ndarray, colwise: bool = False, gs: float | None = None,
                   rnd: int = RTN, seed: int = 0):
    """NVFP4 1x16.  Returns (codes, scales, gs); column-wise quantizes X^T."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if gs is None:
        gs = tensor_scale(amax(x))
    lr, lc = (cols, rows) if colwise else (rows, cols)
    codes = np.zeros((lr, lc // 2), dtype=np.uint8)
    scales = np.zeros((lr, lc // 16), dtype=np.uint8)
    lib().ora_quantize_nvfp4(_ptr(x), _dtype_code(x), rows, cols, int(colwise), gs, rnd, seed,
                             _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(gs)


def quantize_nvfp4_rows(x: np.ndarray, row0: int, nrows: int, colwise: bool, gs: float,
                        rnd: int = RTN, seed: int = 0):
    """NVFP4 1x16 of logical rows [row0, row0+nrows) only, for sampled checks at full size.

    For colwise the logical matrix is X^T, so its rows are columns of x.  SR draws keep
    the element's index in the whole logical matrix."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    item = x.itemsize
    if colwise:
        lcols, base, sr_, sc_, stream = rows, x.ctypes.data + row0 * item, 1, cols, 1
    else:
        lcols, base, sr_, sc_, stream = cols, x.ctypes.data + row0 * cols * item, cols, 1, 0
    codes = np.zeros((nrows, lcols // 2), dtype=np.uint8)
    scales = np.zeros((nrows, lcols // 16), dtype=np.uint8)
    lib().ora_quantize_nvfp4_strided(base, _dtype_code(x), nrows, lcols, sr_, sc_, gs, rnd, seed,
                                     stream, row0, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_nvfp4_2d(x: np.ndarray, gs: float | None = None):
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if gs is None:
        gs = tensor_scale(amax(x))
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows // 16, cols // 16), dtype=np.uint8)
    lib().ora_quantize_nvfp4_2d(_ptr(x), _dtype_code(x), rows, cols, gs, _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(gs)


def quantize_mxfp4(x: np.ndarray, rnd: int = RTN, seed: int = 0):
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    lib().ora_quantize_mxfp4(_ptr(x), _dtype_code(x), rows, cols, rnd, seed, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_if4(x: np.ndarray, gs: float | None = None):
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if gs is None:
        gs = tensor_scale(amax(x))
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    lib().ora_quantize_if4(_ptr(x), _dtype_code(x), rows, cols, gs, _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(gs)


def dequantize(fmt: int, codes: np.ndarray, scales: np.ndarray, gs: float, rows: int, cols: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.zeros((rows, cols), dtype=np.float32)
    lib().ora_dequantize(fmt, _ptr(codes), _ptr(scales), gs, rows, cols, _ptr(y))
    return y


E2M3, E3M2 = 0, 1


def fp6_decode(fmt: int, code: int) -> float:
    return lib().ora_fp6_decode(fmt, code)


def fp6_rtn(fmt: int, v: float) -> int:
    return lib().ora_fp6_rtn(fmt, v)


def quantize_mxfp6(x: np.ndarray, fmt: int):
    """MX FP6 (fmt E2M3 or E3M2): codes [rows][3 cols / 4] (four per three bytes), E8M0 [rows][cols/32]."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 4 * 3), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    lib().ora_quantize_mxfp6(_ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_mxfp6(fmt: int, codes: np.ndarray, scales: np.ndarray, rows: int, cols: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.zeros((rows, cols), dtype=np.float32)
    lib().ora_dequantize_mxfp6(fmt, _ptr(codes), _ptr(scales), rows, cols, _ptr(y))
    return y


def gemm_mxfp4(a_codes: np.ndarray, a_scales: np.ndarray, b_codes: np.ndarray, b_scales: np.ndarray):
    """C = A B^T over two row-wise MXFP4 operands (A [m][k], B [n][k]), exact sum in
    binary64.  Returns (C, sum of |products|) as float64 [m][n]."""
    a_codes, a_scales = np.ascontiguousarray(a_codes), np.ascontiguousarray(a_scales)
    b_codes, b_scales = np.ascontiguousarray(b_codes), np.ascontiguousarray(b_scales)
    m, k = a_codes.shape[0], a_codes.shape[1] * 2
    n = b_codes.shape[0]
    assert b_codes.shape == (n, k // 2) and a_scales.shape == (m, k // 32) and b_scales.shape == (n, k // 32)
    c = np.zeros((m, n), dtype=np.float64)
    cabs = np.zeros((m, n), dtype=np.float64)
    lib().ora_gemm_mxfp4(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), m, n, k, _ptr(c), _ptr(cabs))
    return c, cabs


def gemm_nvfp4(a_codes, a_scales, gs_a, b_codes, b_scales, gs_b, flags: int = 0):
    """C = A B^T over two row-wise NVFP4 (or IF4) operands with tensor scales gs_a, gs_b:
    (sum of exact products r s r' s') / (gs_a gs_b).  Returns (C, sum |products| / same).
    ``flags`` bit 0 / bit 1 marks A / B as carrying 16x16 scale tiles [rows/16][k/16];
    bit 2 / bit 3 marks A / B as IF4, whose INT4 blocks restore as fl(q fl(6/7)) s."""
    a_codes, a_scales = np.ascontiguousarray(a_codes), np.ascontiguousarray(a_scales)
    b_codes, b_scales = np.ascontiguousarray(b_codes), np.ascontiguousarray(b_scales)
    m, k = a_codes.shape[0], a_codes.shape[1] * 2
    n = b_codes.shape[0]
    ra = m // 16 if flags & 1 else m
    rb = n // 16 if flags & 2 else n
    assert b_codes.shape == (n, k // 2) and a_scales.shape == (ra, k // 16) and b_scales.shape == (rb, k // 16)
    c = np.zeros((m, n), dtype=np.float64)
    cabs = np.zeros((m, n), dtype=np.float64)
    lib().ora_gemm_nvfp4(_ptr(a_codes), _ptr(a_scales), float(gs_a), _ptr(b_codes), _ptr(b_scales), float(gs_b),
                         m, n, k, int(flags), _ptr(c), _ptr(cabs))
    return c, cabs


def hadamard_entry(i: int, t: int) -> int:
    return lib().ora_hadamard_entry(i, t)


def rht(x: np.ndarray, signs, inverse: bool = False) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.uint32).reshape(4))
    y = np.zeros((rows, cols), dtype=np.float32)
    lib().ora_rht(_ptr(x), _dtype_code(x), rows, cols, _ptr(s), int(inverse), _ptr(y))
    return y


def rht_column(x: np.ndarray, j: int, signs) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.uint32).reshape(4))
    y = np.zeros(rows, dtype=np.float32)
    lib().ora_rht_column(_ptr(x), _dtype_code(x), rows, cols, j, _ptr(s), _ptr(y))
    return y


def plain_block_roundtrip(x: np.ndarray, block: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    y = np.zeros_like(x)
    lib().ora_plain_block_roundtrip(_ptr(x), x.size, block, _ptr(y))
    return y


# --- block-format variants: Four Over Six, NVINT4, IF3, IF4 (generic), IF6 -------------

VAR_46, VAR_NVINT4, VAR_IF3, VAR_IF4, VAR_IF6 = 0, 1, 2, 3, 4
VARIANT_BITS = {VAR_46: 4, VAR_NVINT4: 4, VAR_IF3: 3, VAR_IF4: 4, VAR_IF6: 6}


def fp3_decode(code: int) -> float:
    return lib().ora_fp3_decode(code)


def fp3_rtn(v: float) -> int:
    return lib().ora_fp3_rtn(v)


def variant_tensor_scale(var: int, amax_value: float) -> float:
    return lib().ora_variant_tensor_scale(var, amax_value)


def quantize_variant(x: np.ndarray, var: int, gs: float | None = None):
    """Returns (codes [rows][cols*bits/8], scales [rows][cols/16], gs)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if gs is None:
        gs = variant_tensor_scale(var, amax(x))
    codes = np.zeros((rows, lib().ora_variant_row_bytes(var, cols)), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    lib().ora_quantize_variant(_ptr(x), _dtype_code(x), rows, cols, var, gs, _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(gs)


def dequantize_variant(var: int, codes: np.ndarray, scales: np.ndarray, gs: float, rows: int, cols: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.zeros((rows, cols), dtype=np.float32)
    lib().ora_dequantize_variant(var, _ptr(codes), _ptr(scales), gs, rows, cols, _ptr(y))
    return y
