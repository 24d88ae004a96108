"""ctypes binding of libfp4q -- argument marshalling only.

Each ``fp4q_*`` function here has the name and argument order of the C entry point
in include/fp4q.h.  Device buffers are passed as torch CUDA tensors (or None for a
NULL pointer), the stream defaults to torch's current stream, and a non-OK status
raises :class:`Fp4qError`.  Every quantization step runs in the HIP library; if
libfp4q.so is missing, loading fails loudly -- there is no fallback.

The ``quantize_*`` / ``dequantize`` / ``rht`` helpers below only allocate the output
tensors with torch and call the same-name entry points.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4q.so")

F32, BF16 = 0, 1
RTN, SR = 0, 1
FMT_NVFP4, FMT_NVFP4_2D, FMT_MXFP4, FMT_IF4 = 0, 1, 2, 3
ROWWISE, COLWISE = 1, 2
AMAX_COMPUTE, AMAX_GIVEN = 0, 1
STATUS = {0: "FP4Q_OK", 1: "FP4Q_E_NULL", 2: "FP4Q_E_SHAPE", 3: "FP4Q_E_ALIGN", 4: "FP4Q_E_ARG", 5: "FP4Q_E_HIP"}

EXPORTS = ["fp4q_workspace_create", "fp4q_workspace_destroy", "fp4q_workspace_set_wait", "fp4q_workspace_fallbacks",
           "fp4q_quantize_nvfp4", "fp4q_quantize_nvfp4_noalloc", "fp4q_quantize_nvfp4_2d", "fp4q_quantize_mxfp4", "fp4q_quantize_mxfp6",
           "fp4q_quantize_if4", "fp4q_quantize_variant", "fp4q_dequantize_variant", "fp4q_rht", "fp4q_gemm_mxfp4", "fp4q_gemm_nvfp4", "fp4q_dequantize", "fp4q_amax",
           "fp4q_rht_signs_from_seed", "fp4q_status_string", "fp4q_abi_version"]


class Fp4qError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


_lib = None
_P, _I64, _U64, _I, _U = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint


def lib() -> ctypes.CDLL:
    """Load libfp4q.so (built in-tree by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with block_scaled_fp4_05_amd/build.py "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "fp4q_workspace_create": [_P],
            "fp4q_workspace_destroy": [_P],
            "fp4q_workspace_set_wait": [_P, _U],
            "fp4q_workspace_fallbacks": [_P, _P, _P],
            "fp4q_quantize_nvfp4": [_P, _I, _I64, _I64, _U, _I, _U64, _P, _U, _P, _P, _P, _P, _P, _P, _P, _P],
            "fp4q_quantize_nvfp4_noalloc": [_P, _I, _I64, _I64, _U, _I, _U64, _P, _U, _P, _P, _P, _P, _P, _P, _P],
            "fp4q_quantize_nvfp4_2d": [_P, _I, _I64, _I64, _U, _P, _P, _P, _P, _P, _P, _P],
            "fp4q_quantize_mxfp4": [_P, _I, _I64, _I64, _I, _U64, _P, _P, _P, _P, _P],
            "fp4q_quantize_mxfp6": [_P, _I, _I64, _I64, _I, _P, _P, _P],
            "fp4q_quantize_if4": [_P, _I, _I64, _I64, _U, _P, _P, _P, _P, _P, _P],
            "fp4q_quantize_variant": [_P, _I, _I64, _I64, _I, _U, _P, _P, _P, _P, _P, _P],
            "fp4q_dequantize_variant": [_I, _P, _P, _P, _I64, _I64, _I, _P, _P],
            "fp4q_rht": [_P, _I, _I64, _I64, _P, _I, _P, _P],
            "fp4q_gemm_mxfp4": [_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P],
            "fp4q_gemm_nvfp4": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _U, _I, _P, _P, _P],
            "fp4q_dequantize": [_I, _P, _P, _P, _I64, _I64, _I, _P, _P],
            "fp4q_amax": [_P, _I, _I64, _I64, _P, _P],
            "fp4q_rht_signs_from_seed": [_U64, _P],
            "fp4q_status_string": [_I],
            "fp4q_abi_version": [],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _I
        L.fp4q_rht_signs_from_seed.restype = None
        L.fp4q_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _p(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, Workspace):
        return t.handle
    return t.data_ptr()


def _s(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> int:
    if status != 0:
        raise Fp4qError(fn, status)
    return status


def _signs_arg(signs):
    if signs is None:
        return None, None
    arr = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in signs])
    return ctypes.addressof(arr), arr


# --- workspaces ----------------------------------------------------------------------

class Workspace:
    """A libfp4q workspace (fp4q_workspace_create on the current device).  close()
    destroys it; the caller makes sure no enqueued work still uses it."""

    def __init__(self):
        h = ctypes.c_void_p(0)
        _check("fp4q_workspace_create", lib().fp4q_workspace_create(ctypes.addressof(h)))
        self.handle = h.value

    def close(self) -> None:
        if self.handle:
            _check("fp4q_workspace_destroy", lib().fp4q_workspace_destroy(self.handle))
            self.handle = None


_ws_cache: dict = {}


def stream_workspace(stream=None) -> Workspace:
    """The helpers' workspace for (current device, stream), created on first use and kept
    for the life of the process (create one yourself, or pass ws=None, where a call must
    not allocate, e.g. inside graph capture)."""
    key = (torch.cuda.current_device(), _s(stream))
    w = _ws_cache.get(key)
    if w is None:
        w = _ws_cache[key] = Workspace()
    return w


def _ws(ws, stream):
    return stream_workspace(stream) if isinstance(ws, str) and ws == "auto" else ws


# --- the C entry points, same names -----------------------------------------------

def fp4q_workspace_set_wait(ws: Workspace, microseconds: int) -> int:
    return _check("fp4q_workspace_set_wait", lib().fp4q_workspace_set_wait(_p(ws), microseconds))


def fp4q_workspace_fallbacks(ws: Workspace, stream=None) -> int:
    out = ctypes.c_uint32(0)
    _check("fp4q_workspace_fallbacks", lib().fp4q_workspace_fallbacks(_p(ws), _s(stream), ctypes.addressof(out)))
    return out.value


def fp4q_quantize_nvfp4(x, dt, rows, cols, layouts, rnd, sr_seed, rht_signs, amax_mode, amax, tensor_scale,
                        row_codes, row_scales, col_codes, col_scales, ws=None, stream=None) -> int:
    sp, _keep = _signs_arg(rht_signs)
    return _check("fp4q_quantize_nvfp4", lib().fp4q_quantize_nvfp4(
        _p(x), dt, rows, cols, layouts, rnd, sr_seed, sp, amax_mode, _p(amax), _p(tensor_scale),
        _p(row_codes), _p(row_scales), _p(col_codes), _p(col_scales), _p(ws), _s(stream)))


def fp4q_quantize_nvfp4_noalloc(x, dt, rows, cols, layouts, rnd, sr_seed, rht_signs, amax_mode, amax, tensor_scale,
                                row_codes, row_scales, col_codes, col_scales, stream=None) -> int:
    sp, _keep = _signs_arg(rht_signs)
    return _check("fp4q_quantize_nvfp4_noalloc", lib().fp4q_quantize_nvfp4_noalloc(
        _p(x), dt, rows, cols, layouts, rnd, sr_seed, sp, amax_mode, _p(amax), _p(tensor_scale),
        _p(row_codes), _p(row_scales), _p(col_codes), _p(col_scales), _s(stream)))


def fp4q_quantize_nvfp4_2d(x, dt, rows, cols, amax_mode, amax, tensor_scale, codes, scales, codes_t,
                           ws=None, stream=None) -> int:
    return _check("fp4q_quantize_nvfp4_2d", lib().fp4q_quantize_nvfp4_2d(
        _p(x), dt, rows, cols, amax_mode, _p(amax), _p(tensor_scale), _p(codes), _p(scales), _p(codes_t),
        _p(ws), _s(stream)))


def fp4q_quantize_mxfp4(x, dt, rows, cols, rnd, sr_seed, codes, scales, amax=None, ws=None, stream=None) -> int:
    return _check("fp4q_quantize_mxfp4", lib().fp4q_quantize_mxfp4(
        _p(x), dt, rows, cols, rnd, sr_seed, _p(codes), _p(scales), _p(amax), _p(ws), _s(stream)))


def fp4q_quantize_mxfp6(x, dt, rows, cols, fmt, codes, scales, stream=None) -> int:
    return _check("fp4q_quantize_mxfp6", lib().fp4q_quantize_mxfp6(
        _p(x), dt, rows, cols, fmt, _p(codes), _p(scales), _s(stream)))


def fp4q_quantize_if4(x, dt, rows, cols, amax_mode, amax, tensor_scale, codes, scales, ws=None,
                      stream=None) -> int:
    return _check("fp4q_quantize_if4", lib().fp4q_quantize_if4(
        _p(x), dt, rows, cols, amax_mode, _p(amax), _p(tensor_scale), _p(codes), _p(scales), _p(ws), _s(stream)))


def fp4q_quantize_variant(x, dt, rows, cols, var, amax_mode, amax, tensor_scale, codes, scales, ws=None,
                          stream=None) -> int:
    return _check("fp4q_quantize_variant", lib().fp4q_quantize_variant(
        _p(x), dt, rows, cols, var, amax_mode, _p(amax), _p(tensor_scale), _p(codes), _p(scales), _p(ws),
        _s(stream)))


def fp4q_dequantize_variant(var, codes, scales, tensor_scale, rows, cols, out_dt, y, stream=None) -> int:
    return _check("fp4q_dequantize_variant", lib().fp4q_dequantize_variant(
        var, _p(codes), _p(scales), _p(tensor_scale), rows, cols, out_dt, _p(y), _s(stream)))


def fp4q_rht(x, dt, rows, cols, signs, inverse, y, stream=None) -> int:
    sp, _keep = _signs_arg(signs)
    return _check("fp4q_rht", lib().fp4q_rht(_p(x), dt, rows, cols, sp, int(inverse), _p(y), _s(stream)))


def fp4q_gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, m, n, k, out_dt, c, amax=None, stream=None) -> int:
    return _check("fp4q_gemm_mxfp4", lib().fp4q_gemm_mxfp4(
        _p(a_codes), _p(a_scales), _p(b_codes), _p(b_scales), m, n, k, out_dt, _p(c), _p(amax), _s(stream)))


TILES_A, TILES_B, IF4_A, IF4_B = 1, 2, 4, 8


def fp4q_gemm_nvfp4(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, m, n, k, operand_flags, out_dt, c, amax=None,
                    stream=None) -> int:
    return _check("fp4q_gemm_nvfp4", lib().fp4q_gemm_nvfp4(
        _p(a_codes), _p(a_scales), _p(a_ts), _p(b_codes), _p(b_scales), _p(b_ts), m, n, k, operand_flags, out_dt,
        _p(c), _p(amax), _s(stream)))


def fp4q_dequantize(fmt, codes, scales, tensor_scale, rows, cols, out_dt, y, stream=None) -> int:
    return _check("fp4q_dequantize", lib().fp4q_dequantize(
        fmt, _p(codes), _p(scales), _p(tensor_scale), rows, cols, out_dt, _p(y), _s(stream)))


def fp4q_amax(x, dt, rows, cols, amax, stream=None) -> int:
    return _check("fp4q_amax", lib().fp4q_amax(_p(x), dt, rows, cols, _p(amax), _s(stream)))


def fp4q_rht_signs_from_seed(seed: int) -> list[int]:
    out = (ctypes.c_uint32 * 4)()
    lib().fp4q_rht_signs_from_seed(seed, ctypes.addressof(out))
    return list(out)


def fp4q_status_string(status: int) -> str:
    return lib().fp4q_status_string(status).decode()


def fp4q_abi_version() -> int:
    return lib().fp4q_abi_version()


# --- allocation helpers --------------------------------------------------------------

def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float32:
        return F32
    raise TypeError(f"libfp4q takes bfloat16 or float32 input, got {x.dtype}")


def _u8(*shape, device):
    return torch.empty(*shape, dtype=torch.uint8, device=device)


def quantize_nvfp4(x: torch.Tensor, layouts: int = ROWWISE | COLWISE, rnd: int = RTN, sr_seed: int = 0,
                   rht_signs=None, amax: torch.Tensor | None = None, ws="auto", stream=None) -> dict:
    """NVFP4 1x16.  If `amax` is given it is used as the tensor amax (AMAX_GIVEN).
    ws: "auto" (the stream's cached workspace), None (no workspace) or a Workspace."""
    rows, cols = x.shape
    dev = x.device
    out = {"tensor_scale": torch.empty(1, dtype=torch.float32, device=dev)}
    mode = AMAX_GIVEN if amax is not None else AMAX_COMPUTE
    out["amax"] = amax if amax is not None else torch.empty(1, dtype=torch.float32, device=dev)
    rc = rs = cc = cs = None
    if layouts & ROWWISE:
        rc, rs = _u8(rows, cols // 2, device=dev), _u8(rows, cols // 16, device=dev)
        out["row_codes"], out["row_scales"] = rc, rs
    if layouts & COLWISE:
        cc, cs = _u8(cols, rows // 2, device=dev), _u8(cols, rows // 16, device=dev)
        out["col_codes"], out["col_scales"] = cc, cs
    fp4q_quantize_nvfp4(x, _dt(x), rows, cols, layouts, rnd, sr_seed, rht_signs, mode, out["amax"],
                        out["tensor_scale"], rc, rs, cc, cs, _ws(ws, stream), stream)
    return out


def quantize_nvfp4_2d(x: torch.Tensor, transposed: bool = False, amax: torch.Tensor | None = None,
                      ws="auto", stream=None) -> dict:
    """NVFP4 16x16.  If `amax` is given it is used as the tensor amax (AMAX_GIVEN)."""
    rows, cols = x.shape
    dev = x.device
    mode = AMAX_GIVEN if amax is not None else AMAX_COMPUTE
    out = {"amax": amax if amax is not None else torch.empty(1, dtype=torch.float32, device=dev),
           "tensor_scale": torch.empty(1, dtype=torch.float32, device=dev),
           "codes": _u8(rows, cols // 2, device=dev), "scales": _u8(rows // 16, cols // 16, device=dev),
           "codes_t": _u8(cols, rows // 2, device=dev) if transposed else None}
    fp4q_quantize_nvfp4_2d(x, _dt(x), rows, cols, mode, out["amax"], out["tensor_scale"], out["codes"],
                           out["scales"], out["codes_t"], _ws(ws, stream), stream)
    return out


def quantize_mxfp4(x: torch.Tensor, rnd: int = RTN, sr_seed: int = 0, with_amax: bool = False,
                   ws="auto", stream=None) -> dict:
    rows, cols = x.shape
    dev = x.device
    out = {"codes": _u8(rows, cols // 2, device=dev), "scales": _u8(rows, cols // 32, device=dev)}
    if with_amax:
        out["amax"] = torch.empty(1, dtype=torch.float32, device=dev)
    fp4q_quantize_mxfp4(x, _dt(x), rows, cols, rnd, sr_seed, out["codes"], out["scales"], out.get("amax"),
                        _ws(ws, stream) if with_amax else None, stream)
    return out


FP6_E2M3, FP6_E3M2 = 0, 1
FMT_MXFP6 = {FP6_E2M3: 4, FP6_E3M2: 5}


def quantize_mxfp6(x: torch.Tensor, fmt: int = FP6_E2M3, stream=None) -> dict:
    """MX FP6: codes [rows][3 cols / 4] (four per three bytes), E8M0 scales [rows][cols/32]."""
    rows, cols = x.shape
    dev = x.device
    out = {"codes": _u8(rows, cols // 4 * 3, device=dev), "scales": _u8(rows, cols // 32, device=dev)}
    fp4q_quantize_mxfp6(x, _dt(x), rows, cols, fmt, out["codes"], out["scales"], stream)
    return out


def quantize_if4(x: torch.Tensor, amax: torch.Tensor | None = None, ws="auto", stream=None) -> dict:
    """IF4.  If `amax` is given it is used as the tensor amax (AMAX_GIVEN)."""
    rows, cols = x.shape
    dev = x.device
    mode = AMAX_GIVEN if amax is not None else AMAX_COMPUTE
    out = {"amax": amax if amax is not None else torch.empty(1, dtype=torch.float32, device=dev),
           "tensor_scale": torch.empty(1, dtype=torch.float32, device=dev),
           "codes": _u8(rows, cols // 2, device=dev), "scales": _u8(rows, cols // 16, device=dev)}
    fp4q_quantize_if4(x, _dt(x), rows, cols, mode, out["amax"], out["tensor_scale"], out["codes"],
                      out["scales"], _ws(ws, stream), stream)
    return out


def rht(x: torch.Tensor, signs, inverse: bool = False, stream=None) -> torch.Tensor:
    rows, cols = x.shape
    y = torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    fp4q_rht(x, _dt(x), rows, cols, signs, inverse, y, stream)
    return y


def gemm_mxfp4(a: dict, b: dict, out_dtype=torch.float32, amax: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """C = A B^T for two row-wise MXFP4 operands as quantize_mxfp4 returns them.

    With ``amax`` (a one-element float32 device tensor) the GEMM also writes max |C| of
    the stored outputs there."""
    m, n, k = a["codes"].shape[0], b["codes"].shape[0], a["codes"].shape[1] * 2
    c = torch.empty(m, n, dtype=out_dtype, device=a["codes"].device)
    fp4q_gemm_mxfp4(a["codes"], a["scales"], b["codes"], b["scales"], m, n, k, _dt(c), c, amax, stream)
    return c


def gemm_nvfp4(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, out_dtype=torch.float32,
               amax: torch.Tensor | None = None, operand_flags: int = 0, stream=None) -> torch.Tensor:
    """C = A B^T / (gs_a gs_b) for two row-wise NVFP4 or IF4 operands (codes, scales, tensor
    scale); ``operand_flags`` marks operands with 16x16 scale tiles (TILES_A, TILES_B) and IF4
    operands (IF4_A, IF4_B); ``amax`` as for gemm_mxfp4."""
    m, n, k = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    c = torch.empty(m, n, dtype=out_dtype, device=a_codes.device)
    fp4q_gemm_nvfp4(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, m, n, k, operand_flags, _dt(c), c, amax, stream)
    return c


def dequantize(fmt: int, codes: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor | None,
               rows: int, cols: int, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    y = torch.empty(rows, cols, dtype=out_dtype, device=codes.device)
    fp4q_dequantize(fmt, codes, scales, tensor_scale, rows, cols, _dt(y), y, stream)
    return y


def amax(x: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    fp4q_amax(x, _dt(x), x.shape[0], x.shape[1], out, stream)
    return out


VAR_46, VAR_NVINT4, VAR_IF3, VAR_IF4, VAR_IF6 = 0, 1, 2, 3, 4
VARIANT_BITS = {VAR_46: 4, VAR_NVINT4: 4, VAR_IF3: 3, VAR_IF4: 4, VAR_IF6: 6}


def quantize_variant(x: torch.Tensor, var: int, amax: torch.Tensor | None = None, ws="auto", stream=None) -> dict:
    """Four Over Six, NVINT4, IF3, IF4 or IF6 (codes [rows][cols * bits / 8], scales [rows][cols/16])."""
    rows, cols = x.shape
    dev = x.device
    mode = AMAX_GIVEN if amax is not None else AMAX_COMPUTE
    out = {"amax": amax if amax is not None else torch.empty(1, dtype=torch.float32, device=dev),
           "tensor_scale": torch.empty(1, dtype=torch.float32, device=dev),
           "codes": _u8(rows, cols * VARIANT_BITS[var] // 8, device=dev), "scales": _u8(rows, cols // 16, device=dev)}
    fp4q_quantize_variant(x, _dt(x), rows, cols, var, mode, out["amax"], out["tensor_scale"], out["codes"],
                          out["scales"], _ws(ws, stream), stream)
    return out


def dequantize_variant(var: int, codes, scales, tensor_scale, rows: int, cols: int, out_dtype=torch.float32,
                       stream=None) -> torch.Tensor:
    y = torch.empty(rows, cols, dtype=out_dtype, device=codes.device)
    fp4q_dequantize_variant(var, codes, scales, tensor_scale, rows, cols, _dt(y), y, stream)
    return y
