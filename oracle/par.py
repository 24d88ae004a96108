"""The oracle over whole full-size tensors, split into independent row ranges that run
on host threads (test infrastructure).

Every quantized unit the oracle computes -- a 1x16 block of a logical row, a 16x16
tile, a 32-element block, a 128-token transform chunk, one dequantized element --
depends only on its own inputs and the tensor scale, so splitting a tensor into row
ranges and calling the oracle on each range gives the same bytes as one call over the
whole tensor (the stochastic-rounding index is kept global by passing each range's
first logical row).  The oracle's C functions run without the Python interpreter lock,
so the ranges run concurrently.  Nothing here changes the oracle's arithmetic.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


_THREADS = None


def set_threads(n: int | None) -> None:
    """Threads for the split calls (None: the host cores this process may use, at most 16)."""
    global _THREADS
    _THREADS = n


def workers() -> int:
    if _THREADS:
        return _THREADS
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ranges(n: int, align: int, parts: int):
    step = max(align, -(-n // parts) // align * align)
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def _run(fn, ranges):
    with ThreadPoolExecutor(workers()) as ex:
        list(ex.map(lambda r: fn(*r), ranges))


def amax(x: np.ndarray) -> float:
    rows = x.shape[0]
    out = {}

    def one(a, b):
        out[a] = oracle.amax(np.ascontiguousarray(x[a:b]))
    _run(one, _ranges(rows, 1, 4 * workers()))
    return float(max(out.values()))


def quantize_nvfp4(x: np.ndarray, colwise: bool, gs: float, rnd: int = oracle.RTN, seed: int = 0):
    """NVFP4 1x16 of the whole tensor: codes and scales of X (row-wise) or X^T."""
    rows, cols = x.shape
    lr, lc = (cols, rows) if colwise else (rows, cols)
    codes = np.empty((lr, lc // 2), np.uint8)
    scales = np.empty((lr, lc // 16), np.uint8)

    def one(a, b):
        c, s = oracle.quantize_nvfp4_rows(x, a, b - a, colwise, gs, rnd=rnd, seed=seed)
        codes[a:b], scales[a:b] = c, s
    _run(one, _ranges(lr, 1, 4 * workers()))
    return codes, scales


def quantize_nvfp4_2d(x: np.ndarray, gs: float):
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows // 16, cols // 16), np.uint8)

    def one(a, b):
        c, s, _ = oracle.quantize_nvfp4_2d(np.ascontiguousarray(x[a:b]), gs=gs)
        codes[a:b], scales[a // 16:b // 16] = c, s
    _run(one, _ranges(rows, 16, 4 * workers()))
    return codes, scales


def quantize_mxfp4_rtn(x: np.ndarray):
    """MXFP4 round-to-nearest (no stream index, so row ranges are independent)."""
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)

    def one(a, b):
        c, s = oracle.quantize_mxfp4(np.ascontiguousarray(x[a:b]))
        codes[a:b], scales[a:b] = c, s
    _run(one, _ranges(rows, 1, 4 * workers()))
    return codes, scales


def quantize_if4(x: np.ndarray, gs: float):
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)

    def one(a, b):
        c, s, _ = oracle.quantize_if4(np.ascontiguousarray(x[a:b]), gs=gs)
        codes[a:b], scales[a:b] = c, s
    _run(one, _ranges(rows, 1, 4 * workers()))
    return codes, scales


def dequantize(fmt: int, codes: np.ndarray, scales: np.ndarray, gs: float, rows: int, cols: int):
    y = np.empty((rows, cols), np.float32)
    tile = 16 if fmt == oracle.FMT_NVFP4_2D else 1

    def one(a, b):
        sc = scales[a // 16:b // 16] if tile == 16 else scales[a:b]
        y[a:b] = oracle.dequantize(fmt, np.ascontiguousarray(codes[a:b]), np.ascontiguousarray(sc), gs, b - a,
                                   cols)
    _run(one, _ranges(rows, tile, 4 * workers()))
    return y


def rht(x: np.ndarray, signs) -> np.ndarray:
    """Forward transform along rows, chunk by chunk of 128 rows."""
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float32)

    def one(a, b):
        y[a:b] = oracle.rht(np.ascontiguousarray(x[a:b]), signs)
    _run(one, _ranges(rows, 128, 4 * workers()))
    return y


def quantize_variant(x: np.ndarray, var: int, gs: float):
    """A block-format variant (Four Over Six, NVINT4, IF3, IF4, IF6) of the whole tensor."""
    rows, cols = x.shape
    codes = np.empty((rows, cols * oracle.VARIANT_BITS[var] // 8), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)

    def one(a, b):
        c, s, _ = oracle.quantize_variant(np.ascontiguousarray(x[a:b]), var, gs=gs)
        codes[a:b], scales[a:b] = c, s
    _run(one, _ranges(rows, 1, 4 * workers()))
    return codes, scales


def dequantize_variant(var: int, codes: np.ndarray, scales: np.ndarray, gs: float, rows: int, cols: int):
    y = np.empty((rows, cols), np.float32)

    def one(a, b):
        y[a:b] = oracle.dequantize_variant(var, np.ascontiguousarray(codes[a:b]), np.ascontiguousarray(scales[a:b]),
                                           gs, b - a, cols)
    _run(one, _ranges(rows, 1, 4 * workers()))
    return y
