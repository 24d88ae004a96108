"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random tensors; it holds none of the quantization
arithmetic, so both the CPU oracle and the HIP library can consume its output
without sharing any code with each other.

Every generator draws float32 values from numpy's PCG64 (``default_rng(seed)``)
and, where the workload is bfloat16, rounds them to bfloat16 with
round-to-nearest-even on the float32 bit pattern.  bfloat16 tensors are returned
as their raw ``uint16`` bit patterns.  The shapes and statistics follow the five
workloads the method is measured on:

* tiny reference: 4096 values from ``torch.manual_seed(0); torch.randn(4096)`` with
  every 512th value multiplied by 20 (the glossary's outlier example);
* activation: N(0,1) with 1% of the columns scaled by 30;
* weight: N(0, 0.02^2) in float32;
* Wgrad operands: a Laplace(0, 1e-3) gradient and an N(0,1) activation whose 1% of
  rows (tokens) are scaled by 30;
* IF4 mix: rows split 50% N(0,1) / 25% U(-1,1) / 25% Laplace(0,1), then 0.1% of all
  elements scaled by 50.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tiny_reference() -> np.ndarray:
    """4096 float32 values: torch's CPU generator seeded with 0, every 512th x20."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    x = torch.randn(4096, generator=g)
    x[::512] *= 20
    return x.numpy().astype(np.float32)


def activation(rows: int = 8192, cols: int = 4096, seed: int = 2, outlier_frac: float = 0.01,
               outlier_gain: float = 30.0) -> np.ndarray:
    """bf16 bits [rows, cols]: N(0,1), a random 1% of the columns scaled by 30."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    n_out = max(1, int(round(outlier_frac * cols)))
    cols_out = rng.choice(cols, n_out, replace=False)
    x[:, cols_out] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


def weight(rows: int = 8192, cols: int = 8192, seed: int = 3, std: float = 0.02) -> np.ndarray:
    """float32 [rows, cols] ~ N(0, std^2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(std)
    return x


def wgrad_gradient(rows: int = 16384, cols: int = 4096, seed: int = 4, b: float = 1e-3) -> np.ndarray:
    """bf16 bits [tokens, cols] ~ Laplace(0, b)."""
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, b, size=(rows, cols)).astype(np.float32)
    return f32_to_bf16_bits(x)


def wgrad_activation(rows: int = 16384, cols: int = 4096, seed: int = 4, outlier_frac: float = 0.01,
                     outlier_gain: float = 30.0) -> np.ndarray:
    """bf16 bits [tokens, cols]: N(0,1) with a random 1% of the tokens (rows) scaled by 30.

    Drawn from the stream after the gradient's, so (seed) gives both operands."""
    rng = np.random.default_rng(seed + 1000)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    n_out = max(1, int(round(outlier_frac * rows)))
    rows_out = rng.choice(rows, n_out, replace=False)
    x[rows_out, :] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


def if4_mix(rows: int = 32768, cols: int = 8192, seed: int = 5, outlier_frac: float = 0.001,
            outlier_gain: float = 50.0) -> np.ndarray:
    """bf16 bits [rows, cols]: first half of the rows N(0,1), next quarter U(-1,1), last
    quarter Laplace(0,1); then a random 0.1% of all elements scaled by 50."""
    rng = np.random.default_rng(seed)
    x = np.empty((rows, cols), dtype=np.float32)
    r_half, r_3q = rows // 2, (3 * rows) // 4
    x[:r_half] = rng.standard_normal((r_half, cols), dtype=np.float32)
    x[r_half:r_3q] = rng.uniform(-1.0, 1.0, size=(r_3q - r_half, cols)).astype(np.float32)
    x[r_3q:] = rng.laplace(0.0, 1.0, size=(rows - r_3q, cols)).astype(np.float32)
    n = rows * cols
    n_out = max(1, int(n * outlier_frac))
    flat = x.reshape(-1)
    idx = rng.choice(n, n_out, replace=False)
    flat[idx] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


def normal_f32(n: int, seed: int) -> np.ndarray:
    """n float32 N(0,1) values (used for the format's error statistics)."""
    return np.random.default_rng(seed).standard_normal(n, dtype=np.float32)
