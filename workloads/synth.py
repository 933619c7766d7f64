"""Seeded synthetic tensors with the shapes and value distributions of the
diffusion-transformer linears described on the pages (no datasets or trained
weights exist here, so these stand in for them).

Only input generation lives here: activation functions applied to random
normals (SiLU, GELU), outlier injection, bf16 rounding of inputs and integer
schedules. None of the quantized linear's own arithmetic is in this module.

Every function is a pure function of (seed, stream name, shape): the same call
gives the same bytes on any machine, so the CPU oracle and the GPU path see
identical inputs.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .rng import Stream


def normal_f64(seed: int, name: str, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return Stream(seed, name).normal(n).reshape(shape)


def silu_normal(seed: int, name: str, M: int, K: int) -> np.ndarray:
    """fp32 [M,K] = SiLU(z), z ~ N(0,1); SiLU(x) = x / (1 + exp(-x)) in float64."""
    z = normal_f64(seed, name, (M, K))
    return (z / (1.0 + np.exp(-z))).astype(np.float32)


def gelu_normal(seed: int, name: str, M: int, K: int) -> np.ndarray:
    """fp32 [M,K] = GELU(z), z ~ N(0,1); exact erf form x * Phi(x) in float64."""
    z = normal_f64(seed, name, (M, K))
    return (0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))).astype(np.float32)


def sinusoid(seed: int, name: str, M: int, K: int) -> np.ndarray:
    """fp32 [M,K] = sin(3 z), z ~ N(0,1): bounded features in [-1, 1], like a
    sinusoidal timestep embedding concatenated to a hidden state."""
    z = normal_f64(seed, name, (M, K))
    return np.sin(3.0 * z).astype(np.float32)


def outlier_columns(seed: int, name: str, K: int, frac: float = 0.001) -> np.ndarray:
    """max(1, round(frac*K)) distinct channel indices, seeded, sorted."""
    cnt = max(1, int(round(frac * K)))
    return Stream(seed, name).choice_without_replacement(K, cnt)


def gelu_with_outliers(seed: int, name: str, M: int, K: int,
                       frac: float = 0.001, factor: float = 20.0) -> np.ndarray:
    """GELU(N(0,1)) with a seeded 0.1 % of channels (same for every row)
    multiplied by 20 after the activation (exact in fp32: the product of an
    fp32 value and 20 is rounded once)."""
    x = gelu_normal(seed, name, M, K)
    cols = outlier_columns(seed, name + "/outcols", K, frac)
    x[:, cols] = (x[:, cols].astype(np.float64) * factor).astype(np.float32)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even), return the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_normal(seed: int, name: str, M: int, K: int) -> np.ndarray:
    """uint16 bf16 bit patterns [M,K] of N(0,1) (float64 -> fp32 -> bf16, both RNE)."""
    z = normal_f64(seed, name, (M, K)).astype(np.float32)
    return f32_to_bf16_bits(z)


def weight_normal(seed: int, name: str, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """fp32 W [N,K] ~ N(0, std^2) (std is the standard deviation)."""
    return (std * normal_f64(seed, name, (N, K))).astype(np.float32)


def lognormal(seed: int, name: str, n: int) -> np.ndarray:
    """float64 [n] = exp(N(0,1)), e.g. synthetic per-layer sensitivities."""
    return np.exp(normal_f64(seed, name, (n,)))


def uniform_choice_schedule(seed: int, name: str, rows: int, cols: int, choices) -> np.ndarray:
    """int32 [rows, cols] drawn uniformly from `choices` (seeded)."""
    ch = np.asarray(choices, dtype=np.int32)
    idx = Stream(seed, name).integers(rows * cols, 0, len(ch))
    return ch[idx].reshape(rows, cols)


def half_mask(seed: int, name: str, n: int) -> np.ndarray:
    """Boolean [n] with exactly n//2 True entries, placed by a seeded shuffle."""
    perm = Stream(seed, name).permutation(n)
    m = np.zeros(n, dtype=bool)
    m[perm[: n // 2]] = True
    return m


def random_int_codes(seed: int, name: str, shape, lo: int, hi: int) -> np.ndarray:
    """int8 codes uniform in [lo, hi] (inclusive), for integer-path tests."""
    n = int(np.prod(shape))
    return Stream(seed, name).integers(n, lo, hi + 1).astype(np.int8).reshape(shape)
