"""Seeded synthetic tensors generated on the GPU with torch's counter-based
generator, for workloads too large to draw on the host (the 50-step sweeps).

Only input generation lives here. A stream is named like the host streams:
its torch seed is the stream key of (seed, name) from ``rng.stream_key``,
so every (seed, name) pair gives the same bytes on every run. The CPU side
of a test gets the very same values by copying the generated tensor to the
host.
"""
from __future__ import annotations

from .rng import stream_key


def _generator(torch, seed: int, name: str):
    g = torch.Generator(device="cuda")
    g.manual_seed(stream_key(seed, name) & ((1 << 63) - 1))
    return g


def silu_normal(torch, seed: int, name: str, M: int, K: int):
    """fp32 [M,K] on the GPU = SiLU(z), z ~ N(0,1) drawn in float64;
    SiLU(x) = x / (1 + exp(-x)) in float64, rounded once to fp32."""
    z = torch.randn((M, K), generator=_generator(torch, seed, name), device="cuda",
                    dtype=torch.float64)
    return (z / (1.0 + torch.exp(-z))).to(torch.float32)


def weight_normal(torch, seed: int, name: str, N: int, K: int, std: float = 0.02):
    """fp32 W [N,K] on the GPU ~ N(0, std^2) (std is the standard deviation)."""
    z = torch.randn((N, K), generator=_generator(torch, seed, name), device="cuda",
                    dtype=torch.float64)
    return (std * z).to(torch.float32)
