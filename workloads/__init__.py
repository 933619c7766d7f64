"""Seeded synthetic inputs shared by the oracle tests and the GPU path.

Holds input generators and workload tables only; no quantization arithmetic.
"""
from . import rng, synth, configs  # noqa: F401
