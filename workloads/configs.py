"""The five synthetic workloads: layer shapes, quantization settings and input
recipes for the quantized linear of a diffusion transformer.

Shapes: DiT-XL/2 (hidden 1152, 32x32 latent with patch 2 -> 256 tokens per
image, 8 images doubled to 16 for the conditional / unconditional pair ->
M = 4096) and an MM-DiT block (hidden 3072, 4096 image + 512 text tokens,
2 images doubled for the pair -> M = 18432).

Seeds: base seed 0; every tensor has its own named substream.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

from . import synth

SEED = 0


@dataclass(frozen=True)
class Layer:
    name: str
    K: int
    N: int
    w_bits: int = 8
    a_bits: int = 8
    hadamard_block: int = 0
    n_segments: int = 1
    w_scale: str = "channel"          # "tensor" | "segment" | "channel"
    a_scale: str = "dual"             # "dual" | "symmetric"
    x_dtype: str = "f32"              # "f32" | "bf16"
    x_kind: str = "silu"              # "silu" | "gelu_outliers" | "bf16_normal"
    cfg: bool = False
    guidance: float = 4.0
    single_hadamard: bool = False     # rotate X only (W enters as H W_int^T)
    k_seg: Tuple[int, ...] = ()       # input branch offsets (SegLinear input segmentation)
    branch_kinds: Tuple[str, ...] = ()  # x_kind of each input branch

    def seg_offsets(self) -> Optional[np.ndarray]:
        if self.n_segments <= 1:
            return None
        assert self.N % self.n_segments == 0
        w = self.N // self.n_segments
        return np.arange(0, self.N + 1, w, dtype=np.int32)


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    M: int
    layers: Tuple[Layer, ...]
    steps: int = 1
    lsb_choices: Tuple[int, ...] = (0,)
    stages: int = 1
    notes: str = ""


DIT_SHAPES = (("qkv", 1152, 3456), ("proj", 1152, 1152), ("fc1", 1152, 4608), ("fc2", 4608, 1152))
MMDIT_SHAPES = (("adaln", 3072, 18432, 6), ("qkv", 3072, 9216, 3), ("fc1", 3072, 12288, 1), ("fc2", 12288, 3072, 1))


def _c1() -> Workload:
    return Workload(
        key="c1", title="single W8A8 linear, M=256 K=512 N=512, SiLU inputs",
        M=256, layers=(Layer("linear", 512, 512, x_kind="silu"),))


def _c2() -> Workload:
    return Workload(
        key="c2", title="DiT-XL/2 block linears, W8A8, CFG-paired M=4096",
        M=4096,
        layers=tuple(Layer(n, k, nn, x_kind="gelu_outliers", cfg=True) for n, k, nn in DIT_SHAPES))


def _c3() -> Workload:
    return Workload(
        key="c3", title="DiT-XL/2 block linears, W4A4 + block Hadamard 128 on X and W, CFG-paired M=4096",
        M=4096,
        layers=tuple(Layer(n, k, nn, w_bits=4, a_bits=4, hadamard_block=128,
                           x_kind="gelu_outliers", cfg=True) for n, k, nn in DIT_SHAPES))


def c3_single() -> Tuple[Layer, ...]:
    """The c3 stack with HQ-DM's single transform: X rotated, W quantized
    unrotated, symmetric activation scales (same inputs as c3)."""
    import dataclasses
    return tuple(dataclasses.replace(L, a_scale="symmetric", single_hadamard=True)
                 for L in WORKLOADS["c3"].layers)


def c4_a8_mask(seed: int = SEED) -> np.ndarray:
    return synth.half_mask(seed, "c4/a8mask", len(MMDIT_SHAPES))


def _c4() -> Workload:
    mask = c4_a8_mask()
    layers = []
    for i, (n, k, nn, segs) in enumerate(MMDIT_SHAPES):
        layers.append(Layer(n, k, nn, w_bits=4, a_bits=8 if mask[i] else 4,
                            n_segments=segs, w_scale="segment" if segs > 1 else "channel",
                            x_dtype="bf16", x_kind="bf16_normal", cfg=False))
    return Workload(
        key="c4", title="MM-DiT SegLinear layers, W4 with per-layer A4/A8, M=18432, bf16 inputs",
        M=18432, layers=tuple(layers))


def _c5() -> Workload:
    return Workload(
        key="c5", title="TASQ sweep: 28 DiT-XL/2 blocks x 4 linears, 50 steps, k in {0,2,4}",
        M=4096,
        layers=tuple(Layer(f"b{b}.{n}", k, nn, x_kind="silu", cfg=True)
                     for b in range(28) for n, k, nn in DIT_SHAPES),
        steps=50, lsb_choices=(0, 2, 4))


def _c6() -> Workload:
    return Workload(
        key="c6", title="TASQ weight-side sweep: 28 DiT-XL/2 blocks x 4 linears, 50 steps in 4 "
                        "stages, one stored W8 buffer per linear, weight LSB depth per (stage, "
                        "layer) in {0,2,4}, per-step static activation scales",
        M=4096,
        layers=tuple(Layer(f"b{b}.{n}", k, nn, x_kind="silu", cfg=True)
                     for b in range(28) for n, k, nn in DIT_SHAPES),
        steps=50, lsb_choices=(0, 2, 4), stages=4)


def _c7() -> Workload:
    return Workload(
        key="c7", title="SegLinear input branches at DiT-XL/2 width, W8A8 DualScale, CFG-paired "
                        "M=4096: a skip fusion [hidden 1152 | skip 1152] -> 1152 and a "
                        "conditioning fusion [timestep embedding 256 | hidden 1152] -> 1152",
        M=4096,
        layers=(Layer("skip", 2304, 1152, x_kind="branches", cfg=True, k_seg=(0, 1152, 2304),
                      branch_kinds=("gelu_outliers", "silu")),
                Layer("temb", 1408, 1152, x_kind="branches", cfg=True, k_seg=(0, 256, 1408),
                      branch_kinds=("sinusoid", "gelu_outliers"))))


WORKLOADS = {w.key: w for w in (_c1(), _c2(), _c3(), _c4(), _c5(), _c6(), _c7())}


def c6_w_schedule(seed: int = SEED) -> np.ndarray:
    """int32 [4, 112]: weight LSB depth per (stage, layer), uniform over {0,2,4}."""
    w = WORKLOADS["c6"]
    return synth.uniform_choice_schedule(seed, "c6/wlsb", w.stages, len(w.layers), w.lsb_choices)


def c4_gamp_inputs(seed: int = SEED):
    """Inputs of the activation-bit allocation for the MM-DiT stack: per-layer
    MACs of the whole step (M rows, both CFG halves), seeded synthetic
    sensitivities (log-normal, one per layer), and a budget of 6 activation
    bits on average by MACs at 4-bit weights."""
    wl = WORKLOADS["c4"]
    macs = np.array([wl.M * L.N * L.K for L in wl.layers], np.int64)
    gain = synth.lognormal(seed, "c4/gamp/gain", len(wl.layers))
    budget = int(macs.sum()) * 4 * 6
    return wl, macs, gain, budget


def stage_of(wl: Workload, t: int) -> int:
    """Denoising stage of step t: the steps split into `stages` runs of
    consecutive steps, as equal as the step count allows."""
    return t * wl.stages // wl.steps


def make_calib_x(wl: Workload, layer: Layer, step: int, seed: int = SEED) -> np.ndarray:
    """Calibration input of a layer at a step, drawn apart from the run's inputs."""
    return synth.silu_normal(seed, f"{wl.key}/calib/t{step}/{layer.name}/X", wl.M, layer.K)


def c5_schedule(seed: int = SEED) -> np.ndarray:
    """int32 [50, 112]: LSB truncation depth per (step, layer), uniform over {0,2,4}."""
    w = WORKLOADS["c5"]
    return synth.uniform_choice_schedule(seed, "c5/lsb", w.steps, len(w.layers), w.lsb_choices)


def make_x(wl: Workload, layer: Layer, M: Optional[int] = None, step: Optional[int] = None,
           seed: int = SEED) -> np.ndarray:
    """Activation input for one layer: fp32 [M,K], or uint16 bf16 bits for bf16 layers."""
    M = wl.M if M is None else M
    name = f"{wl.key}/{layer.name}/X" if step is None else f"{wl.key}/t{step}/{layer.name}/X"
    if layer.x_kind == "silu":
        return synth.silu_normal(seed, name, M, layer.K)
    if layer.x_kind == "gelu_outliers":
        return synth.gelu_with_outliers(seed, name, M, layer.K)
    if layer.x_kind == "bf16_normal":
        return synth.bf16_normal(seed, name, M, layer.K)
    if layer.x_kind == "branches":
        gen = {"silu": synth.silu_normal, "gelu_outliers": synth.gelu_with_outliers,
               "sinusoid": synth.sinusoid}
        return np.concatenate(
            [gen[kd](seed, f"{name}/b{j}", M, b - a) for j, (kd, a, b) in
             enumerate(zip(layer.branch_kinds, layer.k_seg[:-1], layer.k_seg[1:]))], axis=1)
    raise ValueError(layer.x_kind)


def make_w(wl: Workload, layer: Layer, seed: int = SEED) -> np.ndarray:
    return synth.weight_normal(seed, f"{wl.key}/{layer.name}/W", layer.N, layer.K)
