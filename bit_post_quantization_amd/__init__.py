"""MI355X-native quantized linear layer for diffusion transformers.

DualScale (polarity-aware) activation quantization with optional block
Walsh-Hadamard rotation and LSB truncation (of activation codes per call,
of the stored weight codes per step through plan views), an int8-MFMA GEMM
over both polarity planes with per-channel / per-segment weight scales, and
an fp32 epilogue with the classifier-free-guidance combine -- all in hand-written
HIP kernels for gfx950 behind the C ABI of include/qlinear.h.
"""
from .qlinear import (  # noqa: F401
    Plan, QLError, QuantLinear, qlinear_cfg_combine, qlinear_gamp_allocate, qlinear_gemm,
    qlinear_plan,
    qlinear_plan_destroy, qlinear_plan_lsb_update, qlinear_plan_lsb_view, qlinear_plan_weights,
    qlinear_probe_mfma, qlinear_quantize_act, qlinear_quantize_act_noalloc, qlinear_version,
)
