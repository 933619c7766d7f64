"""ctypes binding of libqlinear.so (declared in include/qlinear.h).

Argument marshalling only: every step of the quantized linear runs in the
library's HIP kernels. The library is loaded from this package directory;
if it has not been built, loading raises instead of falling back to
anything else.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlinear.so")

QL_OK, QL_ERR_ARG, QL_ERR_UNSUPPORTED, QL_ERR_OOM, QL_ERR_HIP = range(5)
QL_F32, QL_BF16 = 0, 1
QL_WSCALE_PER_TENSOR, QL_WSCALE_PER_SEGMENT, QL_WSCALE_PER_CHANNEL = 0, 1, 2
QL_ASCALE_DUAL, QL_ASCALE_SYMMETRIC = 0, 1

EXPORTS = (
    "qlinear_plan", "qlinear_plan_destroy", "qlinear_plan_weights", "qlinear_quantize_act",
    "qlinear_gemm", "qlinear_cfg_combine", "qlinear_last_error", "qlinear_version",
    "qlinear_plan_lsb_view", "qlinear_plan_lsb_update", "qlinear_gamp_allocate",
    "qlinear_quantize_act_noalloc", "qlinear_probe_mfma",
)


class QlDesc(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("w_bits", ctypes.c_int32), ("a_bits", ctypes.c_int32),
        ("hadamard_block", ctypes.c_int32), ("n_segments", ctypes.c_int32),
        ("seg_offsets", ctypes.POINTER(ctypes.c_int32)),
        ("w_scale_mode", ctypes.c_int), ("a_scale_mode", ctypes.c_int),
        ("x_dtype", ctypes.c_int), ("single_hadamard", ctypes.c_int32),
        ("n_k_segments", ctypes.c_int32), ("k_seg_offsets", ctypes.POINTER(ctypes.c_int32)),
    ]


class QLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qlinear status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libqlinear.so (built in-tree by the package's _build.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m bit_post_quantization_amd._build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    sig = {
        "qlinear_plan": ([ctypes.POINTER(QlDesc), P, P, ctypes.POINTER(P)], ctypes.c_int),
        "qlinear_plan_destroy": ([P], ctypes.c_int),
        "qlinear_plan_weights": ([P, P, P, P], ctypes.c_int),
        "qlinear_plan_lsb_view": ([P, I32, P, ctypes.POINTER(P)], ctypes.c_int),
        "qlinear_plan_lsb_update": ([P, P, I32, P], ctypes.c_int),
        "qlinear_gamp_allocate": ([I32, P, P, I32, ctypes.c_int64, P, P], ctypes.c_int),
        "qlinear_quantize_act": ([P, P, I32, I32, P, P, P, P], ctypes.c_int),
        "qlinear_quantize_act_noalloc": ([P, P, I32, I32, P, P, P, P], ctypes.c_int),
        "qlinear_gemm": ([P, P, P, I32, I32, F32, P, P, P], ctypes.c_int),
        "qlinear_cfg_combine": ([P, I32, I32, F32, P, P], ctypes.c_int),
        "qlinear_probe_mfma": ([P, I32, I32, P, ctypes.c_int64, P], ctypes.c_int),
        "qlinear_last_error": ([], ctypes.c_char_p),
        "qlinear_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def check(status: int) -> None:
    if status != QL_OK:
        msg = load().qlinear_last_error().decode()
        raise QLError(status, msg)
