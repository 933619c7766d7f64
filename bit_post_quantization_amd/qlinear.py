"""Python binding of the C ABI, function for function (same names).

Tensors are passed as device pointers (``tensor.data_ptr()``) and the stream
as ``torch.cuda.current_stream().cuda_stream`` unless given. PyTorch is used
for device memory and streams only; all arithmetic runs in libqlinear's HIP
kernels. Every call raises QLError on a non-OK status.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

from . import _lib
from ._lib import QLError, QlDesc, check  # noqa: F401

_WMODES = {"tensor": _lib.QL_WSCALE_PER_TENSOR, "segment": _lib.QL_WSCALE_PER_SEGMENT,
           "channel": _lib.QL_WSCALE_PER_CHANNEL}
_AMODES = {"dual": _lib.QL_ASCALE_DUAL, "symmetric": _lib.QL_ASCALE_SYMMETRIC}
_DTYPES = {"f32": _lib.QL_F32, "bf16": _lib.QL_BF16}


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owner of a qlinear_plan_t handle (destroyed with the object)."""

    def __init__(self, handle: int, desc: dict):
        self.handle = handle
        self.desc = desc

    def destroy(self):
        if self.handle:
            check(_lib.load().qlinear_plan_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def qlinear_plan(W, N: int, K: int, w_bits: int = 8, a_bits: int = 8, hadamard_block: int = 0,
                 seg_offsets: Optional[Sequence[int]] = None, w_scale: str = "channel",
                 a_scale: str = "dual", x_dtype: str = "f32", stream=None,
                 single_hadamard: bool = False,
                 k_seg_offsets: Optional[Sequence[int]] = None) -> Plan:
    L = _lib.load()
    segs = None
    nseg = 1
    if seg_offsets is not None:
        nseg = len(seg_offsets) - 1
        segs = (ctypes.c_int32 * len(seg_offsets))(*[int(v) for v in seg_offsets])
    ksegs = None
    nks = 0
    if k_seg_offsets is not None:
        nks = len(k_seg_offsets) - 1
        ksegs = (ctypes.c_int32 * len(k_seg_offsets))(*[int(v) for v in k_seg_offsets])
    d = QlDesc(N=N, K=K, w_bits=w_bits, a_bits=a_bits, hadamard_block=hadamard_block,
               n_segments=nseg,
               seg_offsets=ctypes.cast(segs, ctypes.POINTER(ctypes.c_int32)) if segs else None,
               w_scale_mode=_WMODES[w_scale], a_scale_mode=_AMODES[a_scale],
               x_dtype=_DTYPES[x_dtype], single_hadamard=int(bool(single_hadamard)),
               n_k_segments=nks,
               k_seg_offsets=ctypes.cast(ksegs, ctypes.POINTER(ctypes.c_int32)) if ksegs else None)
    h = ctypes.c_void_p()
    check(L.qlinear_plan(ctypes.byref(d), _ptr(W), _stream(stream), ctypes.byref(h)))
    return Plan(h.value, dict(N=N, K=K, w_bits=w_bits, a_bits=a_bits,
                              hadamard_block=hadamard_block, seg_offsets=seg_offsets,
                              w_scale=w_scale, a_scale=a_scale, x_dtype=x_dtype,
                              single_hadamard=bool(single_hadamard),
                              k_seg_offsets=k_seg_offsets))


def qlinear_plan_destroy(plan: Plan) -> None:
    plan.destroy()


def qlinear_plan_weights(plan: Plan, w_codes, w_scales, stream=None) -> None:
    check(_lib.load().qlinear_plan_weights(plan.handle, _ptr(w_codes), _ptr(w_scales),
                                           _stream(stream)))


def qlinear_plan_lsb_view(base: Plan, w_lsb_k: int, stream=None) -> Plan:
    h = ctypes.c_void_p()
    check(_lib.load().qlinear_plan_lsb_view(base.handle, w_lsb_k, _stream(stream),
                                            ctypes.byref(h)))
    return Plan(h.value, dict(base.desc))


def qlinear_plan_lsb_update(view: Plan, base: Plan, w_lsb_k: int, stream=None) -> None:
    check(_lib.load().qlinear_plan_lsb_update(view.handle, base.handle, w_lsb_k,
                                              _stream(stream)))


def qlinear_quantize_act(plan: Plan, X, M: int, lsb_k: int, static_scales, codes, act_scales,
                         stream=None) -> None:
    check(_lib.load().qlinear_quantize_act(plan.handle, _ptr(X), M, lsb_k, _ptr(static_scales),
                                           _ptr(codes), _ptr(act_scales), _stream(stream)))


def qlinear_quantize_act_noalloc(plan: Plan, X, M: int, lsb_k: int, static_scales, codes,
                                 act_scales, stream=None) -> None:
    check(_lib.load().qlinear_quantize_act_noalloc(plan.handle, _ptr(X), M, lsb_k,
                                                   _ptr(static_scales), _ptr(codes),
                                                   _ptr(act_scales), _stream(stream)))


def qlinear_gemm(plan: Plan, codes, act_scales, M: int, cfg: int, w: float, Y, acc_dbg=None,
                 stream=None) -> None:
    check(_lib.load().qlinear_gemm(plan.handle, _ptr(codes), _ptr(act_scales), M, cfg, float(w),
                                   _ptr(Y), _ptr(acc_dbg), _stream(stream)))


def qlinear_cfg_combine(Y, M: int, N: int, w: float, out, stream=None) -> None:
    check(_lib.load().qlinear_cfg_combine(_ptr(Y), M, N, float(w), _ptr(out), _stream(stream)))


def qlinear_probe_mfma(operands, iters: int, waves_per_simd: int, sink, stream=None) -> None:
    """Measurement aid: the int8 MFMA ceiling microkernel (include/qlinear.h)."""
    check(_lib.load().qlinear_probe_mfma(_ptr(operands), iters, waves_per_simd, _ptr(sink),
                                         sink.numel(), _stream(stream)))


def qlinear_gamp_allocate(macs, gain, w_bits: int, budget_bops: int):
    """Host-only: (a_bits list, total BOPs) of the greedy A4->A8 allocation."""
    n = len(macs)
    m = (ctypes.c_int64 * n)(*[int(v) for v in macs])
    g = (ctypes.c_double * n)(*[float(v) for v in gain])
    a = (ctypes.c_int32 * n)()
    b = ctypes.c_int64(0)
    check(_lib.load().qlinear_gamp_allocate(n, m, g, w_bits, int(budget_bops), a,
                                            ctypes.byref(b)))
    return list(a), int(b.value)


def qlinear_version() -> str:
    return _lib.load().qlinear_version().decode()


class QuantLinear:
    """One quantized linear layer: a plan plus output allocation helpers.

    ``forward`` enqueues the quantize and GEMM calls; the tensors it returns
    are allocated with torch on the current device (allocation only)."""

    def __init__(self, W, w_bits=8, a_bits=8, hadamard_block=0, seg_offsets=None,
                 w_scale="channel", a_scale="dual", x_dtype="f32", stream=None,
                 single_hadamard=False, k_seg_offsets=None):
        N, K = W.shape
        self.N, self.K = int(N), int(K)
        self.a_bits, self.w_bits = a_bits, w_bits
        self.nks = 1 if k_seg_offsets is None else len(k_seg_offsets) - 1
        self.plan = qlinear_plan(W, self.N, self.K, w_bits, a_bits, hadamard_block, seg_offsets,
                                 w_scale, a_scale, x_dtype, stream, single_hadamard,
                                 k_seg_offsets)
        self.base = None

    def lsb_view(self, w_lsb_k: int, stream=None) -> "QuantLinear":
        """The same layer run with w_lsb_k low bits of every weight code
        dropped; ``update_lsb`` changes the depth later without allocating."""
        v = QuantLinear.__new__(QuantLinear)
        v.N, v.K, v.a_bits, v.w_bits, v.nks = self.N, self.K, self.a_bits, self.w_bits, self.nks
        v.plan = qlinear_plan_lsb_view(self.plan, w_lsb_k, stream)
        v.base = self
        return v

    def update_lsb(self, w_lsb_k: int, stream=None) -> None:
        qlinear_plan_lsb_update(self.plan, self.base.plan, w_lsb_k, stream)

    def code_shape(self, M: int):
        return (M, self.K if self.a_bits == 8 else self.K // 2)

    def alloc_codes(self, M: int):
        import torch
        dt = torch.int8 if self.a_bits == 8 else torch.uint8
        return torch.empty(self.code_shape(M), dtype=dt, device="cuda")

    def quantize(self, X, lsb_k=0, static_scales=None, codes=None, act_scales=None, stream=None):
        import torch
        M = X.shape[0]
        codes = self.alloc_codes(M) if codes is None else codes
        act_scales = (torch.empty(2 * self.nks, dtype=torch.float32, device="cuda")
                      if act_scales is None else act_scales)
        qlinear_quantize_act(self.plan, X, M, lsb_k, static_scales, codes, act_scales, stream)
        return codes, act_scales

    def gemm(self, codes, act_scales, cfg=0, w=1.0, Y=None, acc_dbg=None, stream=None):
        import torch
        M = codes.shape[0]
        if Y is None:
            Y = torch.empty((M // 2 if cfg else M, self.N), dtype=torch.float32, device="cuda")
        qlinear_gemm(self.plan, codes, act_scales, M, cfg, w, Y, acc_dbg, stream)
        return Y

    def forward(self, X, lsb_k=0, cfg=0, w=1.0, static_scales=None, stream=None):
        codes, s = self.quantize(X, lsb_k, static_scales, stream=stream)
        return self.gemm(codes, s, cfg, w, stream=stream)

    def weights(self, stream=None):
        import torch
        wc = torch.empty((self.N, self.K), dtype=torch.int8, device="cuda")
        sw = torch.empty(self.N * self.nks, dtype=torch.float32, device="cuda")
        qlinear_plan_weights(self.plan, wc, sw, stream)
        return wc, (sw.view(self.nks, self.N) if self.nks > 1 else sw)
