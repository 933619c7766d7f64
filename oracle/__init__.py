"""CPU oracle for the quantized linear layer (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package. It wraps ``liboracle.so`` (plain single-threaded
C++ built from ``oracle.cpp`` with g++ -O2 -ffp-contract=off) through ctypes
and composes its steps in the order the pages give them:

  1. optional block Walsh-Hadamard rotation (HQ-DM, technical summary 2.1),
  2. DualScale per-tensor act scales and codes (SegQuant, section 2.B),
  3. optional LSB truncation of the codes (TASQ, section 2),
  4. weight scales per channel / output segment / tensor (SegQuant, 2.A),
  5. the two integer contractions and the fp32 epilogue (SegQuant, 2.B),
  6. the classifier-free-guidance combine (Closing the Null Space, problem
     statement).

It shares no code with the GPU library and never calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
# ORACLE_LIB selects another build of the same source (the sanitizer build).
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")

DUAL, SYMMETRIC = 0, 1
W_TENSOR, W_SEGMENT, W_CHANNEL = 0, 1, 2
_WMODES = {"tensor": W_TENSOR, "segment": W_SEGMENT, "channel": W_CHANNEL}
_AMODES = {"dual": DUAL, "symmetric": SYMMETRIC}


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile liboracle.so with the host compiler (plain C++17); with
    sanitize, liboracle_san.so under AddressSanitizer and
    UndefinedBehaviorSanitizer (any report aborts), for running the pins
    under them with the ASan runtime preloaded."""
    out = _SAN_LIB if sanitize else os.path.join(_HERE, "liboracle.so")
    if not force and os.path.exists(out):
        return out
    flags = ["-O2"]
    if sanitize:
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all"]
    cmd = (["g++", "-std=c++17"] + flags + ["-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", out + ".tmp", _SRC])
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False, sanitize=_LIB == _SAN_LIB)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I32, I64, F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sigs = {
            "orc_fwht_block": [P, I32],
            "orc_rotate_rows": [P, I64, I64, I32],
            "orc_act_scales": [P, I64, I32, I32, P],
            "orc_quant_value": [F32, F32, F32, I32],
            "orc_truncate_lsb": [I32, I32],
            "orc_quantize_act": [P, I64, P, I32, I32, P],
            "orc_truncate_codes": [P, I64, I32, I32, P],
            "orc_pack_int4": [P, I64, I64, P],
            "orc_unpack_int4": [P, I64, I64, P],
            "orc_weight_scales": [P, I64, I64, I32, I32, I32, P, P],
            "orc_quantize_weight": [P, I64, I64, P, I32, P],
            "orc_gemm_dual": [P, P, P, I64, I64, I64, P, P],
            "orc_epilogue": [P, P, I64, I64, P, P, I32, I32, P],
            "orc_cfg_combine": [P, P, I64, I64, F32, P],
            "orc_bf16_to_f32": [P, I64, P],
            "orc_gamp_allocate": [I32, P, P, I32, I64, P, P],
            "orc_hadamard_weight_int": [P, I64, I64, I32, P],
            "orc_gemm_int64": [P, P, P, I64, I64, I64, P],
            "orc_epilogue_single": [P, I64, I64, F32, P, I32, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I32
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ck(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with oracle code {rc}")


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def qmax(bits: int) -> int:
    return (1 << (bits - 1)) - 1


# ----------------------------------------------------------------- steps ----

def fwht_block(v: np.ndarray) -> np.ndarray:
    out = np.array(v, dtype=np.float32, copy=True)
    _ck(lib().orc_fwht_block(_p(out), out.size), "fwht_block")
    return out


def rotate(x: np.ndarray, B: int) -> np.ndarray:
    """Rows of x [rows, K] rotated block-wise by the unnormalised H_B (copy)."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    rows, K = out.shape
    _ck(lib().orc_rotate_rows(_p(out), rows, K, B), "rotate_rows")
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    _ck(lib().orc_bf16_to_f32(_p(b), b.size, _p(out)), "bf16_to_f32")
    return out


def act_scales(x: np.ndarray, a_bits: int, mode: str = "dual") -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.zeros(2, dtype=np.float32)
    _ck(lib().orc_act_scales(_p(x), x.size, a_bits, _AMODES[mode], _p(s)), "act_scales")
    return s


def quant_value(v: float, sp: float, sn: float, bits: int) -> int:
    return int(lib().orc_quant_value(v, sp, sn, qmax(bits)))


def truncate_lsb(c: int, k: int) -> int:
    return int(lib().orc_truncate_lsb(int(c), int(k)))


def truncate_codes(codes: np.ndarray, w_bits: int, k: int) -> np.ndarray:
    """Stored weight codes -> operating codes with k low magnitude bits dropped."""
    c = np.ascontiguousarray(codes, dtype=np.int8)
    out = np.empty_like(c)
    _ck(lib().orc_truncate_codes(_p(c), c.size, w_bits, k, _p(out)), "truncate_codes")
    return out


def quantize_act(x: np.ndarray, s: np.ndarray, a_bits: int, lsb_k: int = 0) -> np.ndarray:
    """Signed codes (int8, unpacked) for fp32 x with scales s = (s+, s-)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    c = np.empty(x.shape, dtype=np.int8)
    _ck(lib().orc_quantize_act(_p(x), x.size, _p(s), a_bits, lsb_k, _p(c)), "quantize_act")
    return c


def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    rows, K = codes.shape
    out = np.empty((rows, K // 2), dtype=np.uint8)
    _ck(lib().orc_pack_int4(_p(codes), rows, K, _p(out)), "pack_int4")
    return out


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    out = np.empty((rows, K), dtype=np.int8)
    _ck(lib().orc_unpack_int4(_p(packed), rows, K, _p(out)), "unpack_int4")
    return out


def weight_scales(w: np.ndarray, w_bits: int, mode: str = "channel",
                  seg_offsets: Optional[Sequence[int]] = None) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    sw = np.empty(N, dtype=np.float32)
    seg = None if seg_offsets is None else np.ascontiguousarray(seg_offsets, dtype=np.int32)
    nseg = 1 if seg is None else seg.size - 1
    _ck(lib().orc_weight_scales(_p(w), N, K, w_bits, _WMODES[mode], nseg, _p(seg), _p(sw)),
        "weight_scales")
    return sw


def quantize_weight(w: np.ndarray, sw: np.ndarray, w_bits: int) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    N, K = w.shape
    wc = np.empty((N, K), dtype=np.int8)
    _ck(lib().orc_quantize_weight(_p(w), N, K, _p(sw), w_bits, _p(wc)), "quantize_weight")
    return wc


def gemm_dual(codes: np.ndarray, wc: np.ndarray, rows: Optional[Sequence[int]] = None):
    """(acc+, acc-) int32 [len(rows), N] for the listed rows of codes [M,K]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    wc = np.ascontiguousarray(wc, dtype=np.int8)
    M, K = codes.shape
    N = wc.shape[0]
    assert wc.shape[1] == K
    r = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    accp = np.empty((r.size, N), dtype=np.int32)
    accn = np.empty((r.size, N), dtype=np.int32)
    _ck(lib().orc_gemm_dual(_p(codes), _p(wc), _p(r), r.size, N, K, _p(accp), _p(accn)),
        "gemm_dual")
    return accp, accn


def epilogue(accp: np.ndarray, accn: np.ndarray, s: np.ndarray, sw: np.ndarray,
             B: int = 0, mode: str = "dual") -> np.ndarray:
    accp = np.ascontiguousarray(accp, dtype=np.int32)
    accn = np.ascontiguousarray(accn, dtype=np.int32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    rows, N = accp.shape
    y = np.empty((rows, N), dtype=np.float32)
    _ck(lib().orc_epilogue(_p(accp), _p(accn), rows, N, _p(s), _p(sw), B, _AMODES[mode], _p(y)),
        "epilogue")
    return y


def cfg_combine(y_c: np.ndarray, y_u: np.ndarray, w: float) -> np.ndarray:
    y_c = np.ascontiguousarray(y_c, dtype=np.float32)
    y_u = np.ascontiguousarray(y_u, dtype=np.float32)
    assert y_c.shape == y_u.shape
    rows, N = y_c.shape
    out = np.empty_like(y_c)
    _ck(lib().orc_cfg_combine(_p(y_c), _p(y_u), rows, N, float(w), _p(out)), "cfg_combine")
    return out


def hadamard_weight_int(wc: np.ndarray, B: int) -> np.ndarray:
    """int32 [N,K] = H W_int^T laid out as rows (single-Hadamard weights)."""
    wc = np.ascontiguousarray(wc, dtype=np.int8)
    N, K = wc.shape
    v = np.empty((N, K), dtype=np.int32)
    _ck(lib().orc_hadamard_weight_int(_p(wc), N, K, B, _p(v)), "hadamard_weight_int")
    return v


def gemm_int64(codes: np.ndarray, v: np.ndarray, rows: Optional[Sequence[int]] = None):
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    v = np.ascontiguousarray(v, dtype=np.int32)
    M, K = codes.shape
    N = v.shape[0]
    assert v.shape[1] == K
    r = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    acc = np.empty((r.size, N), dtype=np.int64)
    _ck(lib().orc_gemm_int64(_p(codes), _p(v), _p(r), r.size, N, K, _p(acc)), "gemm_int64")
    return acc


def epilogue_single(acc: np.ndarray, s: float, sw: np.ndarray, B: int) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    rows, N = acc.shape
    y = np.empty((rows, N), dtype=np.float32)
    _ck(lib().orc_epilogue_single(_p(acc), rows, N, float(s), _p(sw), B, _p(y)),
        "epilogue_single")
    return y


class SingleHadamardPlan:
    """[HQ] 2.1 single transform: W quantized unrotated (per channel /
    segment / tensor), its codes kept, and the integer weights H W_int^T."""

    def __init__(self, W: np.ndarray, w_bits: int, B: int, mode: str = "channel",
                 seg_offsets: Optional[Sequence[int]] = None):
        self.w_bits, self.B = w_bits, B
        W = np.ascontiguousarray(W, dtype=np.float32)
        self.scales = weight_scales(W, w_bits, mode, seg_offsets)
        self.codes = quantize_weight(W, self.scales, w_bits)
        self.v = hadamard_weight_int(self.codes, B)

    def truncated(self, k: int) -> "SingleHadamardPlan":
        p = SingleHadamardPlan.__new__(SingleHadamardPlan)
        p.w_bits, p.B, p.scales = self.w_bits, self.B, self.scales
        p.codes = truncate_codes(self.codes, self.w_bits, k)
        p.v = hadamard_weight_int(p.codes, self.B)
        return p


def gamp_allocate(macs, gain, w_bits: int, budget: int):
    """(a_bits int32 [n], total BOPs) of the greedy A4->A8 allocation."""
    macs = np.ascontiguousarray(macs, dtype=np.int64)
    gain = np.ascontiguousarray(gain, dtype=np.float64)
    assert macs.shape == gain.shape and macs.ndim == 1
    a = np.empty(macs.size, dtype=np.int32)
    b = np.zeros(1, dtype=np.int64)
    _ck(lib().orc_gamp_allocate(macs.size, _p(macs), _p(gain), w_bits, int(budget), _p(a), _p(b)),
        "gamp_allocate")
    return a, int(b[0])


# --------------------------------------------------------------- pipeline ----

class WeightPlan:
    """Oracle weights for one linear: codes int8 [N,K] and scales [N]."""

    def __init__(self, W: np.ndarray, w_bits: int, B: int = 0, mode: str = "channel",
                 seg_offsets: Optional[Sequence[int]] = None):
        Wr = rotate(W, B) if B else np.ascontiguousarray(W, dtype=np.float32)
        self.w_bits, self.B = w_bits, B
        self.scales = weight_scales(Wr, w_bits, mode, seg_offsets)
        self.codes = quantize_weight(Wr, self.scales, w_bits)

    def truncated(self, k: int) -> "WeightPlan":
        """The same layer at an operating precision with k dropped bits."""
        v = WeightPlan.__new__(WeightPlan)
        v.w_bits, v.B, v.scales = self.w_bits, self.B, self.scales
        v.codes = truncate_codes(self.codes, self.w_bits, k)
        return v


class InputSegmentedPlan:
    """[SQ] 2.A, input segmentation: the input is a concatenation of branches
    along K, X = [X_0 | X_1 | ...] at k_offsets, and each branch is quantized
    apart: its weight columns W[:, o_j:o_j+1] get their own scales (per
    channel, output segment or tensor) and, in quantize_activations_segmented,
    its activations their own DualScale pair."""

    def __init__(self, W: np.ndarray, w_bits: int, k_offsets: Sequence[int], B: int = 0,
                 mode: str = "channel", seg_offsets: Optional[Sequence[int]] = None):
        self.w_bits, self.B = w_bits, B
        self.k_offsets = [int(v) for v in k_offsets]
        W = np.ascontiguousarray(W, dtype=np.float32)
        self.parts = [WeightPlan(W[:, a:b], w_bits, B=B, mode=mode, seg_offsets=seg_offsets)
                      for a, b in zip(self.k_offsets[:-1], self.k_offsets[1:])]
        self.codes = np.concatenate([p.codes for p in self.parts], axis=1)
        self.scales = np.stack([p.scales for p in self.parts])  # [S, N]

    def truncated(self, k: int) -> "InputSegmentedPlan":
        v = InputSegmentedPlan.__new__(InputSegmentedPlan)
        v.w_bits, v.B, v.k_offsets = self.w_bits, self.B, self.k_offsets
        v.parts = [p.truncated(k) for p in self.parts]
        v.codes = np.concatenate([p.codes for p in v.parts], axis=1)
        v.scales = self.scales
        return v


def quantize_activations_segmented(X: np.ndarray, a_bits: int, k_offsets: Sequence[int],
                                   B: int = 0, mode: str = "dual", lsb_k: int = 0,
                                   static_scales: Optional[np.ndarray] = None,
                                   bf16: bool = False):
    """Every branch quantized on its own. Returns (codes int8 [M,K], scales [S,2])."""
    codes, scales = [], []
    for j, (a, b) in enumerate(zip(k_offsets[:-1], k_offsets[1:])):
        st = None if static_scales is None else np.asarray(static_scales, np.float32)[j]
        c, sc = quantize_activations(X[:, a:b], a_bits, B=B, mode=mode, lsb_k=lsb_k,
                                     static_scales=st, bf16=bf16)
        codes.append(c)
        scales.append(sc)
    return np.concatenate(codes, axis=1), np.stack(scales)


def linear_segmented_rows(codes: np.ndarray, s: np.ndarray, wp: InputSegmentedPlan,
                          rows: Sequence[int], mode: str = "dual"):
    """y [len(rows), N] = sum over branches, in branch order, of each branch's
    epilogue (fp32 adds), then the rotation's 1/B; plus the per-branch
    accumulators [(acc+, acc-), ...]."""
    y, accs = None, []
    for j, (a, b) in enumerate(zip(wp.k_offsets[:-1], wp.k_offsets[1:])):
        accp, accn = gemm_dual(codes[:, a:b], wp.parts[j].codes, rows)
        accs.append((accp, accn))
        yj = epilogue(accp, accn, s[j], wp.scales[j], 0, mode)
        y = yj if y is None else (y + yj).astype(np.float32)
    if wp.B:
        y = (y * np.float32(1.0 / wp.B)).astype(np.float32)
    return y, accs


def quantize_activations(X: np.ndarray, a_bits: int, B: int = 0, mode: str = "dual",
                         lsb_k: int = 0, static_scales: Optional[np.ndarray] = None,
                         bf16: bool = False):
    """Rotate (optional), take per-tensor scales (or the given static ones),
    quantize and truncate. Returns (codes int8 [M,K], scales [2])."""
    x = bf16_to_f32(X) if bf16 else np.ascontiguousarray(X, dtype=np.float32)
    if B:
        x = rotate(x, B)
    s = (act_scales(x, a_bits, mode) if static_scales is None
         else np.ascontiguousarray(static_scales, dtype=np.float32).copy())
    return quantize_act(x, s, a_bits, lsb_k), s


def linear_rows(codes: np.ndarray, s: np.ndarray, wp: WeightPlan, rows: Sequence[int],
                mode: str = "dual"):
    """Epilogue outputs y [len(rows), N] plus the accumulators for those rows."""
    accp, accn = gemm_dual(codes, wp.codes, rows)
    return epilogue(accp, accn, s, wp.scales, wp.B, mode), accp, accn
