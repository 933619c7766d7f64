"""Helpers for the GPU-vs-oracle parity tests.

Comparison rules:
  * integer codes and int32 accumulators are bit-exact, except codes whose
    pre-rounding value x/s (recomputed in float64 from the same fp32 x and s)
    lies within 1e-6 relative of a rounding boundary; those are counted and
    must be at most 1e-5 of all codes;
  * fp32 outputs: max elementwise relative error <= 1e-5 (denominator
    max(|ref|, FLT_MIN)); the implementation aims at bit-exactness.
Accumulators are compared by feeding the GPU's codes to the oracle GEMM, and
outputs by feeding the GPU's accumulators to the oracle epilogue, so each
stage is checked on its own inputs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np

import oracle

FLT_MIN = np.float32(np.finfo(np.float32).tiny)
CODE_FLAG_REL = 1e-6
CODE_FLAG_FRAC = 1e-5
Y_REL_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def unpack_codes(codes: np.ndarray, K: int, a_bits: int) -> np.ndarray:
    if a_bits == 8:
        return codes.view(np.int8).reshape(-1, K)
    return oracle.unpack_int4(codes.view(np.uint8).reshape(-1, K // 2), K)


def compare_codes(gpu: np.ndarray, ref: np.ndarray, x_rot: np.ndarray, s: np.ndarray) -> dict:
    """gpu/ref int8 unpacked codes; x_rot the (rotated) fp32 values."""
    gpu = gpu.reshape(-1)
    ref = ref.reshape(-1)
    mism = np.nonzero(gpu != ref)[0]
    flagged = 0
    if mism.size:
        x = x_rot.reshape(-1)[mism].astype(np.float64)
        sel = np.where(x >= 0, s[0], s[1]).astype(np.float64)
        v = x / sel
        near = np.abs(v - (np.floor(v) + 0.5)) <= CODE_FLAG_REL * np.abs(v)
        flagged = int(near.sum())
        unflagged = int((~near).sum())
    else:
        unflagged = 0
    return dict(n=int(gpu.size), mismatched=int(mism.size), flagged=flagged, unflagged=unflagged)


def compare_codes_scaled(gpu: np.ndarray, ref: np.ndarray, x_rot: np.ndarray,
                         s_el: np.ndarray) -> dict:
    """As compare_codes, with a scale pair per element: s_el [M, K, 2]."""
    gpu = gpu.reshape(-1)
    ref = ref.reshape(-1)
    mism = np.nonzero(gpu != ref)[0]
    flagged = unflagged = 0
    if mism.size:
        x = x_rot.reshape(-1)[mism].astype(np.float64)
        se = s_el.reshape(-1, 2)[mism]
        sel = np.where(x >= 0, se[:, 0], se[:, 1]).astype(np.float64)
        v = x / sel
        near = np.abs(v - (np.floor(v) + 0.5)) <= CODE_FLAG_REL * np.abs(v)
        flagged = int(near.sum())
        unflagged = int((~near).sum())
    return dict(n=int(gpu.size), mismatched=int(mism.size), flagged=flagged, unflagged=unflagged)


def assert_codes(stats: dict, what: str = "codes"):
    assert stats["unflagged"] == 0, f"{what}: {stats}"
    assert stats["flagged"] <= CODE_FLAG_FRAC * stats["n"], f"{what}: {stats}"


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    den = np.maximum(np.abs(r), float(FLT_MIN))
    return float(np.max(np.abs(g - r) / den)) if r.size else 0.0


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    e = rel_err(gpu, ref)
    assert e <= Y_REL_TOL, f"{what}: max rel err {e}"
    return e


def oracle_threads() -> int:
    """Worker threads for running the single-threaded oracle on disjoint row
    shards (at most 16: the CPU share of one GPU on the test hosts)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _sharded(fn, rows, *args):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    P = oracle_threads()
    shards = [r for r in np.array_split(rows, P) if r.size]
    if len(shards) <= 1:
        return [fn(*args, rows)]
    with cf.ThreadPoolExecutor(max_workers=len(shards)) as ex:
        return list(ex.map(lambda r: fn(*args, r), shards))


def gemm_dual_rows(codes: np.ndarray, wc: np.ndarray, rows) -> tuple:
    """oracle.gemm_dual over the listed rows, the rows split into shards that
    independent threads run through the (single-threaded) oracle; the oracle
    releases the interpreter lock while it computes."""
    parts = _sharded(oracle.gemm_dual, rows, np.ascontiguousarray(codes, dtype=np.int8),
                     np.ascontiguousarray(wc, dtype=np.int8))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def gemm_int64_rows(codes: np.ndarray, v: np.ndarray, rows) -> np.ndarray:
    """oracle.gemm_int64 over the listed rows, sharded over threads as above."""
    parts = _sharded(oracle.gemm_int64, rows, np.ascontiguousarray(codes, dtype=np.int8),
                     np.ascontiguousarray(v, dtype=np.int32))
    return np.concatenate(parts)
