"""Build libqlinear.so in-tree with hipcc for gfx950 (MI355X)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_obj")
LIB = os.path.join(PKG, "libqlinear.so")
ARCH = "gfx950"

SOURCES = ["k_quant.hip", "k_gemm.hip", "k_gemm1.hip", "k_misc.hip", "k_probe.hip",
           "qlinear_api.cpp", "gamp.cpp"]

# -ffp-contract=off: the epilogue's multiply-then-add order is part of the
# numerics (no fused multiply-add). Correctly rounded fp32 division is the
# HIP default and stated explicitly. Packed fp32 VALU ops are disabled.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


# The single-Hadamard GEMM keeps its MFMA accumulators in architectural
# VGPRs: with AGPR accumulators the register allocator rotates them through
# copies inside its unrolled K loop.
EXTRA = {"k_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# k_gemm1.hip is compiled once per (4-bit activations, symmetric scales)
# pair, so its instantiations build in parallel.
VARIANTS = {"k_gemm1.hip": [(f"k_gemm1_a{a}_s{s}", [f"-DQL_G1_A4={a}", f"-DQL_G1_SYM={s}"])
                            for a in (0, 1) for s in (0, 1)]}


def units():
    """(source, object name, extra flags) of every object in the library."""
    out = []
    for src in SOURCES:
        for name, flags in VARIANTS.get(src, [(os.path.splitext(src)[0], [])]):
            out.append((src, name, EXTRA.get(src, []) + flags))
    return out


def _compile(unit) -> str:
    src, name, extra = unit
    obj = os.path.join(OBJ, name + ".o")
    cmd = ([hipcc()] + FLAGS + extra
           + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link libqlinear.so (always rebuilds)."""
    os.makedirs(OBJ, exist_ok=True)
    us = units()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(us))) as ex:
        objs = list(ex.map(_compile, us))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
