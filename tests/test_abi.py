"""The C-ABI library loads and exports every entry point include/qlinear.h
declares; host-side argument checks reject bad calls before anything
touches a GPU (these run on the CPU)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from bit_post_quantization_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qlinear_\w+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.load()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qlinear_\w+)", out))
    assert exported == set(_declared())


def test_version_string():
    assert "gfx950" in _lib.load().qlinear_version().decode()


def _desc(**kw):
    base = dict(N=64, K=128, w_bits=8, a_bits=8, hadamard_block=0, n_segments=1,
                seg_offsets=None, w_scale_mode=2, a_scale_mode=0, x_dtype=0)
    base.update(kw)
    return _lib.QlDesc(**base)


def _plan_status(d, W=0x1000):
    L = _lib.load()
    h = ctypes.c_void_p()
    st = L.qlinear_plan(ctypes.byref(d) if d is not None else None, W, None, ctypes.byref(h))
    return st, L.qlinear_last_error().decode()


@pytest.mark.parametrize("kw,frag", [
    (dict(N=0), "N = 0"),
    (dict(K=8), "K = 8"),
    (dict(K=70000), "K = 70000"),
    (dict(w_bits=6), "w_bits"),
    (dict(a_bits=2), "a_bits"),
    (dict(K=48, w_bits=4), "multiple of 32"),
    (dict(K=40), "multiple of 16"),
    (dict(hadamard_block=48), "power of two"),
    (dict(K=192, hadamard_block=128), "not a multiple"),
    (dict(w_scale_mode=7), "w_scale_mode"),
    (dict(a_scale_mode=3), "a_scale_mode"),
    (dict(x_dtype=5), "x_dtype"),
    (dict(n_segments=0), "n_segments"),
    (dict(n_segments=2), "seg_offsets is NULL"),
])
def test_plan_rejects_bad_descriptor(kw, frag):
    st, msg = _plan_status(_desc(**kw))
    assert st == _lib.QL_ERR_ARG and frag in msg


def test_plan_rejects_bad_segments():
    for segs in ([0, 32, 32, 64], [0, 40, 30, 64], [1, 32, 64], [0, 32, 60]):
        arr = (ctypes.c_int32 * len(segs))(*segs)
        d = _desc(n_segments=len(segs) - 1, w_scale_mode=1,
                  seg_offsets=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
        st, msg = _plan_status(d)
        assert st == _lib.QL_ERR_ARG, (segs, msg)


def test_plan_rejects_unsupported_block():
    st, msg = _plan_status(_desc(K=512, hadamard_block=256))
    assert st == _lib.QL_ERR_UNSUPPORTED and "256" in msg


def test_plan_rejects_null_pointers():
    st, _ = _plan_status(None)
    assert st == _lib.QL_ERR_ARG
    st, msg = _plan_status(_desc(), W=0)
    assert st == _lib.QL_ERR_ARG and "NULL" in msg
    st, msg = _plan_status(_desc(), W=0x1004)
    assert st == _lib.QL_ERR_ARG and "aligned" in msg


def test_calls_reject_null_plan():
    L = _lib.load()
    assert L.qlinear_quantize_act(None, 0x1000, 4, 0, None, 0x1000, 0x1000, None) == _lib.QL_ERR_ARG
    assert L.qlinear_gemm(None, 0x1000, 0x1000, 4, 0, 1.0, 0x1000, None, None) == _lib.QL_ERR_ARG
    assert L.qlinear_plan_weights(None, None, None, None) == _lib.QL_ERR_ARG
    h = ctypes.c_void_p()
    assert L.qlinear_plan_lsb_view(None, 1, None, ctypes.byref(h)) == _lib.QL_ERR_ARG
    assert L.qlinear_plan_lsb_update(None, None, 1, None) == _lib.QL_ERR_ARG
    assert L.qlinear_plan_destroy(None) == _lib.QL_OK


def test_cfg_combine_host_checks():
    L = _lib.load()
    assert L.qlinear_cfg_combine(0x1000, 3, 4, 4.0, 0x9000, None) == _lib.QL_ERR_ARG
    assert "even" in L.qlinear_last_error().decode()
    assert L.qlinear_cfg_combine(0x1000, 4, 0, 4.0, 0x9000, None) == _lib.QL_ERR_ARG
    assert L.qlinear_cfg_combine(None, 4, 4, 4.0, 0x9000, None) == _lib.QL_ERR_ARG
    assert L.qlinear_cfg_combine(None, 0, 4, 4.0, None, None) == _lib.QL_OK
    # out overlapping Y
    assert L.qlinear_cfg_combine(0x1000, 4, 4, 4.0, 0x1010, None) == _lib.QL_ERR_ARG
    assert "overlaps" in L.qlinear_last_error().decode()
    # empty input is a no-op and never reaches a launch
    assert L.qlinear_cfg_combine(0x1000, 0, 4, 4.0, 0x9000, None) == _lib.QL_OK


def test_probe_host_checks():
    # the MFMA ceiling probe validates its arguments before any device call
    L = _lib.load()
    n = 1 << 20
    assert L.qlinear_probe_mfma(None, 10, 1, 0x1000, n, None) == _lib.QL_ERR_ARG
    assert L.qlinear_probe_mfma(0x1000, 10, 1, None, n, None) == _lib.QL_ERR_ARG
    assert L.qlinear_probe_mfma(0x1000, -1, 1, 0x1000, n, None) == _lib.QL_ERR_ARG
    assert "iters" in L.qlinear_last_error().decode()
    assert L.qlinear_probe_mfma(0x1000, 10, 3, 0x1000, n, None) == _lib.QL_ERR_ARG
    assert "waves_per_simd" in L.qlinear_last_error().decode()
    assert L.qlinear_probe_mfma(0x1008, 10, 1, 0x1000, n, None) == _lib.QL_ERR_ARG
    assert "aligned" in L.qlinear_last_error().decode()


def test_plan_rejects_bad_input_branches():
    def st(offs, **kw):
        arr = (ctypes.c_int32 * len(offs))(*offs)
        d = _desc(K=512, n_k_segments=len(offs) - 1,
                  k_seg_offsets=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), **kw)
        return _plan_status(d)
    assert st([0, 256, 512], hadamard_block=128, a_scale_mode=1, single_hadamard=1)[0] == \
        _lib.QL_ERR_UNSUPPORTED
    assert st([0, 200, 512])[0] == _lib.QL_ERR_UNSUPPORTED          # not a multiple of 128
    assert st([0, 128, 256, 384, 448, 512])[0] == _lib.QL_ERR_UNSUPPORTED  # 5 branches
    assert st([0, 256, 256, 512])[0] == _lib.QL_ERR_ARG             # empty branch
    assert st([0, 256, 500])[0] == _lib.QL_ERR_ARG                  # does not end at K
    assert st([128, 256, 512])[0] == _lib.QL_ERR_ARG                # does not start at 0
    d = _desc(K=512, n_k_segments=2, k_seg_offsets=None)
    assert _plan_status(d)[0] == _lib.QL_ERR_ARG
    assert _plan_status(_desc(n_k_segments=-1))[0] == _lib.QL_ERR_ARG


def test_bench_refuses_more_than_one_gpu():
    import json as _json
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in _json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_header_compiles_and_links_as_c(tmp_path):
    # A plain C99 client of include/qlinear.h, linked against libqlinear.so,
    # exercising a host-side argument error (no GPU needed).
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = tmp_path / "client.c"
    src.write_text(r"""
#include <stdio.h>
#include <string.h>
#include "qlinear.h"
int main(void) {
  ql_desc d;
  memset(&d, 0, sizeof d);
  d.N = 64; d.K = 40; d.w_bits = 8; d.a_bits = 8; d.n_segments = 1;
  qlinear_plan_t p = 0;
  ql_status st = qlinear_plan(&d, (const float*)0x1000, NULL, &p);
  printf("%d %s\n", (int)st, qlinear_last_error());
  return st == QL_ERR_ARG && p == 0 ? 0 : 1;
}
""")
    exe = tmp_path / "client"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
                    str(src), f"-L{libdir}", "-lqlinear", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "multiple of 16" in r.stdout
