"""The no-allocation variant of the activation quantizer
(qlinear_quantize_act_noalloc, partial maxima in the library's static
scratch) against qlinear_quantize_act (partial maxima in the plan's
workspace), through the C ABI: codes and scales must be identical, on two
calls in a row with the second on a smaller input, so that the second call
runs over the scratch contents the first one left."""
from __future__ import annotations

import numpy as np
import pytest

from tests.parity import say
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a ROCm device"
    import bit_post_quantization_amd  # noqa: F401  (fails loudly if the library is missing)
    return _t


CASES = [
    # (K, w_bits, a_bits, B, a_scale, x_dtype, k_seg, lsb_k, M1, M2)
    (1152, 8, 8, 0, "dual", "f32", None, 0, 4096, 200),
    (4608, 8, 8, 0, "dual", "f32", None, 2, 4096, 1000),
    (1152, 4, 4, 128, "dual", "f32", None, 0, 4096, 64),
    (3072, 4, 8, 0, "symmetric", "bf16", None, 0, 2048, 18),
    (1408, 8, 8, 0, "dual", "f32", (0, 256, 1408), 0, 4096, 130),
    (2304, 8, 4, 0, "dual", "f32", (0, 1152, 2304), 1, 512, 2),
]


@pytest.mark.parametrize("case", CASES)
def test_noalloc_quantize_matches_plan_workspace(torch, case):
    from bit_post_quantization_amd import (QuantLinear, qlinear_quantize_act,
                                           qlinear_quantize_act_noalloc)
    K, wb, ab, B, a_scale, x_dtype, kseg, lsb_k, M1, M2 = case
    say(f"[noalloc] K={K} w{wb}a{ab} B={B} {a_scale} {x_dtype} kseg={kseg} k={lsb_k} "
        f"M={M1} then {M2}")
    N = 64
    W = torch.from_numpy(synth.weight_normal(7, f"noalloc/W/{K}", N, K)).cuda()
    ql = QuantLinear(W, w_bits=wb, a_bits=ab, hadamard_block=B, a_scale=a_scale,
                     x_dtype=x_dtype, k_seg_offsets=None if kseg is None else list(kseg))
    nks = 1 if kseg is None else len(kseg) - 1
    for call, M in enumerate((M1, M2)):
        X = synth.gelu_with_outliers(11 + call, f"noalloc/X/{K}/{M}", M, K)
        if x_dtype == "bf16":
            Xd = torch.from_numpy(synth.f32_to_bf16_bits(X).view(np.int16)).cuda()
        else:
            Xd = torch.from_numpy(X).cuda()
        ref_c = ql.alloc_codes(M)
        ref_s = torch.empty(2 * nks, dtype=torch.float32, device="cuda")
        got_c = ql.alloc_codes(M).fill_(0x55)
        got_s = torch.full((2 * nks,), -1.0, dtype=torch.float32, device="cuda")
        qlinear_quantize_act(ql.plan, Xd, M, lsb_k, None, ref_c, ref_s)
        qlinear_quantize_act_noalloc(ql.plan, Xd, M, lsb_k, None, got_c, got_s)
        torch.cuda.synchronize()
        assert torch.equal(got_s.view(torch.int32), ref_s.view(torch.int32)), (call, got_s, ref_s)
        assert torch.equal(got_c, ref_c), f"codes differ on call {call} (M={M})"
        # static scales take no scratch; the variant accepts them the same way
        qlinear_quantize_act_noalloc(ql.plan, Xd, M, lsb_k, ref_s, got_c, got_s)
        torch.cuda.synchronize()
        assert torch.equal(got_c, ref_c) and torch.equal(got_s, ref_s)
        say(f"  call {call}: M={M} codes and scales identical ({ref_s.cpu().numpy()})")


def test_noalloc_rejects_bad_arguments(torch):
    from bit_post_quantization_amd import QLError, QuantLinear, qlinear_quantize_act_noalloc
    ql = QuantLinear(torch.zeros((32, 128), dtype=torch.float32, device="cuda"))
    X = torch.zeros((4, 128), dtype=torch.float32, device="cuda")
    c = ql.alloc_codes(4)
    s = torch.empty(2, dtype=torch.float32, device="cuda")
    with pytest.raises(QLError):
        qlinear_quantize_act_noalloc(ql.plan, X, 4, 8, None, c, s)   # lsb_k out of range
    with pytest.raises(QLError):
        qlinear_quantize_act_noalloc(ql.plan, X, 4, 0, None, None, s)  # NULL codes
    qlinear_quantize_act_noalloc(ql.plan, X, 0, 0, None, None, None)  # empty: no-op
