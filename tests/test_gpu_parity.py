"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs. Sizes span several tiles plus ragged tails; the
full-size workloads are checked on sampled rows (codes in full)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.parity import (assert_close, assert_codes, compare_codes, compare_codes_scaled,
                          gemm_dual_rows, gemm_int64_rows, say, unpack_codes)
from workloads import configs, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a ROCm device"
    import bit_post_quantization_amd  # noqa: F401  (fails loudly if the library is missing)
    return _t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def sample_rows(M: int, cfg: bool, n: int = 48, seed: int = 0) -> np.ndarray:
    """Seeded sample of rows (conditional rows when cfg), plus tile edges."""
    top = M // 2 if cfg else M
    edges = [0, 1, 15, 16, 63, 64, 127, 128, top - 1]
    rnd = synth.random_int_codes(seed, f"rows/{M}/{cfg}", (n,), 0, 127).astype(np.int64)
    rnd = (rnd * 7919 + np.arange(n) * 104729) % top
    return np.unique(np.concatenate([np.array([e for e in edges if 0 <= e < top]), rnd]))


def check_weights(torch, ql, wp):
    wc_g, sw_g = ql.weights()
    torch.cuda.synchronize()
    wc_g, sw_g = wc_g.cpu().numpy(), sw_g.cpu().numpy()
    assert np.array_equal(sw_g.view(np.uint32), wp.scales.view(np.uint32)), "weight scales"
    assert np.array_equal(wc_g, wp.codes), "weight codes"


def check_layer(torch, X, W, *, M, K, N, w_bits=8, a_bits=8, B=0, seg=None, w_scale="channel",
                a_scale="dual", x_dtype="f32", cfg=0, guidance=4.0, lsb_k=0,
                static_scales=None, rows=None, w_lsb_k=0, tag=""):
    """Run one quantized linear on the GPU and check every stage against the oracle.
    rows=None checks every output row. w_lsb_k > 0 runs the layer through a
    weight LSB view of its plan (the base plan is destroyed first)."""
    from bit_post_quantization_amd import QuantLinear
    say(f"[case] {tag} M={M} K={K} N={N} w{w_bits}a{a_bits} B={B} seg={seg} {w_scale} "
        f"{a_scale} {x_dtype} cfg={cfg} k={lsb_k} wk={w_lsb_k} "
        f"static={static_scales is not None}")
    # --- plan / weights ---
    Wd = _dev(torch, W)
    ql = QuantLinear(Wd, w_bits=w_bits, a_bits=a_bits, hadamard_block=B, seg_offsets=seg,
                     w_scale=w_scale, a_scale=a_scale, x_dtype=x_dtype)
    wp = oracle.WeightPlan(W, w_bits, B=B, mode=w_scale, seg_offsets=seg)
    check_weights(torch, ql, wp)
    if w_lsb_k:
        view = ql.lsb_view(w_lsb_k)
        ql.plan.destroy()
        ql = view
        wp = wp.truncated(w_lsb_k)
        check_weights(torch, ql, wp)
    # --- activations ---
    Xd = _dev(torch, X) if x_dtype == "f32" else _dev(torch, X.view(np.int16))
    ss = None if static_scales is None else _dev(torch, np.asarray(static_scales, np.float32))
    codes_d, s_d = ql.quantize(Xd, lsb_k=lsb_k, static_scales=ss)
    torch.cuda.synchronize()
    s_g = s_d.cpu().numpy()
    codes_g = unpack_codes(codes_d.cpu().numpy(), K, a_bits)
    x32 = oracle.bf16_to_f32(X) if x_dtype == "bf16" else X
    x_rot = oracle.rotate(x32, B) if B else x32
    s_o = (oracle.act_scales(x_rot, a_bits, a_scale) if static_scales is None
           else np.asarray(static_scales, np.float32))
    assert np.array_equal(s_g.view(np.uint32), s_o.view(np.uint32)), f"act scales {s_g} vs {s_o}"
    codes_o = oracle.quantize_act(x_rot, s_o, a_bits, lsb_k)
    st = compare_codes(codes_g, codes_o, x_rot, s_o)
    say(f"  codes: {st}")
    assert_codes(st)
    # --- GEMM with accumulator dump ---
    Mo = M // 2 if cfg else M
    Yd = torch.empty((Mo, N), dtype=torch.float32, device="cuda")
    dbg = torch.empty((2, M, N), dtype=torch.int32, device="cuda")
    ql.gemm(codes_d, s_d, cfg=cfg, w=guidance, Y=Yd, acc_dbg=dbg)
    Yd2 = torch.empty_like(Yd)
    ql.gemm(codes_d, s_d, cfg=cfg, w=guidance, Y=Yd2)  # launch configuration without the dump
    torch.cuda.synchronize()
    assert torch.equal(Yd.view(torch.int32), Yd2.view(torch.int32)), "Y differs without acc dump"
    out_rows = np.arange(Mo) if rows is None else np.asarray(rows)
    acc_rows = np.concatenate([out_rows, out_rows + M // 2]) if cfg else out_rows
    idx = torch.from_numpy(acc_rows).cuda()
    accp_g = dbg[0].index_select(0, idx).cpu().numpy()
    accn_g = dbg[1].index_select(0, idx).cpu().numpy()
    Y_g = Yd.index_select(0, torch.from_numpy(out_rows).cuda()).cpu().numpy()
    accp_o, accn_o = gemm_dual_rows(codes_g, wp.codes, acc_rows)
    if a_scale == "symmetric":
        assert np.array_equal(accp_g.astype(np.int64), accp_o.astype(np.int64) + accn_o), "acc (sym)"
        assert not accn_g.any()
    else:
        assert np.array_equal(accp_g, accp_o), "acc+"
        assert np.array_equal(accn_g, accn_o), "acc-"
    y_o = oracle.epilogue(accp_o, accn_o, s_g, wp.scales, B, a_scale)
    if cfg:
        h = out_rows.size
        ref = oracle.cfg_combine(y_o[:h], y_o[h:], guidance)
    else:
        ref = y_o
    e = assert_close(Y_g, ref, "Y")
    exact = np.array_equal(Y_g.view(np.uint32), ref.view(np.uint32))
    say(f"  acc exact; Y max rel err {e:.3g}; bit-exact={exact}")
    del dbg
    return dict(codes=st, y_rel=e, y_exact=exact)


def check_single(torch, X, W, *, M, K, N, B, w_bits=8, a_bits=8, cfg=0, guidance=4.0,
                 w_scale="channel", seg=None, x_dtype="f32", rows=None, w_lsb_k=0, tag=""):
    """HQ-DM single Hadamard (X rotated, W not) on the GPU against the oracle:
    unrotated weight codes and scales, activation codes, the exact int64
    contraction with H W_int^T (from the GPU's hi/lo plane sums) and Y."""
    from bit_post_quantization_amd import QuantLinear
    say(f"[single] {tag} M={M} K={K} N={N} B={B} w{w_bits}a{a_bits} cfg={cfg} wk={w_lsb_k}")
    ql = QuantLinear(_dev(torch, W), w_bits=w_bits, a_bits=a_bits, hadamard_block=B,
                     seg_offsets=seg, w_scale=w_scale, a_scale="symmetric", x_dtype=x_dtype,
                     single_hadamard=True)
    wp = oracle.SingleHadamardPlan(W, w_bits, B, mode=w_scale, seg_offsets=seg)
    check_weights(torch, ql, wp)
    if w_lsb_k:
        view = ql.lsb_view(w_lsb_k)
        ql.plan.destroy()
        ql, wp = view, wp.truncated(w_lsb_k)
        check_weights(torch, ql, wp)
    Xd = _dev(torch, X) if x_dtype == "f32" else _dev(torch, X.view(np.int16))
    codes_d, s_d = ql.quantize(Xd)
    torch.cuda.synchronize()
    codes_g = unpack_codes(codes_d.cpu().numpy(), K, a_bits)
    s_g = s_d.cpu().numpy()
    x32 = oracle.bf16_to_f32(X) if x_dtype == "bf16" else X
    x_rot = oracle.rotate(x32, B)
    s_o = oracle.act_scales(x_rot, a_bits, "symmetric")
    assert np.array_equal(s_g.view(np.uint32), s_o.view(np.uint32)), "act scales"
    st = compare_codes(codes_g, oracle.quantize_act(x_rot, s_o, a_bits), x_rot, s_o)
    assert_codes(st)
    Mo = M // 2 if cfg else M
    Yd = torch.empty((Mo, N), dtype=torch.float32, device="cuda")
    dbg = torch.empty((2, M, N), dtype=torch.int32, device="cuda")
    ql.gemm(codes_d, s_d, cfg=cfg, w=guidance, Y=Yd, acc_dbg=dbg)
    Yd2 = torch.empty_like(Yd)
    ql.gemm(codes_d, s_d, cfg=cfg, w=guidance, Y=Yd2)
    torch.cuda.synchronize()
    assert torch.equal(Yd.view(torch.int32), Yd2.view(torch.int32)), "Y differs without acc dump"
    out_rows = np.arange(Mo) if rows is None else np.asarray(rows)
    acc_rows = np.concatenate([out_rows, out_rows + M // 2]) if cfg else out_rows
    idx = torch.from_numpy(acc_rows).cuda()
    hi = dbg[0].index_select(0, idx).cpu().numpy().astype(np.int64)
    lo = dbg[1].index_select(0, idx).cpu().numpy().astype(np.int64)
    acc_o = gemm_int64_rows(codes_g, wp.v, acc_rows)
    assert np.array_equal(128 * hi + lo, acc_o), "exact accumulators"
    y_o = oracle.epilogue_single(acc_o, s_g[0], wp.scales, B)
    if cfg:
        h = out_rows.size
        ref = oracle.cfg_combine(y_o[:h], y_o[h:], guidance)
    else:
        ref = y_o
    Y_g = Yd.index_select(0, torch.from_numpy(out_rows).cuda()).cpu().numpy()
    e = assert_close(Y_g, ref, "Y")
    exact = np.array_equal(Y_g.view(np.uint32), ref.view(np.uint32))
    say(f"  codes {st}; acc exact; Y max rel err {e:.3g}; bit-exact={exact}; "
        f"max |acc| {np.abs(acc_o).max()}")
    return dict(y_exact=exact, acc_max=int(np.abs(acc_o).max()))


def check_kseg(torch, X, W, *, M, K, N, offs, w_bits=8, a_bits=8, B=0, a_scale="dual",
               x_dtype="f32", cfg=0, guidance=4.0, lsb_k=0, static_scales=None, w_lsb_k=0,
               rows=None, w_scale="channel", seg=None, tag=""):
    """SegLinear input branches on the GPU against the oracle: per-branch
    weight codes and scales, per-branch activation scales and codes, every
    branch's accumulators, and Y."""
    from bit_post_quantization_amd import QuantLinear
    S = len(offs) - 1
    say(f"[kseg] {tag} M={M} K={K} N={N} offs={offs} w{w_bits}a{a_bits} B={B} {a_scale} "
        f"{x_dtype} cfg={cfg} k={lsb_k} wk={w_lsb_k} static={static_scales is not None}")
    ql = QuantLinear(_dev(torch, W), w_bits=w_bits, a_bits=a_bits, hadamard_block=B,
                     a_scale=a_scale, x_dtype=x_dtype, k_seg_offsets=offs, w_scale=w_scale,
                     seg_offsets=seg)
    wp = oracle.InputSegmentedPlan(W, w_bits, offs, B=B, mode=w_scale, seg_offsets=seg)
    check_weights(torch, ql, wp)
    if w_lsb_k:
        view = ql.lsb_view(w_lsb_k)
        ql.plan.destroy()
        ql, wp = view, wp.truncated(w_lsb_k)
        check_weights(torch, ql, wp)
    Xd = _dev(torch, X) if x_dtype == "f32" else _dev(torch, X.view(np.int16))
    ss = None if static_scales is None else _dev(torch, np.asarray(static_scales, np.float32).reshape(-1))
    codes_d, s_d = ql.quantize(Xd, lsb_k=lsb_k, static_scales=ss)
    torch.cuda.synchronize()
    codes_g = unpack_codes(codes_d.cpu().numpy(), K, a_bits)
    s_g = s_d.cpu().numpy().reshape(S, 2)
    codes_o, s_o = oracle.quantize_activations_segmented(
        X, a_bits, offs, B=B, mode=a_scale, lsb_k=lsb_k, static_scales=static_scales,
        bf16=x_dtype == "bf16")
    assert np.array_equal(s_g.view(np.uint32), s_o.view(np.uint32)), f"act scales {s_g} vs {s_o}"
    x32 = oracle.bf16_to_f32(X) if x_dtype == "bf16" else X
    x_rot = np.concatenate([oracle.rotate(x32[:, a:b], B) if B else x32[:, a:b]
                            for a, b in zip(offs[:-1], offs[1:])], axis=1)
    s_el = np.concatenate([np.tile(s_o[j], (M, (b - a), 1)) for j, (a, b) in
                           enumerate(zip(offs[:-1], offs[1:]))], axis=1)
    st = compare_codes_scaled(codes_g, codes_o, x_rot, s_el)
    assert_codes(st)
    Mo = M // 2 if cfg else M
    Yd = torch.empty((Mo, N), dtype=torch.float32, device="cuda")
    dbg = torch.empty((2 * S, M, N), dtype=torch.int32, device="cuda")
    ql.gemm(codes_d, s_d, cfg=cfg, w=guidance, Y=Yd, acc_dbg=dbg)
    Yd2 = torch.empty_like(Yd)
    ql.gemm(codes_d, s_d, cfg=cfg, w=guidance, Y=Yd2)
    torch.cuda.synchronize()
    assert torch.equal(Yd.view(torch.int32), Yd2.view(torch.int32)), "Y differs without acc dump"
    out_rows = np.arange(Mo) if rows is None else np.asarray(rows)
    acc_rows = np.concatenate([out_rows, out_rows + M // 2]) if cfg else out_rows
    idx = torch.from_numpy(acc_rows).cuda()
    y_o, accs = oracle.linear_segmented_rows(codes_g, s_g, wp, acc_rows, a_scale)
    for j, (ap_o, an_o) in enumerate(accs):
        ap_g = dbg[2 * j].index_select(0, idx).cpu().numpy()
        an_g = dbg[2 * j + 1].index_select(0, idx).cpu().numpy()
        if a_scale == "symmetric":
            assert np.array_equal(ap_g.astype(np.int64), ap_o.astype(np.int64) + an_o), f"acc {j}"
        else:
            assert np.array_equal(ap_g, ap_o) and np.array_equal(an_g, an_o), f"acc {j}"
    if cfg:
        h = out_rows.size
        ref = oracle.cfg_combine(y_o[:h], y_o[h:], guidance)
    else:
        ref = y_o
    Y_g = Yd.index_select(0, torch.from_numpy(out_rows).cuda()).cpu().numpy()
    e = assert_close(Y_g, ref, "Y")
    say(f"  codes {st}; acc exact; Y max rel err {e:.3g}; "
        f"bit-exact={np.array_equal(Y_g.view(np.uint32), ref.view(np.uint32))}")


# ---------------------------------------------------------------- small ----

def test_config1_full(torch):
    wl = configs.WORKLOADS["c1"]
    L = wl.layers[0]
    X = configs.make_x(wl, L)
    W = configs.make_w(wl, L)
    r = check_layer(torch, X, W, M=wl.M, K=L.K, N=L.N, tag="c1")
    assert r["y_exact"]


GRID = [
    # (a_bits, w_bits, B, cfg, a_scale, x_dtype, K)
    (8, 8, 0, 0, "dual", "f32", 1056),
    (8, 8, 0, 1, "dual", "f32", 1056),
    (4, 4, 0, 1, "dual", "f32", 1056),
    (4, 4, 32, 1, "dual", "f32", 1056),
    (8, 4, 0, 0, "dual", "bf16", 1056),
    (4, 8, 0, 0, "dual", "f32", 1056),
    (8, 8, 128, 1, "dual", "f32", 640),
    (4, 4, 128, 0, "symmetric", "f32", 640),
    (8, 8, 0, 1, "symmetric", "bf16", 1056),
    (8, 8, 64, 0, "dual", "bf16", 1088),
]


@pytest.mark.parametrize("a_bits,w_bits,B,cfg,a_scale,x_dtype,K", GRID)
def test_grid_full_rows(torch, a_bits, w_bits, B, cfg, a_scale, x_dtype, K):
    M, N = 302, 200
    name = f"grid/{a_bits}{w_bits}{B}{cfg}{a_scale}{x_dtype}{K}"
    X = synth.gelu_with_outliers(1, name + "/X", M, K)
    if x_dtype == "bf16":
        X = synth.f32_to_bf16_bits(X)
    W = synth.weight_normal(1, name + "/W", N, K)
    check_layer(torch, X, W, M=M, K=K, N=N, w_bits=w_bits, a_bits=a_bits, B=B, cfg=cfg,
                a_scale=a_scale, x_dtype=x_dtype, tag=name)


@pytest.mark.parametrize("lsb_k,a_bits", [(2, 8), (4, 8), (7, 8), (1, 4), (3, 4)])
def test_lsb_truncation(torch, lsb_k, a_bits):
    M, K, N = 130, 512, 96
    X = synth.silu_normal(2, f"lsb/{lsb_k}{a_bits}", M, K)
    W = synth.weight_normal(2, f"lsb/W{lsb_k}{a_bits}", N, K)
    check_layer(torch, X, W, M=M, K=K, N=N, a_bits=a_bits, w_bits=a_bits, cfg=1, lsb_k=lsb_k,
                tag=f"lsb{lsb_k}")


@pytest.mark.parametrize("w_bits,a_bits,wk,B,a_scale,seg", [
    (8, 8, 1, 0, "dual", None), (8, 8, 4, 0, "dual", None), (8, 8, 7, 0, "dual", None),
    (8, 4, 3, 128, "dual", None), (4, 4, 1, 128, "dual", None), (4, 4, 3, 0, "symmetric", None),
    (4, 8, 2, 0, "dual", [0, 10, 11, 96])])
def test_weight_lsb_view(torch, w_bits, a_bits, wk, B, a_scale, seg):
    M, K, N = 130, 512, 96
    X = synth.gelu_normal(21, f"wlsb/{w_bits}{a_bits}{wk}{B}", M, K)
    W = synth.weight_normal(21, f"wlsb/W{w_bits}{a_bits}{wk}{B}", N, K)
    check_layer(torch, X, W, M=M, K=K, N=N, w_bits=w_bits, a_bits=a_bits, B=B, a_scale=a_scale,
                seg=seg, w_scale="segment" if seg else "channel", cfg=1, w_lsb_k=wk,
                tag=f"wlsb{wk}")


@pytest.mark.parametrize("M,K,N,B,w_bits,a_bits,cfg", [
    (130, 512, 96, 128, 8, 8, 1), (200, 256, 100, 16, 8, 8, 0), (64, 1024, 33, 128, 4, 4, 1),
    (97, 128, 80, 4, 8, 4, 0), (2, 64, 1, 32, 4, 8, 1)])
def test_single_hadamard(torch, M, K, N, B, w_bits, a_bits, cfg):
    X = synth.gelu_with_outliers(23, f"single/{M}{K}{N}{B}", M, K)
    W = synth.weight_normal(23, f"single/W{M}{K}{N}{B}", N, K)
    check_single(torch, X, W, M=M, K=K, N=N, B=B, w_bits=w_bits, a_bits=a_bits, cfg=cfg,
                 tag="single")


@pytest.mark.parametrize("M,K,N,a_bits,cfg", [(4096, 256, 1152, 8, 1), (4096, 512, 1530, 4, 0)])
def test_single_hadamard_wide_tiles(torch, M, K, N, a_bits, cfg):
    # Shapes whose tile count makes the launcher pick 192-row (96-channel)
    # tiles; the 8-bit case fills the whole 160 KB of LDS.
    X = synth.gelu_with_outliers(30, f"single/wide/{M}{K}{N}", M, K)
    W = synth.weight_normal(30, f"single/wide/W{M}{K}{N}", N, K)
    rows = sample_rows(M, bool(cfg), 32, seed=7)
    check_single(torch, X, W, M=M, K=K, N=N, B=128, w_bits=8, a_bits=a_bits, cfg=cfg, rows=rows,
                 tag="wide")


@pytest.mark.parametrize("M,K,N,a_bits,cfg", [(4096, 256, 4608, 8, 1), (4096, 512, 1530, 4, 0)])
def test_symmetric_wide_tiles(torch, M, K, N, a_bits, cfg):
    # Symmetric activations at shapes whose tile count makes the launcher
    # pick 192-column tiles.
    X = synth.gelu_with_outliers(31, f"sym/wide/{M}{K}{N}", M, K)
    W = synth.weight_normal(31, f"sym/wide/W{M}{K}{N}", N, K)
    rows = sample_rows(M, bool(cfg), 32, seed=8)
    check_layer(torch, X, W, M=M, K=K, N=N, a_bits=a_bits, w_bits=8, B=128, a_scale="symmetric",
                cfg=cfg, rows=rows, tag="sym-wide")


def test_single_hadamard_extremes(torch):
    # A bent sign pattern b of 64 entries (the inner product of the two 3-bit
    # halves of the index) has a flat transform: |H b| = 8 everywhere. Rows
    # built from +-b per block give activation and weight codes of +-127 and
    # |H W_int^T| = 1016 throughout, so at the largest K the exact sums reach
    # 127 * 1016 * 65536 > 2^31: only the hi/lo split keeps them exact.
    M, K, N, B = 8, 65536, 16, 64
    i = np.arange(B)
    b = np.where(np.array([bin((j & 7) & (j >> 3)).count("1") & 1 for j in i]) == 1, -1.0, 1.0)
    rng = np.random.default_rng(24)
    sx = np.where(rng.random((M, K // B)) < 0.5, -1.0, 1.0)
    sw = np.where(rng.random((N, K // B)) < 0.5, -1.0, 1.0)
    sx[0] = sw[0]  # row 0 against channel 0: every block adds +127 * 1016 * 64
    X = (np.repeat(sx, B, axis=1) * np.tile(b, K // B)).astype(np.float32)
    W = (np.repeat(sw, B, axis=1) * np.tile(b, K // B) * 0.01).astype(np.float32)
    r = check_single(torch, X, W, M=M, K=K, N=N, B=B, tag="extremes")
    assert r["acc_max"] == 127 * 1016 * K > 2 ** 31


def test_single_hadamard_weight_view(torch):
    M, K, N, B = 96, 1152, 144, 128
    X = synth.silu_normal(25, "single/view/X", M, K)
    W = synth.weight_normal(25, "single/view/W", N, K)
    check_single(torch, X, W, M=M, K=K, N=N, B=B, cfg=1, w_lsb_k=3, tag="view")


def test_single_hadamard_rejects_dual_scales(torch):
    from bit_post_quantization_amd import QLError, QuantLinear
    W = _dev(torch, synth.weight_normal(26, "single/rej", 32, 128))
    with pytest.raises(QLError):
        QuantLinear(W, hadamard_block=128, a_scale="dual", single_hadamard=True)
    with pytest.raises(QLError):
        QuantLinear(W, hadamard_block=0, a_scale="symmetric", single_hadamard=True)


@pytest.mark.parametrize("M,K,N,offs,w_bits,a_bits,B,a_scale,cfg,x_dtype", [
    (130, 512, 96, [0, 256, 512], 8, 8, 0, "dual", 1, "f32"),
    (200, 384, 100, [0, 128, 384], 8, 4, 0, "dual", 0, "f32"),
    (98, 1152, 80, [0, 768, 1152], 4, 4, 128, "dual", 1, "f32"),
    (64, 640, 144, [0, 128, 256, 512, 640], 8, 8, 0, "symmetric", 0, "bf16"),
    (66, 2304, 72, [0, 1152, 2304], 8, 8, 128, "symmetric", 1, "f32"),
    (2, 272, 1, [0, 256, 272], 8, 8, 0, "dual", 1, "f32")])
def test_input_branches(torch, M, K, N, offs, w_bits, a_bits, B, a_scale, cfg, x_dtype):
    # Branches with different distributions: GELU with outliers, then a
    # narrower SiLU, then N(0,1) scaled down (each branch on its own range).
    parts, kinds = [], [synth.gelu_with_outliers, synth.silu_normal, synth.gelu_normal]
    for j, (a, b) in enumerate(zip(offs[:-1], offs[1:])):
        xj = kinds[j % 3](41, f"kseg/{M}{K}{N}/{j}", M, b - a) * np.float32(4.0 ** -j)
        parts.append(xj.astype(np.float32))
    X = np.concatenate(parts, axis=1)
    if x_dtype == "bf16":
        X = synth.f32_to_bf16_bits(X)
    W = synth.weight_normal(41, f"kseg/W{M}{K}{N}", N, K)
    check_kseg(torch, X, W, M=M, K=K, N=N, offs=offs, w_bits=w_bits, a_bits=a_bits, B=B,
               a_scale=a_scale, x_dtype=x_dtype, cfg=cfg, tag="kseg")


@pytest.mark.parametrize("w_scale,seg,a_bits,x_dtype", [
    ("segment", [0, 48, 96, 144], 8, "f32"), ("tensor", None, 4, "bf16")])
def test_input_branches_with_output_segments(torch, w_scale, seg, a_bits, x_dtype):
    # Input branches and output-segment (or per-tensor) weight scales together.
    M, K, N, offs = 100, 640, 144, [0, 384, 640]
    X = np.concatenate([synth.silu_normal(43, "kseg/os/0", M, 384),
                        synth.sinusoid(43, "kseg/os/1", M, 256)], axis=1)
    if x_dtype == "bf16":
        X = synth.f32_to_bf16_bits(X)
    W = synth.weight_normal(43, "kseg/os/W", N, K)
    check_kseg(torch, X, W, M=M, K=K, N=N, offs=offs, w_bits=4, a_bits=a_bits, cfg=1,
               x_dtype=x_dtype, w_scale=w_scale, seg=seg, tag=f"kseg+{w_scale}")


@pytest.mark.parametrize("M,K,N,wk", [
    (130, 528, 288, 1), (130, 528, 288, 4), (130, 528, 288, 7), (20480, 256, 288, 3)])
def test_weight_lsb_view_wide_tiles(torch, M, K, N, wk):
    # int8 W8A8 DualScale with CFG and 144-column tiles: the 8-wave GEMM masks
    # the view's depth in LDS. Ragged rows and K; the large case streams one
    # or two tiles per workgroup.
    X = synth.gelu_normal(23, f"wlsbw/{M}/{K}/{wk}", M, K)
    W = synth.weight_normal(23, f"wlsbw/W{M}/{K}/{wk}", N, K)
    rows = None if M <= 1024 else sample_rows(M, True, 48, seed=wk)
    check_layer(torch, X, W, M=M, K=K, N=N, cfg=1, w_lsb_k=wk, rows=rows, tag=f"wlsbw{wk}")


def test_input_branches_static_lsb_view(torch):
    M, K, N, offs = 96, 768, 64, [0, 512, 768]
    X = np.concatenate([synth.silu_normal(42, "kseg/st/0", M, 512),
                        synth.gelu_normal(42, "kseg/st/1", M, 256) * np.float32(0.01)], axis=1)
    W = synth.weight_normal(42, "kseg/st/W", N, K)
    check_kseg(torch, X, W, M=M, K=K, N=N, offs=offs, cfg=1, lsb_k=2, w_lsb_k=3,
               static_scales=[[0.02, 0.003], [0.0002, 0.0001]], tag="static+lsb+view")


def test_weight_lsb_update(torch):
    # One view re-targeted between steps without allocation: new depth, then
    # another layer of the same shape; depth 0 reproduces the stored layer.
    from bit_post_quantization_amd import QLError, QuantLinear, qlinear_plan_lsb_update
    M, K, N = 96, 256, 160
    Ws = [synth.weight_normal(22, f"upd/W{i}", N, K) for i in range(2)]
    qls = [QuantLinear(_dev(torch, W)) for W in Ws]
    wps = [oracle.WeightPlan(W, 8) for W in Ws]
    view = qls[0].lsb_view(2)
    check_weights(torch, view, wps[0].truncated(2))
    X = _dev(torch, synth.silu_normal(22, "upd/X", M, K))
    codes, s = qls[0].quantize(X)
    for li, k in [(0, 4), (1, 2), (1, 0), (0, 0)]:
        view.base = qls[li]
        view.update_lsb(k)
        check_weights(torch, view, wps[li].truncated(k))
        Yv = view.gemm(codes, s, cfg=1)
        Yb = qls[li].gemm(codes, s, cfg=1) if k == 0 else None
        torch.cuda.synchronize()
        if k == 0:
            assert torch.equal(Yv.view(torch.int32), Yb.view(torch.int32))
        else:
            ap, an = oracle.gemm_dual(unpack_codes(codes.cpu().numpy(), K, 8),
                                      wps[li].truncated(k).codes)
            y = oracle.epilogue(ap, an, s.cpu().numpy(), wps[li].scales)
            ref = oracle.cfg_combine(y[: M // 2], y[M // 2:], 1.0)
            assert_close(Yv.cpu().numpy(), ref, "Y view")
    other = QuantLinear(_dev(torch, synth.weight_normal(22, "upd/W2", N, K + 32)))
    with pytest.raises(QLError):
        qlinear_plan_lsb_update(view.plan, other.plan, 1)
    with pytest.raises(QLError):
        qlinear_plan_lsb_update(view.plan, view.plan, 1)
    with pytest.raises(QLError):
        qlinear_plan_lsb_update(view.plan, qls[0].plan, 8)
    with pytest.raises(QLError):
        qls[0].lsb_view(-1)
    w4 = QuantLinear(_dev(torch, Ws[0]), w_bits=4)
    with pytest.raises(QLError):
        w4.lsb_view(4)
    with pytest.raises(QLError):
        qlinear_plan_lsb_update(view.plan, w4.plan, 1)  # same shape, other width


@pytest.mark.parametrize("w_scale,seg", [
    ("segment", [0, 64, 128, 192]), ("tensor", None), ("segment", [0, 10, 11, 100, 192]),
    ("segment", list(range(0, 193, 1)))])
def test_segments(torch, w_scale, seg):
    M, K, N = 200, 256, 192
    X = synth.bf16_normal(3, f"seg/{len(seg or [])}", M, K)
    W = synth.weight_normal(3, f"seg/W{len(seg or [])}", N, K)
    check_layer(torch, X, W, M=M, K=K, N=N, w_bits=4, a_bits=8, seg=seg, w_scale=w_scale,
                x_dtype="bf16", tag="seg")


@pytest.mark.parametrize("a_bits", [8, 4])
@pytest.mark.parametrize("mx,mn", [(100.0, 50.0), (3.7, 91.3), (0.0123, 0.777), (1234.5, 0.5)])
def test_codes_at_rounding_boundaries(torch, a_bits, mx, mn):
    """Values whose quotient by the scale lies on, or within a few ulps of, a
    half-integer: the cases where a product with the reciprocal scale could
    round differently from the IEEE quotient, including quotients that the
    float division rounds onto a half-integer (then rounded half to even)
    although the exact quotient is not one. Codes must match exactly."""
    from fractions import Fraction
    from bit_post_quantization_amd import QuantLinear
    qa = 127 if a_bits == 8 else 7
    mx, mn = np.float32(mx), np.float32(mn)
    sp, sn = mx / np.float32(qa), mn / np.float32(qa)
    vals = []
    for k in range(qa + 1):
        for sgn, s in ((1.0, sp), (-1.0, sn)):
            c = np.float32(sgn * (k + 0.5)) * s
            for d in range(-4, 5):
                v = c
                step = np.float32(np.inf) if d > 0 else np.float32(-np.inf)
                for _ in range(abs(d)):
                    v = np.nextafter(v, step)
                vals.append(v)
    vals = np.asarray(vals, np.float32)
    vals = vals[(vals <= mx) & (vals >= -mn)]
    # the set holds double-rounding cases: fl(v / s) on a half-integer, v / s not
    ties = 0
    for v in vals:
        s_ = sp if v >= 0 else sn
        fq = np.float32(v) / s_
        if fq - np.floor(fq) == 0.5 and Fraction(float(v)) / Fraction(float(s_)) != Fraction(float(fq)):
            ties += 1
    assert ties > 0
    K = 256
    M = 2 * ((vals.size + K - 1) // K + 1)
    # filler strictly inside [-mn, mx], so that mx and -mn set the scales
    X = (synth.random_int_codes(3, "bnd/X", (M, K), -40, 40).astype(np.float32)
         * np.float32(min(mx, mn) / 64))
    flat = X.reshape(-1)
    flat[: vals.size] = vals
    flat[-1], flat[-2] = mx, -mn
    W = synth.weight_normal(3, "bnd/W", 64, K)
    ql = QuantLinear(_dev(torch, W), w_bits=8, a_bits=a_bits)
    codes_d, s_d = ql.quantize(_dev(torch, X))
    torch.cuda.synchronize()
    s_g = s_d.cpu().numpy()
    assert np.array_equal(s_g, np.array([sp, sn], np.float32)), s_g
    codes_g = unpack_codes(codes_d.cpu().numpy(), K, a_bits)
    codes_o = oracle.quantize_act(X, s_g, a_bits, 0)
    bad = np.nonzero(codes_g.reshape(-1) != codes_o.reshape(-1))[0]
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}: x={flat[bad[:5]]}"



@pytest.mark.parametrize("a_bits,B,x_dtype,lsb_k,a_scale", [
    (8, 0, "f32", 0, "dual"), (4, 128, "bf16", 1, "dual"), (8, 128, "f32", 2, "symmetric")])
def test_one_pass_quantizer_limits(torch, a_bits, B, x_dtype, lsb_k, a_scale):
    # Dynamic scales run in one pass when X fits in 40 units of 4 values per
    # lane, 512 lanes per CU: the largest such tensor (its last workgroup
    # ragged) and one row more (two passes) must both give the oracle's
    # scales and codes.
    from bit_post_quantization_amd import QuantLinear
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K, N = 4608, 16
    M1 = (40 * cus * 512 * 4) // K
    W = synth.weight_normal(44, "onepass/W", N, K)
    ql = QuantLinear(_dev(torch, W), a_bits=a_bits, hadamard_block=B, x_dtype=x_dtype,
                     a_scale=a_scale)
    for M in (M1, M1 + 1):
        say(f"[case] one-pass limit M={M} K={K} a{a_bits} B={B} {x_dtype} k={lsb_k} {a_scale}")
        X = synth.silu_normal(44, f"onepass/{M}/{a_bits}/{B}", M, K)
        if x_dtype == "bf16":
            X = synth.f32_to_bf16_bits(X)
        Xd = _dev(torch, X) if x_dtype == "f32" else _dev(torch, X.view(np.int16))
        codes_d, s_d = ql.quantize(Xd, lsb_k=lsb_k)
        torch.cuda.synchronize()
        s_g = s_d.cpu().numpy()
        codes_g = unpack_codes(codes_d.cpu().numpy(), K, a_bits)
        del Xd, codes_d
        x32 = oracle.bf16_to_f32(X) if x_dtype == "bf16" else X
        x_rot = oracle.rotate(x32, B) if B else x32
        s_o = oracle.act_scales(x_rot, a_bits, a_scale)
        assert np.array_equal(s_g.view(np.uint32), s_o.view(np.uint32)), f"scales {s_g} vs {s_o}"
        st = compare_codes(codes_g, oracle.quantize_act(x_rot, s_o, a_bits, lsb_k), x_rot, s_o)
        say(f"  codes: {st}")
        assert_codes(st)

@pytest.mark.parametrize("K,offs,a_bits,B,x_dtype,lsb_k,a_scale", [
    (1408, (0, 256, 1408), 8, 0, "f32", 0, "dual"),
    (2304, (0, 1152, 2304), 4, 128, "bf16", 1, "dual"),
    (4608, (0, 3456, 4608), 8, 128, "f32", 2, "symmetric")])
def test_one_pass_quantizer_limits_two_branches(torch, K, offs, a_bits, B, x_dtype, lsb_k,
                                                a_scale):
    # Two input branches (SegQuant explainer 2.A) also run in one pass up to
    # 40 units of 4 values per lane: each lane tracks its units' columns
    # (K / 4 = 352 units per row makes the lane's column step 160, wrapping
    # within rows), and the grid exchanges one maxima pair per branch. The
    # largest such tensor and one row more (two passes) must both give the
    # oracle's per-branch scales, codes, accumulators and outputs.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 16
    M1 = (40 * cus * 512 * 4) // K
    W = synth.weight_normal(45, f"onepass2/W/{K}", N, K)
    for M in (M1, M1 + 1):
        X = synth.silu_normal(45, f"onepass2/{M}/{K}", M, K)
        if x_dtype == "bf16":
            X = synth.f32_to_bf16_bits(X)
        rows = np.arange(0, M, 61)
        check_kseg(torch, X, W, M=M, K=K, N=N, offs=list(offs), a_bits=a_bits, w_bits=8, B=B,
                   a_scale=a_scale, x_dtype=x_dtype, lsb_k=lsb_k, rows=rows,
                   tag=f"one-pass limit M={M}")


def _probe_expected(ops: np.ndarray, iters: int) -> int:
    """Sum, modulo 2^32, of every accumulator of one probe wave: accumulator
    j adds iters products of fragments (j % 8, 8 + (j + j // 8) % 8); a 16 x
    16 x 64 product's entries sum to sum_k colsum(A)[k] * rowsum(B)[k], and
    lane l of a fragment carries row (column) l % 16 and K chunk l // 16."""
    f = ops.astype(np.int64).reshape(16, 4, 16, 16)   # fragment, K chunk, row/col, byte
    sums = f.sum(axis=2)                               # [fragment, chunk, byte]: K-indexed sums
    tot = 0
    for j in range(16):
        a, b = j % 8, 8 + (j + j // 8) % 8
        tot += int((sums[a] * sums[b]).sum())
    return (tot * iters) % (1 << 32)


@pytest.mark.parametrize("kind", ["random", "constant"])
def test_mfma_probe_sums(torch, kind):
    # The measurement aid behind the GEMM's measured ceiling: every wave's
    # accumulators must hold exactly iters times the fragments' products.
    from bit_post_quantization_amd import qlinear_probe_mfma
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if kind == "random":
        ops = np.random.default_rng(7).integers(-128, 128, size=(16, 64, 16), dtype=np.int8)
    else:
        ops = np.full((16, 64, 16), 3, np.int8)
    od = _dev(torch, ops)
    for wps in (1, 2):
        for iters in (0, 1, 5, 1000):
            sink = torch.full((cus * 256 * wps,), -1, dtype=torch.int32, device="cuda")
            qlinear_probe_mfma(od, iters, wps, sink)
            torch.cuda.synchronize()
            per_wave = sink.cpu().numpy().astype(np.int64).reshape(-1, 64).sum(axis=1) % (1 << 32)
            exp = _probe_expected(ops, iters)
            assert (per_wave == exp).all(), (kind, wps, iters, per_wave[:4], exp)
        say(f"[probe] {kind} operands: {cus * 4 * wps} waves, sums exact")
    # a sink one element short of the grid is refused before any launch
    from bit_post_quantization_amd import QLError
    short = torch.zeros(cus * 256 - 1, dtype=torch.int32, device="cuda")
    with pytest.raises(QLError, match="sink holds"):
        qlinear_probe_mfma(od, 1, 1, short)


def test_static_scales(torch):
    M, K, N = 64, 256, 80
    X = synth.silu_normal(4, "static/X", M, K)
    W = synth.weight_normal(4, "static/W", N, K)
    check_layer(torch, X, W, M=M, K=K, N=N, static_scales=[0.01, 0.002], tag="static")
    check_layer(torch, X, W, M=M, K=K, N=N, a_bits=4, w_bits=4, static_scales=[0.5, 0.0],
                tag="static-zero-neg")


@pytest.mark.parametrize("M,K,N,a_bits,w_bits,cfg", [
    (2, 16, 1, 8, 8, 1), (1, 32, 3, 4, 4, 0), (129, 64, 129, 8, 8, 0), (256, 128, 256, 8, 4, 1),
    (4, 1024, 1, 4, 8, 1)])
def test_small_and_ragged_shapes(torch, M, K, N, a_bits, w_bits, cfg):
    X = synth.gelu_normal(5, f"shape/{M}{K}{N}", M, K)
    W = synth.weight_normal(5, f"shape/W{M}{K}{N}", N, K)
    check_layer(torch, X, W, M=M, K=K, N=N, a_bits=a_bits, w_bits=w_bits, cfg=cfg, tag="shape")


def test_degenerate_inputs(torch):
    M, K, N = 64, 128, 64
    W = synth.weight_normal(6, "deg/W", N, K)
    pos = np.abs(synth.silu_normal(6, "deg/pos", M, K)) + np.float32(0.01)
    check_layer(torch, pos, W, M=M, K=K, N=N, tag="all-positive")       # s- = 0
    check_layer(torch, -pos, W, M=M, K=K, N=N, cfg=1, tag="all-negative")  # s+ = 0
    z = np.zeros((M, K), np.float32)
    z[::3, ::5] = -0.0
    r = check_layer(torch, z, W, M=M, K=K, N=N, tag="all-zero")
    assert r["y_exact"]
    Wz = np.zeros((N, K), np.float32)
    check_layer(torch, pos, Wz, M=M, K=K, N=N, tag="zero-weights")


def test_extreme_magnitudes(torch):
    # Subnormal inputs (subnormal scales: the reciprocal overflows and the
    # exact division path takes over), a 1e-30 .. 1e30 dynamic range (most
    # codes 0) and large values whose products stay finite.
    M, K, N = 96, 256, 80
    W = synth.weight_normal(28, "ext/W", N, K)
    z = synth.normal_f64(28, "ext/z", (M, K))
    sub = (z * 1e-40).astype(np.float32)
    assert np.abs(sub).max() < np.finfo(np.float32).tiny
    check_layer(torch, sub, W, M=M, K=K, N=N, cfg=1, tag="subnormal")
    check_layer(torch, sub, W, M=M, K=K, N=N, a_bits=4, w_bits=4, B=64, a_scale="symmetric",
                tag="subnormal-h64-a4")
    wide = (np.sign(z) * 10.0 ** (60.0 * synth.normal_f64(28, "ext/e", (M, K)).clip(-1, 1) / 2)
            ).astype(np.float32)
    check_layer(torch, wide, W, M=M, K=K, N=N, cfg=1, tag="1e-30..1e30")
    big = (z * 1e30).astype(np.float32)
    check_layer(torch, big, W, M=M, K=K, N=N, B=128, tag="1e30")


def test_empty_input_is_noop(torch):
    from bit_post_quantization_amd import QuantLinear
    W = _dev(torch, synth.weight_normal(7, "empty/W", 32, 64))
    ql = QuantLinear(W)
    X = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    codes, s = ql.quantize(X)
    Y = ql.gemm(codes, s, cfg=1)
    torch.cuda.synchronize()
    assert codes.shape == (0, 64) and Y.shape == (0, 32)


def test_repeated_dynamic_calls_reset_workspace(torch):
    # The reduction workspace must come back to zero after every call: a
    # second tensor with a smaller range must get its own scales.
    from bit_post_quantization_amd import QuantLinear
    K, N = 256, 64
    ql = QuantLinear(_dev(torch, synth.weight_normal(8, "rep/W", N, K)))
    for i, mult in enumerate([10.0, 1.0, 0.1, 5.0]):
        X = (synth.gelu_normal(8, f"rep/X{i}", 97, K) * np.float32(mult)).astype(np.float32)
        codes, s = ql.quantize(_dev(torch, X))
        torch.cuda.synchronize()
        assert np.array_equal(s.cpu().numpy(), oracle.act_scales(X, 8)), i


def test_graph_capture_replays(torch):
    # quantize + gemm enqueue no allocation, memset or host synchronisation,
    # so a step can be captured into a HIP graph: every replay (with new data
    # in the captured input, eager work and synchronisation in between) must
    # equal the eager result on the same data.
    from bit_post_quantization_amd import QuantLinear
    M, K, N = 256, 512, 192
    ql = QuantLinear(_dev(torch, synth.weight_normal(27, "graph/W", N, K)))
    X = torch.empty((M, K), dtype=torch.float32, device="cuda")
    codes = ql.alloc_codes(M)
    sc = torch.empty(2, dtype=torch.float32, device="cuda")
    Y = torch.empty((M // 2, N), dtype=torch.float32, device="cuda")

    def step():
        ql.quantize(X, codes=codes, act_scales=sc)
        ql.gemm(codes, sc, cfg=1, w=4.0, Y=Y)

    X.copy_(_dev(torch, synth.silu_normal(27, "graph/X0", M, K)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        X.copy_(_dev(torch, synth.gelu_with_outliers(27, f"graph/X{i + 1}", M, K)
                     * np.float32(10.0 ** (i - 2))))
        g.replay()
        torch.cuda.synchronize()
        y_graph = Y.clone()
        s_graph = sc.clone()
        step()  # eager on the same data
        torch.cuda.synchronize()
        assert torch.equal(s_graph.view(torch.int32), sc.view(torch.int32)), i
        assert torch.equal(y_graph.view(torch.int32), Y.view(torch.int32)), i


def test_plan_lifecycle_releases_memory(torch):
    # Plans and views of every kind (single Hadamard, input branches, weight
    # views destroyed before and after their base) give back all their
    # device memory.
    from bit_post_quantization_amd import QuantLinear
    W = _dev(torch, synth.weight_normal(29, "life/W", 384, 512))

    def cycle():
        a = QuantLinear(W, w_bits=4, a_bits=4, hadamard_block=128, a_scale="symmetric",
                        single_hadamard=True)
        b = QuantLinear(W, k_seg_offsets=[0, 256, 512])
        c = QuantLinear(W)
        va, vb, vc = a.lsb_view(1), b.lsb_view(2), c.lsb_view(3)
        vc.update_lsb(1)
        a.plan.destroy()      # base before its view
        va.plan.destroy()
        vb.plan.destroy()     # view before its base
        b.plan.destroy()
        c.plan.destroy()
        vc.plan.destroy()

    cycle()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(20):
        cycle()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert abs(free1 - free0) < (8 << 20), (free0, free1)


def test_cfg_combine_standalone(torch):
    from bit_post_quantization_amd import qlinear_cfg_combine
    for M, N in [(302, 77), (2, 1), (4096, 1152)]:
        Y = synth.normal_f64(9, f"cfg/{M}{N}", (M, N)).astype(np.float32)
        Yd = _dev(torch, Y)
        out = torch.empty((M // 2, N), dtype=torch.float32, device="cuda")
        qlinear_cfg_combine(Yd, M, N, 4.0, out)
        torch.cuda.synchronize()
        ref = oracle.cfg_combine(Y[: M // 2], Y[M // 2:], 4.0)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_gpu_argument_errors(torch):
    from bit_post_quantization_amd import QLError, QuantLinear, qlinear_gemm, qlinear_quantize_act
    ql = QuantLinear(_dev(torch, synth.weight_normal(10, "err/W", 32, 64)))
    X = torch.zeros((5, 64), dtype=torch.float32, device="cuda")
    codes = torch.empty((5, 64), dtype=torch.int8, device="cuda")
    s = torch.empty(2, dtype=torch.float32, device="cuda")
    with pytest.raises(QLError):
        qlinear_quantize_act(ql.plan, X, 5, 8, None, codes, s)
    with pytest.raises(QLError):
        qlinear_quantize_act(ql.plan, X, -1, 0, None, codes, s)
    Y = torch.empty((5, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(QLError):
        qlinear_gemm(ql.plan, codes, s, 5, 1, 4.0, Y)  # odd M with CFG
    with pytest.raises(QLError):
        qlinear_gemm(ql.plan, codes, s, 4, 2, 4.0, Y)  # bad cfg flag


# ------------------------------------------------------------ full size ----

def _run_workload_layer(torch, key, li, rows_n=48):
    """One layer of a workload at full size; rows_n=None checks every
    output row (the oracle GEMM sharded over threads)."""
    wl = configs.WORKLOADS[key]
    L = wl.layers[li]
    X = configs.make_x(wl, L)
    W = configs.make_w(wl, L)
    rows = None if rows_n is None else sample_rows(wl.M, L.cfg, rows_n, seed=li)
    return check_layer(torch, X, W, M=wl.M, K=L.K, N=L.N, w_bits=L.w_bits, a_bits=L.a_bits,
                       B=L.hadamard_block, seg=None if L.seg_offsets() is None else L.seg_offsets().tolist(),
                       w_scale=L.w_scale, a_scale=L.a_scale, x_dtype=L.x_dtype, cfg=int(L.cfg),
                       guidance=L.guidance, rows=rows, tag=f"{key}/{L.name}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("li", range(4))
def test_config2_dit_w8a8_cfg(torch, li):
    _run_workload_layer(torch, "c2", li, rows_n=None)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("li", range(4))
def test_config3_dit_w4a4_hadamard(torch, li):
    _run_workload_layer(torch, "c3", li, rows_n=None)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("li", range(4))
def test_config3_single_hadamard(torch, li):
    wl = configs.WORKLOADS["c3"]
    L = configs.c3_single()[li]
    X = configs.make_x(wl, L)
    W = configs.make_w(wl, L)
    check_single(torch, X, W, M=wl.M, K=L.K, N=L.N, B=L.hadamard_block, w_bits=L.w_bits,
                 a_bits=L.a_bits, cfg=int(L.cfg), guidance=L.guidance, rows=None,
                 tag=f"c3s/{L.name}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("li", range(2))
def test_config7_input_branches(torch, li):
    wl = configs.WORKLOADS["c7"]
    L = wl.layers[li]
    X = configs.make_x(wl, L)
    W = configs.make_w(wl, L)
    rows = sample_rows(wl.M, True, 48, seed=300 + li)
    check_kseg(torch, X, W, M=wl.M, K=L.K, N=L.N, offs=list(L.k_seg), cfg=1,
               guidance=L.guidance, rows=rows, tag=f"c7/{L.name}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("li", range(4))
def test_config4_mmdit_segments(torch, li):
    _run_workload_layer(torch, "c4", li, rows_n=64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("li", range(4))
def test_config4_gamp_bits(torch, li):
    # The MM-DiT stack with activation bits from the greedy allocation.
    import dataclasses
    from bit_post_quantization_amd import qlinear_gamp_allocate
    wl, macs, gain, budget = configs.c4_gamp_inputs()
    bits, _ = qlinear_gamp_allocate(macs.tolist(), gain.tolist(), 4, budget)
    L = dataclasses.replace(wl.layers[li], a_bits=bits[li])
    X = configs.make_x(wl, L)
    W = configs.make_w(wl, L)
    rows = sample_rows(wl.M, False, 24, seed=100 + li)
    seg = L.seg_offsets()
    check_layer(torch, X, W, M=wl.M, K=L.K, N=L.N, w_bits=L.w_bits, a_bits=L.a_bits,
                seg=None if seg is None else seg.tolist(), w_scale=L.w_scale,
                x_dtype=L.x_dtype, rows=rows, tag=f"c4g/{L.name}/a{L.a_bits}")


@pytest.mark.timeout(900)
def test_config5_tasq_steps(torch):
    # Every layer of one block over several steps of the schedule, plus the
    # first layer of every block at step 0 (the full sweep is a benchmark).
    wl = configs.WORKLOADS["c5"]
    sched = configs.c5_schedule()
    cases = [(t, li) for t in (0, 1, 49) for li in range(4)] + [(0, 4 * b) for b in range(1, 28, 9)]
    for t, li in cases:
        L = wl.layers[li]
        X = configs.make_x(wl, L, step=t)
        W = configs.make_w(wl, L)
        rows = sample_rows(wl.M, True, 16, seed=t * 1000 + li)
        check_layer(torch, X, W, M=wl.M, K=L.K, N=L.N, cfg=1, guidance=L.guidance,
                    lsb_k=int(sched[t, li]), rows=rows, tag=f"c5/t{t}/{L.name}")


@pytest.mark.timeout(900)
def test_config6_tasq_weight_stages(torch):
    # One stored W8 layer per linear run through a view at the stage's depth,
    # activations at per-step static scales calibrated on a separate input
    # (dynamic scales of the calibration batch, from the GPU, checked here).
    from bit_post_quantization_amd import QuantLinear
    wl = configs.WORKLOADS["c6"]
    ws = configs.c6_w_schedule()
    cases = [(0, 0), (0, 2), (15, 1), (30, 3), (49, 2), (49, 4 * 13 + 3)]
    for t, li in cases:
        L = wl.layers[li]
        g = configs.stage_of(wl, t)
        Xc = configs.make_calib_x(wl, L, t)
        qc = QuantLinear(_dev(torch, np.zeros((L.N, L.K), np.float32)))
        _, s_cal = qc.quantize(_dev(torch, Xc))
        torch.cuda.synchronize()
        s_cal = s_cal.cpu().numpy()
        assert np.array_equal(s_cal.view(np.uint32), oracle.act_scales(Xc, 8).view(np.uint32))
        del qc, Xc
        X = configs.make_x(wl, L, step=t)
        W = configs.make_w(wl, L)
        rows = sample_rows(wl.M, True, 16, seed=t * 1000 + li)
        check_layer(torch, X, W, M=wl.M, K=L.K, N=L.N, cfg=1, guidance=L.guidance,
                    static_scales=s_cal, w_lsb_k=int(ws[g, li]), rows=rows,
                    tag=f"c6/t{t}/g{g}/{L.name}")
