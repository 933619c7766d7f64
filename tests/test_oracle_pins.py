"""Pins for the CPU oracle: closed forms, invariants, library special cases,
hand-derived fixtures and brute force. None of these re-types the oracle's
own formulas; each is chosen so that a plausible slip (dropped term, wrong
sign, swapped scale, transposed operand, wrong rounding) fails one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ P1 FWHT --

def test_fwht_golden_block8(orc):
    g = _golden("hadamard8.json")
    out = orc.fwht_block(np.array(g["x"], np.float32))
    assert out.tolist() == g["Hx"]


@pytest.mark.parametrize("B", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_equals_sylvester_matrix_exactly(orc, B):
    # scipy.linalg.hadamard builds the Sylvester-ordered matrix. Integer inputs
    # with |sums| < 2^24 make every fp32 butterfly exact.
    H = scipy.linalg.hadamard(B).astype(np.int64)
    rng = np.random.default_rng(B)
    for _ in range(4):
        x = rng.integers(-1000, 1000, size=B)
        out = orc.fwht_block(x.astype(np.float32))
        assert np.array_equal(out.astype(np.int64), H @ x)


@pytest.mark.parametrize("B", [4, 16, 128])
def test_fwht_involution_and_orthogonality(orc, B):
    H = scipy.linalg.hadamard(B).astype(np.int64)
    assert np.array_equal(H @ H.T, B * np.eye(B, dtype=np.int64))
    x = np.arange(-B // 2, B // 2, dtype=np.float32)
    twice = orc.fwht_block(orc.fwht_block(x))
    assert np.array_equal(twice, B * x)


def test_rotate_rows_is_block_diagonal(orc):
    B, K, rows = 8, 32, 3
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 50, size=(rows, K))
    Hbd = np.kron(np.eye(K // B, dtype=np.int64), scipy.linalg.hadamard(B).astype(np.int64))
    out = orc.rotate(x.astype(np.float32), B)
    assert np.array_equal(out.astype(np.int64), x @ Hbd.T)


def test_rotation_preserves_product(orc):
    # (1/B) (X H)(W H)^T = X W^T: the normalisation folded as 1/B.
    B = 128
    rng = np.random.default_rng(2)
    X = rng.integers(-8, 8, size=(5, 256)).astype(np.float32)
    W = rng.integers(-8, 8, size=(7, 256)).astype(np.float32)
    Xr = orc.rotate(X, B).astype(np.float64)
    Wr = orc.rotate(W, B).astype(np.float64)
    lhs = (Xr @ Wr.T) / B
    rhs = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(lhs, rhs)


def test_rotate_rejects_bad_block(orc):
    with pytest.raises(orc.OracleError):
        orc.rotate(np.zeros((2, 24), np.float32), 16)
    with pytest.raises(orc.OracleError):
        orc.rotate(np.zeros((2, 24), np.float32), 12)


# ------------------------------------------------------- golden end to end --

def test_golden_dualscale_cfg(orc):
    g = _golden("dualscale_cfg_2x4.json")
    X = np.array(g["X"], np.float32)
    W = np.array(g["W"], np.float32)
    codes, s = orc.quantize_activations(X, g["a_bits"])
    assert s.tolist() == g["act_scales"]
    assert codes.tolist() == g["codes"]
    wp = orc.WeightPlan(W, g["w_bits"])
    assert wp.scales.tolist() == g["w_scales"]
    assert wp.codes.tolist() == g["w_codes"]
    y, accp, accn = orc.linear_rows(codes, s, wp, [0, 1])
    assert accp.tolist() == g["acc_plus"]
    assert accn.tolist() == g["acc_minus"]
    assert y.tolist() == g["y"]
    out = orc.cfg_combine(y[:1], y[1:], g["guidance"])
    assert out.tolist() == g["cfg_out"]


# -------------------------------------------------------------- P2 scales --

@pytest.mark.parametrize("bits", [8, 4])
def test_scales_extremes_map_to_qmax(orc, bits):
    x = synth.silu_normal(3, "t/p2", 64, 96)
    s = orc.act_scales(x, bits)
    q = orc.qmax(bits)
    c = orc.quantize_act(x, s, bits)
    assert c.reshape(-1)[np.argmax(x)] == q
    assert c.reshape(-1)[np.argmin(x)] == -q
    assert c.max() == q and c.min() == -q
    # s+ and s- differ for an asymmetric (SiLU) tensor: a swapped pair would
    # put the negative extreme far from -q.
    assert s[0] > 10 * s[1]


def test_scales_degenerate_regions(orc):
    pos = np.abs(synth.silu_normal(4, "t/pos", 8, 8)) + 0.1
    s = orc.act_scales(pos, 8)
    assert s[1] == 0.0 and s[0] > 0
    c = orc.quantize_act(-pos, orc.act_scales(-pos, 8), 8)
    assert (c <= 0).all() and c.min() == -127
    z = np.zeros((4, 4), np.float32)
    z[0, 0] = -0.0
    s0 = orc.act_scales(z, 8)
    assert s0.tolist() == [0.0, 0.0] and not np.signbit(s0).any()
    assert (orc.quantize_act(z, s0, 8) == 0).all()


def test_scales_reject_nonfinite(orc):
    x = np.ones((2, 2), np.float32)
    x[1, 1] = np.inf
    with pytest.raises(orc.OracleError):
        orc.act_scales(x, 8)
    x[1, 1] = np.nan
    with pytest.raises(orc.OracleError):
        orc.quantize_act(x, np.array([1, 1], np.float32), 8)


# --------------------------------------------------- P3 dual -> symmetric --

@pytest.mark.parametrize("bits", [8, 4])
def test_equal_scales_reduce_to_symmetric(orc, bits):
    x = synth.gelu_normal(5, "t/p3", 33, 70)
    q = orc.qmax(bits)
    s_sym = orc.act_scales(x, bits, "symmetric")
    assert s_sym[0] == s_sym[1]
    c = orc.quantize_act(x, s_sym, bits)
    # numpy: IEEE fp32 division and round-half-even, then clip.
    ref = np.clip(np.rint(x / s_sym[0]), -q, q).astype(np.int8)
    assert np.array_equal(c, ref)
    W = synth.weight_normal(5, "t/p3w", 9, 70)
    wp = orc.WeightPlan(W, 8)
    accp, accn = orc.gemm_dual(c, wp.codes)
    acc_sym = c.astype(np.int64) @ wp.codes.astype(np.int64).T
    assert np.array_equal(accp.astype(np.int64) + accn, acc_sym)


def test_weight_codes_match_numpy_symmetric(orc):
    W = synth.weight_normal(6, "t/wq", 17, 40)
    for bits in (8, 4):
        q = orc.qmax(bits)
        sw = orc.weight_scales(W, bits, "channel")
        wc = orc.quantize_weight(W, sw, bits)
        ref = np.clip(np.rint(W / sw[:, None]), -q, q).astype(np.int8)
        assert np.array_equal(wc, ref)
        # absmax row element hits +-q
        am = np.argmax(np.abs(W), axis=1)
        assert (np.abs(wc[np.arange(17), am]) == q).all()


# ------------------------------------------------------ P4 error bound ------

@pytest.mark.parametrize("bits", [8, 4])
def test_quantization_error_bound(orc, bits):
    x = synth.gelu_with_outliers(7, "t/p4", 64, 1152)
    s = orc.act_scales(x, bits)
    c = orc.quantize_act(x, s, bits).astype(np.float64)
    sel = np.where(x >= 0, s[0], s[1]).astype(np.float64)
    err = np.abs(x.astype(np.float64) - sel * c)
    assert (err <= sel / 2 * (1 + 2.0 ** -22)).all()


# ------------------------------------------------------ P5 monotonicity ------

def test_codes_monotone(orc):
    x = np.sort(synth.silu_normal(8, "t/p5", 1, 5000).reshape(-1))
    s = orc.act_scales(x, 8)
    c = orc.quantize_act(x, s, 8).astype(np.int32)
    assert (np.diff(c) >= 0).all()
    c4 = orc.quantize_act(x, orc.act_scales(x, 4), 4).astype(np.int32)
    assert (np.diff(c4) >= 0).all() and c4.min() == -7 and c4.max() == 7


# -------------------------------------------------------- P6 segments -------

def test_segments_special_cases(orc):
    W = synth.weight_normal(9, "t/p6", 24, 16)
    for bits in (8, 4):
        per_t = orc.weight_scales(W, bits, "tensor")
        one = orc.weight_scales(W, bits, "segment", [0, 24])
        assert np.array_equal(per_t, one)
        assert (per_t == per_t[0]).all()
        assert per_t[0] == np.float32(np.abs(W).max()) / np.float32(orc.qmax(bits))
        per_c = orc.weight_scales(W, bits, "channel")
        width1 = orc.weight_scales(W, bits, "segment", list(range(25)))
        assert np.array_equal(per_c, width1)
        seg = [0, 6, 12, 24]
        per_s = orc.weight_scales(W, bits, "segment", seg)
        for g in range(3):
            blk = per_s[seg[g]:seg[g + 1]]
            assert (blk == blk[0]).all()
            # monotone rounding: max of per-channel scales == segment scale
            assert blk[0] == per_c[seg[g]:seg[g + 1]].max()


def test_segments_reject_bad_offsets(orc):
    W = np.ones((8, 4), np.float32)
    for bad in ([0, 4], [1, 8], [0, 4, 4, 8], [0, 6, 3, 8]):
        with pytest.raises(orc.OracleError):
            orc.weight_scales(W, 8, "segment", bad)


# ------------------------------------------------------------- P7 GEMM ------

def _gemm_ref(c, wc):
    c = c.astype(np.int64)
    w = wc.astype(np.int64)
    return np.maximum(c, 0) @ w.T, np.minimum(c, 0) @ w.T


def test_gemm_bruteforce_8x8x8(orc):
    rng = np.random.default_rng(10)
    for _ in range(20):
        c = rng.integers(-128, 128, size=(8, 8)).astype(np.int8)
        w = rng.integers(-128, 128, size=(8, 8)).astype(np.int8)
        accp, accn = orc.gemm_dual(c, w)
        # independent triple loop
        for i in range(8):
            for j in range(8):
                sp = sum(int(c[i, k]) * int(w[j, k]) for k in range(8) if c[i, k] > 0)
                sn = sum(int(c[i, k]) * int(w[j, k]) for k in range(8) if c[i, k] < 0)
                assert accp[i, j] == sp and accn[i, j] == sn


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 17), (13, 7, 64), (9, 33, 1040)])
def test_gemm_random_shapes(orc, M, N, K):
    rng = np.random.default_rng(M * N + K)
    c = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    accp, accn = orc.gemm_dual(c, w)
    rp, rn = _gemm_ref(c, w)
    assert np.array_equal(accp, rp) and np.array_equal(accn, rn)
    rows = [M - 1, 0]
    sp, sn = orc.gemm_dual(c, w, rows)
    assert np.array_equal(sp, rp[rows]) and np.array_equal(sn, rn[rows])


def test_gemm_not_transposed(orc):
    # A non-square case where W^T vs W would differ in shape and value.
    c = np.array([[1, 2, 3]], np.int8)
    w = np.array([[1, 0, 0], [0, 0, 1]], np.int8)
    accp, accn = orc.gemm_dual(c, w)
    assert accp.tolist() == [[1, 3]] and accn.tolist() == [[0, 0]]


def test_gemm_overflow_reported(orc):
    K = 140000
    c = np.full((1, K), 127, np.int8)
    w = np.full((1, K), 127, np.int8)
    with pytest.raises(orc.OracleError):
        orc.gemm_dual(c, w)


# ---------------------------------------------------------- P8 int4 -------

def test_int4_golden_and_roundtrip(orc):
    g = _golden("int4_and_lsb.json")
    for e in g["pack"]:
        b = orc.pack_int4(np.array([e["codes"]], np.int8))
        assert b.tolist() == [[e["byte"]]]
    a, b = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8))
    codes = np.stack([a.reshape(-1), b.reshape(-1)], axis=1).astype(np.int8).reshape(1, -1)
    packed = orc.pack_int4(codes)
    assert np.array_equal(orc.unpack_int4(packed, codes.shape[1]), codes)
    assert len(set(packed.reshape(-1).tolist())) == 256
    with pytest.raises(orc.OracleError):
        orc.pack_int4(np.array([[8, 0]], np.int8))


# ----------------------------------------------------------- P9 TASQ -------

def test_lsb_golden(orc):
    for e in _golden("int4_and_lsb.json")["lsb"]:
        assert orc.truncate_lsb(e["c"], e["k"]) == e["out"], e


def test_lsb_properties_all_codes(orc):
    for k in range(8):
        for c in range(-127, 128):
            t = orc.truncate_lsb(c, k)
            assert t % (1 << k) == 0
            assert abs(c - t) < (1 << k) and abs(t) <= abs(c)
            assert t == 0 or (t > 0) == (c > 0)
            assert orc.truncate_lsb(t, k) == t
            # right-shift form of the same operation on the magnitude
            assert t == int(np.sign(c)) * ((abs(c) >> k) << k)
            if k == 0:
                assert t == c


def test_weight_truncation_bit_planes(orc):
    # A stored code with k planes masked keeps the sign and the planes >= k
    # of its magnitude (the mask equation of TASQ read bit-plane-wise).
    for w_bits in (8, 4):
        q = (1 << (w_bits - 1)) - 1
        c = np.arange(-q, q + 1, dtype=np.int8)
        planes = np.unpackbits(np.abs(c.astype(np.int16)).astype(np.uint8)[:, None], axis=1,
                               bitorder="little")
        for k in range(w_bits):
            kept = (planes[:, k:] * (1 << np.arange(k, 8))).sum(axis=1)
            t = orc.truncate_codes(c, w_bits, k)
            assert np.array_equal(t.astype(np.int64), np.sign(c) * kept), (w_bits, k)
        with pytest.raises(orc.OracleError):
            orc.truncate_codes(c, w_bits, w_bits)
        with pytest.raises(orc.OracleError):
            orc.truncate_codes(np.array([-(q + 1)], np.int8), w_bits, 1)


def test_weight_truncation_gemm(orc):
    # Dropping 4 planes of 8-bit codes leaves a 4-bit grid (codes 16 * j,
    # |j| <= 7): the layer equals the one with codes j and scales 16 * s_w,
    # bit for bit, since the factor 16 is exact in int32 and in fp32.
    W = synth.weight_normal(12, "t/tq/W", 48, 64)
    x = synth.silu_normal(12, "t/tq/X", 24, 64)
    wp = orc.WeightPlan(W, 8)
    v = wp.truncated(4)
    assert np.all(v.codes % 16 == 0) and np.abs(v.codes).max() <= 112
    s = orc.act_scales(x, 8)
    codes = orc.quantize_act(x, s, 8)
    y = orc.epilogue(*orc.gemm_dual(codes, v.codes), s, v.scales)
    y16 = orc.epilogue(*orc.gemm_dual(codes, (v.codes // 16).astype(np.int8)), s,
                       (v.scales * np.float32(16)).astype(np.float32))
    assert np.array_equal(y.view(np.uint32), y16.view(np.uint32))
    # The dropped planes carry the rest of the full-precision product.
    ap, an = orc.gemm_dual(codes, wp.codes)
    tp, tn = orc.gemm_dual(codes, v.codes)
    rp, rn = orc.gemm_dual(codes, (wp.codes - v.codes).astype(np.int8))
    assert np.array_equal(tp + rp, ap) and np.array_equal(tn + rn, an)
    assert np.array_equal(wp.truncated(0).codes, wp.codes)


def test_quantize_with_lsb(orc):
    x = synth.silu_normal(11, "t/p9", 20, 64)
    s = orc.act_scales(x, 8)
    c0 = orc.quantize_act(x, s, 8, 0).astype(np.int32)
    for k in (2, 4):
        ck = orc.quantize_act(x, s, 8, k).astype(np.int32)
        assert np.array_equal(ck, np.sign(c0) * ((np.abs(c0) >> k) << k))
    with pytest.raises(orc.OracleError):
        orc.quantize_act(x, s, 8, 8)
    with pytest.raises(orc.OracleError):
        orc.quantize_act(x, s, 4, 4)


# ------------------------------------------------------ P10 epilogue/CFG ---

def test_epilogue_unit_scales(orc):
    rng = np.random.default_rng(12)
    accp = rng.integers(0, 1 << 20, size=(4, 5)).astype(np.int32)
    accn = -rng.integers(0, 1 << 20, size=(4, 5)).astype(np.int32)
    ones = np.ones(2, np.float32)
    y = orc.epilogue(accp, accn, ones, np.ones(5, np.float32))
    assert np.array_equal(y, accp.astype(np.float32) + accn.astype(np.float32))


def test_epilogue_scales_land_on_their_plane(orc):
    # acc- must be multiplied by s- and acc+ by s+: swapping them changes y.
    accp = np.array([[10]], np.int32)
    accn = np.array([[-3]], np.int32)
    y = orc.epilogue(accp, accn, np.array([2.0, 5.0], np.float32), np.array([0.5], np.float32))
    assert y.tolist() == [[(10 * 2 - 3 * 5) * 0.5]]
    ys = orc.epilogue(accp, accn, np.array([3.0, 3.0], np.float32), np.array([1.0], np.float32),
                      mode="symmetric")
    assert ys.tolist() == [[21.0]]


def test_epilogue_hadamard_fold_is_power_of_two(orc):
    rng = np.random.default_rng(13)
    accp = rng.integers(0, 1 << 24, size=(6, 7)).astype(np.int32)
    accn = -rng.integers(0, 1 << 24, size=(6, 7)).astype(np.int32)
    s = np.array([0.013, 0.0021], np.float32)
    sw = rng.random(7).astype(np.float32)
    y0 = orc.epilogue(accp, accn, s, sw, 0)
    for B in (2, 16, 128):
        yb = orc.epilogue(accp, accn, s, sw, B)
        assert np.array_equal(yb, y0 / np.float32(B))


def test_cfg_properties(orc):
    rng = np.random.default_rng(14)
    yc = rng.standard_normal((5, 9)).astype(np.float32)
    yu = rng.standard_normal((5, 9)).astype(np.float32)
    assert np.array_equal(orc.cfg_combine(yc, yu, 0.0), yu)
    out = orc.cfg_combine(yc, yu, 4.0).astype(np.float64)
    ref = yu.astype(np.float64) + 4.0 * (yc.astype(np.float64) - yu.astype(np.float64))
    scale = np.abs(yu).astype(np.float64) + 4.0 * np.abs(yc - yu)
    assert (np.abs(out - ref) <= 3 * 2.0 ** -24 * scale + 1e-30).all()
    # swapping the branches is not the same combine
    assert not np.allclose(orc.cfg_combine(yu, yc, 4.0), orc.cfg_combine(yc, yu, 4.0))


# ------------------------------------------------------- P11 end to end ----

@pytest.mark.parametrize("a_bits,w_bits,B", [(8, 8, 0), (4, 4, 128), (8, 4, 0), (4, 8, 64)])
def test_end_to_end_error_bound(orc, a_bits, w_bits, B):
    M, N, K = 16, 24, 256
    X = synth.gelu_with_outliers(15, f"t/p11x{a_bits}{w_bits}{B}", M, K)
    W = synth.weight_normal(15, f"t/p11w{a_bits}{w_bits}{B}", N, K)
    codes, s = orc.quantize_activations(X, a_bits, B=B)
    wp = orc.WeightPlan(W, w_bits, B=B)
    y, _, _ = orc.linear_rows(codes, s, wp, range(M))
    Xr = (orc.rotate(X, B) if B else X).astype(np.float64)
    Wr = (orc.rotate(W, B) if B else W).astype(np.float64)
    exact = Xr @ Wr.T / (B if B else 1)
    sx = np.where(Xr >= 0, s[0], s[1]).astype(np.float64)  # [M,K]
    sw = wp.scales.astype(np.float64)  # [N]
    bound = (np.abs(Xr) @ (np.ones((N, K)) * sw[:, None]).T / 2
             + sx @ np.abs(Wr).T / 2 + sx @ (np.ones((N, K)) * sw[:, None]).T / 4)
    bound = bound / (B if B else 1)
    slack = 1e-5 * (np.abs(Xr) @ np.abs(Wr).T) / (B if B else 1) + 1e-6
    assert (np.abs(y - exact) <= bound + slack).all()


# -------------------------------------------------- P12 tiny exhaustive ----

@pytest.mark.parametrize("a_bits", [4, 8])
@pytest.mark.parametrize("w_bits", [4, 8])
@pytest.mark.parametrize("K", [1, 2, 5, 16])
def test_tiny_dequantized_product(orc, a_bits, w_bits, K):
    # y must equal the dequantized dot product sum_k (c_k s_pol(k))(wc_k s_w)
    # up to the few fp32 roundings of the epilogue.
    X = synth.silu_normal(16, f"t/p12x{K}", 6, K)
    W = synth.weight_normal(16, f"t/p12w{K}", 5, K)
    codes, s = orc.quantize_activations(X, a_bits)
    wp = orc.WeightPlan(W, w_bits)
    y, accp, accn = orc.linear_rows(codes, s, wp, range(6))
    c = codes.astype(np.float64)
    sx = np.where(c > 0, s[0], np.where(c < 0, s[1], 0.0))
    deq_x = c * sx
    deq_w = wp.codes.astype(np.float64) * wp.scales[:, None]
    ref = deq_x @ deq_w.T
    mag = np.abs(deq_x) @ np.abs(deq_w).T
    assert (np.abs(y - ref) <= 4 * 2.0 ** -24 * mag + 1e-30).all()
    qa, qw = orc.qmax(a_bits), orc.qmax(w_bits)
    assert np.abs(codes).max() <= qa and np.abs(wp.codes).max() <= qw


def test_all_int4_code_pairs_in_gemm(orc):
    # every (activation code, weight code) pair of 4-bit values, one K-slot each
    a = np.repeat(np.arange(-7, 8), 15).astype(np.int8).reshape(1, -1)
    w = np.tile(np.arange(-7, 8), 15).astype(np.int8).reshape(1, -1)
    accp, accn = orc.gemm_dual(a, w)
    av = np.repeat(np.arange(-7, 8), 15)
    wv = np.tile(np.arange(-7, 8), 15)
    assert accp[0, 0] == int((np.maximum(av, 0) * wv).sum())
    assert accn[0, 0] == int((np.minimum(av, 0) * wv).sum())


def test_bf16_conversion_exact(orc):
    x = synth.normal_f64(17, "t/bf", (1000,)).astype(np.float32)
    b = synth.f32_to_bf16_bits(x)
    f = orc.bf16_to_f32(b)
    assert np.array_equal(f.view(np.uint32) >> 16, b.astype(np.uint32))
    assert (np.abs(f - x) <= np.abs(x) * 2.0 ** -8).all()


# ------------------------------------------------------------- GAMP ---------

def test_gamp_golden(orc):
    for c in _golden("gamp_greedy.json")["cases"]:
        a, b = orc.gamp_allocate(c["macs"], c["gain"], c["w_bits"], c["budget"])
        assert a.tolist() == c["a_bits"] and b == c["bops"], c["note"]


def _brute_force(macs, gain, w_bits, budget):
    n = len(macs)
    base = sum(m * w_bits * 4 for m in macs)
    best = 0.0
    for mask in range(1 << n):
        cost = base + sum(macs[l] * w_bits * 4 for l in range(n) if mask >> l & 1)
        if cost <= budget:
            best = max(best, sum(gain[l] for l in range(n) if mask >> l & 1))
    return best


def test_gamp_against_exhaustive_search(orc):
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(1, 9))
        w_bits = int(rng.choice([4, 8]))
        gain = rng.lognormal(0, 1, n)
        equal = trial % 2 == 0
        macs = np.full(n, 1000, np.int64) if equal else rng.integers(1, 5000, n)
        base = int(sum(int(m) * w_bits * 4 for m in macs))
        budget = base + int(rng.integers(0, int(macs.sum()) * w_bits * 4 + 1))
        a, bops = orc.gamp_allocate(macs, gain, w_bits, budget)
        assert set(a.tolist()) <= {4, 8}
        assert bops == int(sum(int(m) * w_bits * int(b) for m, b in zip(macs, a))) <= budget
        got = float(sum(g for g, b in zip(gain, a) if b == 8))
        opt = _brute_force([int(m) for m in macs], list(gain), w_bits, budget)
        if equal:
            # equal costs: the greedy by gain is the optimum
            assert got == pytest.approx(opt, rel=1e-12)
        else:
            # greedy knapsack bound: greedy + the largest single gain >= optimum
            assert got + gain.max() >= opt * (1 - 1e-12)
        # no unpromoted layer still fits in the remaining budget
        for l in range(n):
            if a[l] == 4:
                assert bops + int(macs[l]) * w_bits * 4 > budget


def test_gamp_extremes(orc):
    macs = np.array([5, 7, 11, 13], np.int64)
    gain = np.array([0.5, 3.0, 1.0, 2.0])
    lo = int(macs.sum()) * 4 * 4
    a, b = orc.gamp_allocate(macs, gain, 4, lo)
    assert a.tolist() == [4, 4, 4, 4] and b == lo
    a, b = orc.gamp_allocate(macs, gain, 4, 2 * lo)
    assert a.tolist() == [8, 8, 8, 8] and b == 2 * lo
    for bad in [dict(budget=lo - 1), dict(w_bits=6)]:
        kw = dict(macs=macs, gain=gain, w_bits=4, budget=lo)
        kw.update(bad)
        with pytest.raises(orc.OracleError):
            orc.gamp_allocate(**kw)
    with pytest.raises(orc.OracleError):
        orc.gamp_allocate(np.array([0, 1]), np.array([1.0, 1.0]), 4, 1000)
    with pytest.raises(orc.OracleError):
        orc.gamp_allocate(np.array([1, 1]), np.array([-1.0, 1.0]), 4, 1000)


# ------------------------------------------------ single Hadamard (HQ-DM) ----

@pytest.mark.parametrize("B", [4, 16, 128])
def test_single_hadamard_weights_vs_scipy(orc, B):
    rng = np.random.default_rng(B)
    K = 2 * B
    wc = rng.integers(-127, 128, (5, K)).astype(np.int8)
    v = orc.hadamard_weight_int(wc, B)
    H = scipy.linalg.hadamard(B).astype(np.int64)
    ref = np.concatenate([wc[:, j:j + B].astype(np.int64) @ H for j in range(0, K, B)], axis=1)
    assert np.array_equal(v, ref)
    # applying H again gives B times the codes (H H = B I)
    back = np.concatenate([v[:, j:j + B].astype(np.int64) @ H for j in range(0, K, B)], axis=1)
    assert np.array_equal(back, B * wc.astype(np.int64))
    assert np.abs(v).max() <= B * 127


def test_int64_gemm_beyond_int32(orc):
    rng = np.random.default_rng(3)
    K = 4608
    c = np.full((2, K), 127, np.int8)
    c[1] = rng.integers(-127, 128, K)
    v = np.full((3, K), 16256, np.int32)
    v[2] = rng.integers(-16256, 16257, K)
    acc = orc.gemm_int64(c, v)
    assert acc[0, 0] == 127 * 16256 * K > 2 ** 31
    assert np.array_equal(acc, c.astype(np.int64) @ v.astype(np.int64).T)


def test_single_epilogue_rounding(orc):
    acc = np.array([[2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 33 + 5), 7, 0, 123456789012]], np.int64)
    sw = np.ones(acc.shape[1], np.float32)
    y = orc.epilogue_single(acc, 1.0, sw, 1)
    assert np.array_equal(y, acc.astype(np.float32))  # one round to nearest even
    y8 = orc.epilogue_single(acc, 1.0, sw, 8)
    assert np.array_equal(y8, acc.astype(np.float32) / np.float32(8))


def test_single_hadamard_exact_on_grid(orc):
    # Inputs built so that nothing is lost to quantization: X = (s/B) C H with
    # max|C| = 127 in every tensor, W = s_w W_int with max|W_int| = 127 per
    # row, s and s_w powers of two. The single-Hadamard layer then returns
    # X W^T rounded once, computed here from the integers alone.
    rng = np.random.default_rng(5)
    B, M, K, N = 16, 6, 64, 10
    H = scipy.linalg.hadamard(B).astype(np.int64)
    C = rng.integers(-127, 128, (M, K))
    C[0, 0] = 127
    Hk = np.kron(np.eye(K // B, dtype=np.int64), H)
    s = 2.0 ** -6
    X = (s / B * (C @ Hk)).astype(np.float32)
    assert np.array_equal(X.astype(np.float64), s / B * (C @ Hk))  # exact in fp32
    Wi = rng.integers(-127, 128, (N, K))
    Wi[:, 0] = 127
    sw = 2.0 ** -9
    W = (sw * Wi).astype(np.float32)
    codes, sc = orc.quantize_activations(X, 8, B=B, mode="symmetric")
    assert sc[0] == np.float32(s) and np.array_equal(codes, C)
    wp = orc.SingleHadamardPlan(W, 8, B)
    assert np.array_equal(wp.codes, Wi) and np.all(wp.scales == np.float32(sw))
    y = orc.epilogue_single(orc.gemm_int64(codes, wp.v), sc[0], wp.scales, B)
    exact = (C @ Hk) @ Wi.T  # = B (X W^T) / (s s_w), integers
    ref = (exact.astype(np.float64) * (s * sw / B)).astype(np.float32)
    assert np.array_equal(y, ref)
    assert np.allclose(y, X.astype(np.float64) @ W.astype(np.float64).T, rtol=0, atol=1e-6)


# --------------------------------------------- SegLinear input segments -----

def test_input_segments_one_branch_is_unsegmented(orc):
    X = synth.gelu_with_outliers(31, "kseg/one/X", 40, 256)
    W = synth.weight_normal(31, "kseg/one/W", 24, 256)
    for B, mode in [(0, "dual"), (128, "dual"), (16, "symmetric")]:
        wp = orc.WeightPlan(W, 8, B=B)
        sp = orc.InputSegmentedPlan(W, 8, [0, 256], B=B)
        assert np.array_equal(sp.codes, wp.codes) and np.array_equal(sp.scales[0], wp.scales)
        c1, s1 = orc.quantize_activations(X, 8, B=B, mode=mode)
        c2, s2 = orc.quantize_activations_segmented(X, 8, [0, 256], B=B, mode=mode)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2[0])
        rows = np.arange(40)
        y1, _, _ = orc.linear_rows(c1, s1, wp, rows, mode)
        y2, _ = orc.linear_segmented_rows(c2, s2, sp, rows, mode)
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_input_segments_exact_on_grid(orc):
    # Two branches on their own quantization grids (power-of-two scales that
    # differ by 2^8 between the branches, max codes reached in each): the
    # segmented layer returns X W^T rounded once, from the integers alone.
    # One shared scale pair would round the small branch's values to zero.
    rng = np.random.default_rng(32)
    M, N, offs = 12, 20, [0, 128, 384]
    s_b = [2.0 ** -3, 2.0 ** -11]
    w_b = [2.0 ** -7, 2.0 ** -5]
    C = rng.integers(-127, 128, (M, 384))
    C[0, 0] = C[0, 128] = 127
    C[1, 1] = C[1, 129] = -127
    Wi = rng.integers(-127, 128, (N, 384))
    Wi[:, 0] = Wi[:, 128] = 127
    X = np.concatenate([C[:, :128] * s_b[0], C[:, 128:] * s_b[1]], axis=1).astype(np.float32)
    W = np.concatenate([Wi[:, :128] * w_b[0], Wi[:, 128:] * w_b[1]], axis=1).astype(np.float32)
    wp = orc.InputSegmentedPlan(W, 8, offs)
    codes, s = orc.quantize_activations_segmented(X, 8, offs)
    assert np.array_equal(codes, C) and np.array_equal(wp.codes, Wi)
    assert s.tolist() == [[s_b[0], s_b[0]], [s_b[1], s_b[1]]]
    y, accs = orc.linear_segmented_rows(codes, s, wp, np.arange(M))
    exact = (C[:, :128] @ Wi[:, :128].T) * (s_b[0] * w_b[0]) + \
            (C[:, 128:] @ Wi[:, 128:].T) * (s_b[1] * w_b[1])
    assert np.array_equal(y, exact.astype(np.float32))
    ap, an = accs[1]
    cp = np.maximum(C[:, 128:], 0)
    assert np.array_equal(ap, cp @ Wi[:, 128:].T) and np.array_equal(an, (C[:, 128:] - cp) @ Wi[:, 128:].T)
    # a single scale pair over the concatenation loses the second branch
    c1, s1 = orc.quantize_activations(X, 8)
    assert np.count_nonzero(c1[:, 128:]) == 0
