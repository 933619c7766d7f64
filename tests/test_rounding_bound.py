"""The quantizer kernels' fast-path tests, emulated exactly on the CPU.

The code of a value is round-half-even of the IEEE quotient Q = fl(v / s),
clamped to +-qa (SegQuant explainer, section 2.B, DualScale quantization).
The kernels avoid the division: they take the integer of a product with
fl(1/s) and keep it only when a margin test proves it equals rint(Q),
else they divide. These tests replay both tests' decisions with exact
float64 arithmetic (a product of two float32 values is exact in float64)
on values on and within a few ulps of half-integer quotients, and require
that no kept integer differs from the definition; a margin that is too
small must be caught by the same check. No GPU and no oracle involved.
"""
import numpy as np
import pytest

f32 = np.float32


def _near_half(rng, n, qa, mx):
    """Values whose quotient by fl(mx/qa) is within +-8 ulps of k + 1/2."""
    s = (mx / f32(qa)).astype(f32)
    h = rng.integers(-qa, qa, n) + 0.5
    v = (h * s.astype(np.float64)).astype(f32)
    k = rng.integers(-8, 9, n)
    for i in range(1, 9):
        m = k >= i
        v[m] = np.nextafter(v[m], f32(np.inf))
        m = k <= -i
        v[m] = np.nextafter(v[m], f32(-np.inf))
    return np.clip(v, -mx, mx)


def _at_max(rng, n, mx):
    v = mx.copy()
    j = rng.integers(0, 4, n)
    for i in range(1, 4):
        m = j >= i
        v[m] = np.nextafter(v[m], f32(0))
    return v * np.where(rng.random(n) < 0.5, f32(1), f32(-1))


def _reference(v, s, qa):
    q = (v / s).astype(f32)  # correctly rounded quotient
    return np.clip(np.rint(q.astype(np.float64)), -qa, qa)


def _own_scale_fast(v, mx, qa, margin_ulps=1.0):
    """One-pass form: scales from the tensor's own maxima. c = rint(v*r)
    (what fma(v, r, 1.5*2^23) - 1.5*2^23 gives), e = fl(v*r - c) (what
    fma(v, r, -c) gives), kept when |e| < 0.5 - (qa + 1) 2^-23."""
    s = (mx / f32(qa)).astype(f32)
    r = (f32(1) / s).astype(f32)
    p = v.astype(np.float64) * r.astype(np.float64)
    c = np.rint(p)
    e = (p - c).astype(f32)
    lim = f32(0.5 - (qa + 1) * 2.0 ** -23 * margin_ulps)
    return s, c, np.abs(e) < lim


def _product_fast(v, s, margin=2.0 ** -22):
    """General form (any scale): t = fl(v*r), kept when
    fl(|t| 2^-22 + |t - rint t|) < 0.5 - 2^-23, then clamped."""
    r = (f32(1) / s).astype(f32)
    t = (v * r).astype(f32)
    # (non-finite t gives a NaN z, and |t| >= 2^21 a z >= 0.5: both fail)
    with np.errstate(invalid="ignore"):
        ri = np.rint(t.astype(np.float64))
        d = np.abs(t.astype(np.float64) - ri).astype(f32)
        z = (np.abs(t).astype(np.float64) * margin + d.astype(np.float64)).astype(f32)
        return ri, z < f32(0.5 - 2.0 ** -23)


@pytest.mark.parametrize("qa", [127, 63, 15, 7, 3])
def test_own_scale_fast_path_matches_division(qa):
    rng = np.random.default_rng(100 + qa)
    n = 400_000
    mx = np.exp(rng.uniform(-40, 40, n)).astype(f32)
    for v in (_near_half(rng, n, qa, mx), _at_max(rng, n, mx),
              np.clip((rng.standard_normal(n) * mx / 4).astype(f32), -mx, mx)):
        s, c, fast = _own_scale_fast(v, mx, qa)
        ref = _reference(v, s, qa)
        assert not np.any(fast & (c != ref))
        assert not np.any(fast & (np.abs(c) > qa))  # no clamp needed
    # the near-half set really probes the boundary: a margin 16x too small errs
    v = _near_half(rng, n, qa, mx)
    s, c, fast = _own_scale_fast(v, mx, qa, margin_ulps=1.0 / 16)
    assert np.count_nonzero(fast & (c != _reference(v, s, qa))) > 0


def test_general_fast_path_matches_division():
    rng = np.random.default_rng(7)
    n = 400_000
    for qa in (127, 7):
        s = np.exp(rng.uniform(-30, 5, n)).astype(f32)  # arbitrary (static) scales
        v = _near_half(rng, n, qa, (s * f32(qa)).astype(f32))
        v2 = (rng.standard_normal(n) * 300).astype(f32) * s  # far beyond the range too
        v3 = np.concatenate([np.array([np.inf, -np.inf, np.nan], f32),
                             (np.float32(2.0 ** 21) * s[:1000]).astype(f32),
                             (np.float32(2.0 ** 23) * s[:1000]).astype(f32)])
        ri, fast = _product_fast(v3, np.concatenate([s[:3], s[:1000], s[:1000]]))
        assert not fast.any()  # these always take the division
        for x in (v, v2):
            ri, fast = _product_fast(x, s)
            ref = _reference(x, s, qa)
            assert not np.any(fast & (np.clip(ri, -qa, qa) != ref))
        ri, fast = _product_fast(v, s, margin=2.0 ** -26)
        assert np.count_nonzero(fast & (np.clip(ri, -qa, qa) != _reference(v, s, qa))) > 0
