"""The quantizer kernel divides by the scale with a reciprocal and one FMA
correction step instead of an IEEE divide (residual taken as q0 s - x so
that signed zeros come out right without a sign copy), and computes the
scale amax / 448 the same way.  For fp32 inputs (the fused producers) the
quotient is a float64 product x d rounded to fp32, with d a float64
reciprocal of the scale from three Newton steps.  This CPU test checks, for
every pair of (bf16 value significand, scale significand) the activation
path can produce, for random and near-midpoint fp32 values (the fused
producers quantize fp32 values), and for every fp32 significand divided by
448, that these sequences give exactly the IEEE single-precision quotient;
and, with exact rational arithmetic, that the Newton steps reach 2^-52 from
any starting reciprocal within 2^-8.  Scales come from bf16 amax values (one per
bf16 significand) and from eps; power-of-two (UE8M0) scales are exact
trivially and are checked too.  Scaling x or s by powers of two scales every
intermediate exactly, so significands at one exponent cover the normal range;
the tiny and signed-zero cases are checked separately.
"""
import ctypes
import ctypes.util

import numpy as np

_libm = ctypes.CDLL(ctypes.util.find_library("m"))
_libm.fmaf.restype = ctypes.c_float
_libm.fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]


def _kernel_div(x: np.float32, s: np.float32, y: np.float32) -> np.float32:
    q0 = np.float32(x * y)
    r = np.float32(_libm.fmaf(float(q0), float(s), float(-x)))
    return np.float32(_libm.fmaf(float(-r), float(y), float(q0)))


def _kernel_div_vec(x: np.ndarray, s: np.ndarray, y: np.ndarray) -> np.ndarray:
    """The same three operations on arrays.  q0 s - x is exact in float64 (48-bit
    product, difference within 53 bits) and, by the theorem, representable in
    fp32 (asserted).  q0 - r y is exact only to float64, so the few results
    whose float64 value sits within a few float64 ulps of an fp32 rounding
    midpoint are recomputed with the C library's exact fmaf."""
    x = x.astype(np.float32)
    s = np.broadcast_to(s, x.shape).astype(np.float32)
    y = np.broadcast_to(y, x.shape).astype(np.float32)
    q0 = (x * y).astype(np.float32)
    r64 = q0.astype(np.float64) * s.astype(np.float64) - x.astype(np.float64)
    r = r64.astype(np.float32)
    assert np.array_equal(r.astype(np.float64), r64), "residual not exact in fp32"
    t64 = q0.astype(np.float64) - r.astype(np.float64) * y.astype(np.float64)
    t = t64.astype(np.float32)
    half = np.spacing(np.abs(t)).astype(np.float64) / 2
    near = np.abs(np.abs(t64 - t.astype(np.float64)) - half) <= 4 * np.spacing(np.abs(t64))
    for i in np.nonzero(near)[0]:
        t[i] = _kernel_div(x[i], s[i], y[i])
    return t


def _exact_fma_vec(a, b, c):
    """RN32(a b + c) for fp32 arrays: a b is exact in float64; where the
    float64 sum could sit on an fp32 rounding midpoint the C library's exact
    fmaf is used instead."""
    t64 = a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)
    t = t64.astype(np.float32)
    half = np.spacing(np.abs(t)).astype(np.float64) / 2
    near = np.abs(np.abs(t64 - t.astype(np.float64)) - half) <= 4 * np.spacing(np.abs(t64))
    for i in np.nonzero(near)[0]:
        t[i] = _libm.fmaf(float(a[i]), float(b[i]), float(c[i]))
    return t


def _bf16_significands():
    # every bf16 value in [1, 2): 128 patterns
    bits = (np.arange(128, dtype=np.uint32) + np.uint32(0x3F80)) << 16
    return bits.view(np.float32)


def test_markstein_division_matches_ieee_for_bf16_inputs():
    xs = _bf16_significands()
    amaxs = _bf16_significands()
    scales = [np.float32(a) / np.float32(448) for a in amaxs]
    scales.append(np.float32(1e-10) / np.float32(448))
    scales += [np.float32(2.0) ** e for e in (-3, 0, 5)]
    bad = []
    for s in scales:
        s = np.float32(s)
        y = np.float32(1) / s
        for x0 in xs:
            for ex in (-14, -9, -3, 0, 4, 8):
                for sign in (1, -1):
                    x = np.float32(sign * x0 * np.float32(2.0) ** ex)
                    # same relative position with a scale of a different exponent
                    ref = np.float32(x / s)
                    got = _kernel_div(x, s, y)
                    if got.view(np.uint32) != ref.view(np.uint32):
                        bad.append((float(x), float(s), float(got), float(ref)))
    assert not bad, bad[:5]


def test_signed_zero_and_tiny_values():
    """Where an intermediate underflows the quotient may differ in its last
    bit, but only far below 2^-10, where every value encodes to a signed zero:
    the e4m3 code (sign and zero) must still agree."""
    for s in (np.float32(1.0), np.float32(3.0) / np.float32(448), np.float32(1e30)):
        y = np.float32(1) / s
        for x in (np.float32(0.0), np.float32(-0.0), np.float32(-2.0 ** -133), np.float32(2.0 ** -133),
                  np.float32(-1e-38), np.float32(1e-30), np.float32(-3e-36)):
            ref = np.float32(x / s)
            got = _kernel_div(x, s, y)
            if got.view(np.uint32) != ref.view(np.uint32):
                assert abs(ref) < 2.0 ** -60 and abs(got) < 2.0 ** -60, (x, s, got, ref)
            assert np.signbit(got) == np.signbit(ref) == np.signbit(x)


def test_scale_division_by_448_for_every_fp32_significand():
    # every significand at one exponent (the quotient and residual scale
    # exactly with the exponent of amax) plus both ends of the range in use
    m = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)
    y = np.float32(1) / np.float32(448)
    assert float(y) == float.fromhex("0x1.24924ap-9")
    for a in (m, m * np.float32(2.0 ** -100), m * np.float32(2.0 ** 127)):
        got = _kernel_div_vec(a, np.float32(448), y)
        ref = (a / np.float32(448)).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _random_fp32_groups(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    x = (g.standard_normal(n) * np.exp(g.uniform(-20, 20, n))).astype(np.float32)
    amax = np.abs((g.standard_normal(n) * np.exp(g.uniform(-20, 20, n)))).astype(np.float32)
    s = (np.maximum(amax, np.float32(1e-10)) / np.float32(448)).astype(np.float32)
    x = np.clip(x, -amax, amax).astype(np.float32)  # |x| <= amax, as in a group
    return x, s, (np.float32(1) / s).astype(np.float32)


def test_one_step_division_is_not_enough_for_fp32_inputs():
    # with 24-bit x, q0 = RN(x y) can be 1.5 ulp off and the residual then
    # needs 25 bits: the single-step form is reserved for bf16 inputs
    x, s, y = _random_fp32_groups(1 << 16, 96)
    q0 = (x * y).astype(np.float32)
    r64 = q0.astype(np.float64) * s.astype(np.float64) - x.astype(np.float64)
    assert np.any(r64.astype(np.float32).astype(np.float64) != r64)


def _fma64(a, b, c):
    """float64 FMA, exactly: the rational a b + c rounded once (CPython's
    integer true division is correctly rounded)."""
    from fractions import Fraction
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _recip_f64(s: float, d0: float) -> float:
    """The kernel's three Newton steps d <- d + d (1 - s d), each with two FMAs."""
    d = d0
    for _ in range(3):
        d = _fma64(d, _fma64(-s, d, 1.0), d)
    return d


def test_newton_reciprocal_reaches_2_pow_minus_52_from_2_pow_minus_8():
    from fractions import Fraction
    g = np.random.Generator(np.random.PCG64(98))
    sig = np.concatenate([
        (np.uint32(0x3F800000) | g.integers(0, 1 << 23, 600, dtype=np.uint32)),
        np.array([0x3F800000, 0x3F800001, 0x3FFFFFFF, 0x3FB504F3, 0x3FAAAAAB], np.uint32)]).view(np.float32)
    worst = 0.0
    for i, m in enumerate(sig):
        for e in (-100, -20, 0, 30):
            s = float(np.float32(m * np.float32(2.0) ** e))
            for eps0 in (2.0 ** -8, -(2.0 ** -8), float(g.uniform(-2.0 ** -8, 2.0 ** -8)), 0.0):
                d0 = float(Fraction(1) / Fraction(s) * (1 + Fraction(eps0)))
                d = _recip_f64(s, d0)
                err = abs(float(Fraction(d) * Fraction(s) - 1))
                worst = max(worst, err)
    assert worst <= 2.0 ** -52, worst


def _div_f64_product(x, d):
    """The kernel's fp32-input division: RN32(RN64(x d))."""
    return (x.astype(np.float64) * d).astype(np.float32)


def _reciprocals_at_the_error_bound(s):
    """RN64(1/s) and its neighbours two float64 ulps away on either side
    (relative error up to 2^-51, beyond the 2^-52 the Newton steps reach)."""
    d = 1.0 / s.astype(np.float64)
    up = np.nextafter(np.nextafter(d, np.inf), np.inf)
    dn = np.nextafter(np.nextafter(d, 0), 0)
    return (d, up, dn)


def test_f64_product_division_matches_ieee_for_random_fp32_inputs():
    x, s, _ = _random_fp32_groups(1 << 20, 97)
    ref = (x / s).astype(np.float32)
    for d in _reciprocals_at_the_error_bound(s):
        got = _div_f64_product(x, d)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_f64_product_division_near_rounding_midpoints():
    # x = RN32(m s) for fp32 rounding midpoints m (odd 25-bit significands):
    # the quotients x / s closest to a midpoint that fp32 operands can give
    g = np.random.Generator(np.random.PCG64(99))
    mids = ((g.integers(1 << 23, 1 << 24, 1 << 14, dtype=np.int64) * 2 + 1).astype(np.float64)) * 2.0 ** -24
    sigs = np.concatenate([
        (np.uint32(0x3F800000) | g.integers(0, 1 << 23, 62, dtype=np.uint32)),
        np.array([0x3FFFFFFF, 0x3F800001], np.uint32)]).view(np.float32)
    for sb in sigs:
        for e in (-30, 0, 7):
            s1 = np.float32(sb * np.float32(2.0) ** e)
            x0 = (mids * np.float64(s1)).astype(np.float32)  # m s is exact in float64
            xs = np.concatenate([x0, np.nextafter(x0, np.float32(np.inf)), np.nextafter(x0, np.float32(0)), -x0])
            s = np.full(xs.shape, s1, np.float32)
            ref = (xs / s).astype(np.float32)
            for d in _reciprocals_at_the_error_bound(s):
                got = _div_f64_product(xs, d)
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (float(s1),)


def _closest_quotients(n_s=64, seed=5):
    """Pairs (x, s) whose quotient lies as close to an fp32 rounding midpoint
    as fp32 operands allow: for an odd scale significand S and a midpoint
    significand M (odd, 25 bits) with M S = +-r (mod 2^25), r small and odd,
    x = RN32(M S) differs from the midpoint times s by r units of 2^-47."""
    g = np.random.Generator(np.random.PCG64(seed))
    xs, ss = [], []
    for S in (g.integers(1 << 22, 1 << 23, n_s) * 2 + 1):
        S = int(S)
        inv = pow(S, -1, 1 << 25)
        for r in range(1, 40, 2):
            for sg in (1, -1):
                M = (sg * r * inv) % (1 << 25)
                if M < (1 << 24):
                    continue
                s = np.float32(S * 2.0 ** -23)
                xs.append(np.float32(M * 2.0 ** -24 * float(s)))  # the 49-bit product rounded once
                ss.append(s)
    return np.array(xs, np.float32), np.array(ss, np.float32)


def test_f64_product_division_at_the_closest_quotients():
    x, s = _closest_quotients()
    assert len(x) > 1000
    ref = (x / s).astype(np.float32)
    for d in _reciprocals_at_the_error_bound(s):
        assert np.array_equal(_div_f64_product(x, d).view(np.uint32), ref.view(np.uint32))
    # these cases are hard: a reciprocal 2^-47 off already changes results
    d_bad = (1.0 / s.astype(np.float64)) * (1 + 2.0 ** -47)
    assert np.any(_div_f64_product(x, d_bad) != ref)


def test_f64_product_division_signed_zero_and_tiny():
    for s in (np.float32(1.0), np.float32(3.0) / np.float32(448), np.float32(1e30), np.float32(0.3),
              np.float32(0.7), np.float32(1.1)):
        xs = np.array([0.0, -0.0, -2.0 ** -133, 2.0 ** -133, -1e-38, 1e-30, -3e-36], np.float32)
        s_ = np.full(xs.shape, s, np.float32)
        ref = (xs / s_).astype(np.float32)
        for d in _reciprocals_at_the_error_bound(s_):
            got = _div_f64_product(xs, d)
            assert np.array_equal(np.signbit(got), np.signbit(xs))
            big = np.abs(ref) >= 2.0 ** -60
            assert np.array_equal(got[big], ref[big])
