"""The quantizer kernel divides by the scale with a reciprocal and one FMA
correction step instead of an IEEE divide (residual taken as q0 s - x so
that signed zeros come out right without a sign copy), and computes the
scale amax / 448 the same way.  For fp32 inputs (the fused producers) the
first quotient comes from a two-term reciprocal (yd + yl), which makes it
faithful, before the correction.  This CPU test checks, for every pair of
(bf16 value significand, scale significand) the activation path can
produce, for random fp32 values (the fused producers quantize fp32 values),
and for every fp32 significand divided by 448, that the 3-operation
sequence gives exactly the IEEE single-precision quotient.  Scales come from bf16 amax values (one per
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


def _recip_pair(s):
    """yn = RN(1/s); yd = yn, or its predecessor when s yn > 1; yl = RN(RN(1 - s yd) yd)."""
    s = s.astype(np.float32)
    yn = (np.float32(1) / s).astype(np.float32)
    e = _exact_fma_vec(-s, yn, np.ones_like(s))
    yd = np.where(e < 0, (yn.view(np.uint32) - np.uint32(1)).view(np.float32), yn).astype(np.float32)
    yl = (_exact_fma_vec(-s, yd, np.ones_like(s)) * yd).astype(np.float32)
    assert np.all(yl >= 0)
    return yn, yd, yl


def _kernel_div_f32_vec(x, s):
    """The fp32-input division: q0 = RN(x yd + RN(x yl)) (faithful), then one
    Markstein correction with yn = RN(1/s)."""
    x = x.astype(np.float32)
    s = np.broadcast_to(s, x.shape).astype(np.float32)
    yn, yd, yl = _recip_pair(s)
    q0 = _exact_fma_vec(x, yd, (x * yl).astype(np.float32))
    r = _exact_fma_vec(q0, s, -x)
    return _exact_fma_vec(-r, yn, q0)


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


def test_fp32_division_matches_ieee_for_random_fp32_inputs():
    x, s, y = _random_fp32_groups(1 << 20, 97)
    got = _kernel_div_f32_vec(x, s)
    ref = (x / s).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the hardest significands: x just below a power of two over scales with
    # significands near 2 (largest error of RN(1/s))
    xs = (np.uint32(0x3FFFFFFF) - np.arange(4096, dtype=np.uint32)).view(np.float32)
    for sb in (0x3FFFFFFF, 0x3FFFFF00, 0x3F800001, 0x3FB504F3):
        s1 = np.uint32(sb).view(np.float32)
        got = _kernel_div_f32_vec(xs, s1)
        assert np.array_equal(got.view(np.uint32), (xs / s1).astype(np.float32).view(np.uint32))


def test_fp32_division_signed_zero_and_tiny():
    # scales whose reciprocal pair has yl > 0, yl = 0 (power of two) and yd < yn
    for s in (np.float32(1.0), np.float32(3.0) / np.float32(448), np.float32(1e30), np.float32(0.3),
              np.float32(0.7), np.float32(1.1)):
        xs = np.array([0.0, -0.0, -2.0 ** -133, 2.0 ** -133, -1e-38, 1e-30, -3e-36], np.float32)
        got = _kernel_div_f32_vec(xs, s)
        ref = (xs / s).astype(np.float32)
        assert np.array_equal(np.signbit(got), np.signbit(xs))
        big = np.abs(ref) >= 2.0 ** -60
        assert np.array_equal(got[big], ref[big])
