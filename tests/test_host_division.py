"""The quantizer kernel divides by the scale with a reciprocal and one FMA
correction step instead of an IEEE divide.  This CPU test checks, for every
pair of (bf16 value significand, scale significand) the activation path can
produce, that the 3-operation sequence plus the sign copy gives exactly the
IEEE single-precision quotient.  Scales come from bf16 amax values (one per
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
    r = np.float32(_libm.fmaf(float(-q0), float(s), float(x)))
    t = np.float32(_libm.fmaf(float(r), float(y), float(q0)))
    return np.copysign(t, x)


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
