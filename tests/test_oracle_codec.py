"""Pins of the oracle's e4m3fn codec (CPU only).

The codec is pinned against: the OCP e4m3fn definition worked by hand
(tests/golden/e4m3fn_codes.txt), torch's own float8_e4m3fn conversion (an
independent library routine; round to nearest even, sign of zero kept), the
round trip over every finite code, and every midpoint between neighbours.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.txt")


def _golden():
    dec, enc = [], []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, a, b = line.split()
        if kind == "decode":
            dec.append((int(a, 16), float(b)))
        else:
            enc.append((np.float32(float(a)), int(b, 16)))
    return dec, enc


def test_golden_decode():
    dec, _ = _golden()
    for code, val in dec:
        got = oracle.e4m3_decode([code])[0]
        assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_golden_encode():
    _, enc = _golden()
    for t, code in enc:
        assert oracle.e4m3_encode([t])[0] == code, (t, hex(code))


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    # largest finite and smallest subnormal / normal
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_midpoints_round_to_even():
    vals = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    for c in range(126):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)  # at most 5 significant bits: exact
        assert float(mid) == (vals[c] + vals[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        for sgn in (1, -1):
            t = np.float32(sgn * mid)
            exp = even | (0x80 if sgn < 0 else 0)
            assert oracle.e4m3_encode([t])[0] == exp, (c, t)
            below = np.nextafter(np.float32(mid), np.float32(0))
            above = np.nextafter(np.float32(mid), np.float32(1e9))
            assert oracle.e4m3_encode([np.float32(sgn * below)])[0] == (c | (exp & 0x80))
            assert oracle.e4m3_encode([np.float32(sgn * above)])[0] == ((c + 1) | (exp & 0x80))


def test_sign_of_zero_and_underflow():
    t = np.array([0.0, -0.0, -2.0 ** -11, 2.0 ** -11, -1e-30, 1e-45, -1e-45], dtype=np.float32)
    assert list(oracle.e4m3_encode(t)) == [0x00, 0x80, 0x80, 0x00, 0x80, 0x00, 0x80]


def _torch_codes(f: np.ndarray) -> np.ndarray:
    return torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_exhaustive_positive_fp32_vs_torch():
    """Every fp32 bit pattern in [+0, 448] (1.14e9 values) against torch."""
    top = int(np.float32(448.0).view(np.uint32))
    chunk = 1 << 26
    start = 0
    while start <= top:
        n = min(chunk, top + 1 - start)
        bits = np.arange(start, start + n, dtype=np.uint32)
        f = bits.view(np.float32)
        ours = oracle.e4m3_encode(f)
        ref = _torch_codes(f)
        if not np.array_equal(ours, ref):
            bad = np.nonzero(ours != ref)[0][:5]
            raise AssertionError([(hex(int(bits[i])), float(f[i]), ours[i], ref[i]) for i in bad])
        start += n


def test_negative_fp32_vs_torch_strided():
    """Negative half: every 7th pattern plus all patterns near code boundaries."""
    top = int(np.float32(448.0).view(np.uint32))
    bits = np.arange(0, top + 1, 7, dtype=np.uint32)
    vals = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2]).astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-64, 65)[None, :]).ravel()
    near = near[(near >= 0) & (near <= top)].astype(np.uint32)
    bits = np.concatenate([bits, near]) | np.uint32(0x80000000)
    f = bits.view(np.float32)
    assert np.array_equal(oracle.e4m3_encode(f), _torch_codes(f))
