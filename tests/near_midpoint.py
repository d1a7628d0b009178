"""Exact comparison of a producer's codes and scales with the oracle's, where
the oracle's float32 intermediate is the single rounding of a float64 value.

The oracle computes silu(g) * u (and RMSNorm's 1/rms) in float64 and rounds
it once to float32.  The kernel reaches the same float32 value through a
different float64 evaluation; both float64 values lie within a few float64
ulps of the true value, so the two float32 roundings can only differ where
the oracle's float64 value is within that distance of a float32 rounding
midpoint.  Such positions are found from the oracle alone (never from the
kernel's output): every value within ``rel`` (relative) of a midpoint is
flagged, and at a flagged position either float32 neighbour is accepted --
the whole group (or row) is re-quantized by the oracle with each choice and
the kernel's codes and scales must equal one of those results exactly.
Everywhere else the codes and scales must be identical.

Host-side test logic only (numpy); it holds none of the method's arithmetic
except through the oracle functions it is given.
"""
from __future__ import annotations

import itertools

import numpy as np

# float64 evaluations on both sides are within 2^-50 (relative) of each
# other; flag four times that distance
SILU_REL = 2.0 ** -48


def fp32_alternatives(v64: np.ndarray, rel: float):
    """For every float64 value: its float32 rounding, the float32 neighbour on
    the other side of the value, and whether the value lies within rel*|v| of
    the midpoint between the two."""
    v64 = np.asarray(v64, dtype=np.float64)
    y32 = v64.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        up = np.nextafter(y32, np.float32(np.inf))
        dn = np.nextafter(y32, np.float32(-np.inf))
        other = np.where(v64 > y32.astype(np.float64), up, dn)
        mid = (y32.astype(np.float64) + other.astype(np.float64)) / 2.0
        flag = np.abs(v64 - mid) <= rel * np.abs(v64)
    flag &= np.isfinite(y32) & np.isfinite(other)
    return y32, other, flag


def _mismatch(what, kind, where, got, want):
    raise AssertionError(f"{what}: {kind} differ from the oracle at {where}: got {got}, oracle {want}")


def assert_groups_match(q: np.ndarray, s: np.ndarray, y64: np.ndarray, quant_f32, what="",
                        rel: float = SILU_REL, max_flag_rate: float = 1e-5):
    """q, s: the kernel's codes [M, K] and scales [M, K/128] (float32 values);
    y64: the oracle's float64 values [M, K]; quant_f32(y32 [rows, K]) -> (q, s):
    the oracle's group rule on float32 values.  Returns the number of flagged
    positions."""
    M, K = y64.shape
    G = K // 128
    y32, other, flag = fp32_alternatives(y64, rel)
    nflag = int(flag.sum())
    assert nflag <= max(4, max_flag_rate * flag.size), (what, "too many near-midpoint values", nflag)
    rq, rs = quant_f32(y32)
    gflag = flag.reshape(M, G, 128).any(axis=2)
    code_ok = (q == rq).reshape(M, G, 128).all(axis=2)
    scale_ok = s == rs
    bad = ~(code_ok & scale_ok) & ~gflag
    if bad.any():
        m, g = np.argwhere(bad)[0]
        if not scale_ok[m, g]:
            _mismatch(what, "scales", (m, g), s[m, g], rs[m, g])
        j = np.argwhere(q[m, 128 * g:128 * g + 128] != rq[m, 128 * g:128 * g + 128])[0][0]
        _mismatch(what, "codes", (m, 128 * g + j), q[m, 128 * g + j], rq[m, 128 * g + j])
    for m, g in np.argwhere(gflag):
        lo, hi = 128 * g, 128 * g + 128
        pos = np.flatnonzero(flag[m, lo:hi])
        accepted = False
        for choice in itertools.product((False, True), repeat=len(pos)):
            yg = y32[m, lo:hi].copy()
            for p, take_other in zip(pos, choice):
                if take_other:
                    yg[p] = other[m, lo + p]
            cq, cs = quant_f32(yg.reshape(1, 128))
            if cs[0, 0] == s[m, g] and np.array_equal(cq[0], q[m, lo:hi]):
                accepted = True
                break
        if not accepted:
            raise AssertionError(f"{what}: group {(m, g)} with near-midpoint values at {list(pos)} matches "
                                 "no rounding of them")
    return nflag


def rms_rel(H: int) -> float:
    """Flag distance for RMSNorm's 1/rms: the kernel and the oracle add the
    same exact float64 squares in different orders (each sum within
    (H - 1) 2^-53 of the exact one, relative), then take the same float64
    steps; twice that bound plus the steps' roundings, doubled."""
    return 2.0 * (2 * H + 8) * 2.0 ** -53


def assert_rms_rows_match(q: np.ndarray, s: np.ndarray, r64: np.ndarray, apply_rows, what=""):
    """q, s: the kernel's codes and scales; r64: the oracle's float64 1/rms per
    row; apply_rows(rows, r32) -> (q, s) of those rows with the given float32
    1/rms.  Rows whose r64 lies next to a float32 midpoint accept either
    rounding of it.  Returns the number of flagged rows."""
    M, H = q.shape
    r32, other, flag = fp32_alternatives(r64, rms_rel(H))
    rows = np.arange(M)
    rq, rs = apply_rows(rows, r32)
    row_ok = (q == rq).all(axis=1) & (s == rs).all(axis=1)
    bad = ~row_ok & ~flag
    if bad.any():
        m = int(np.argwhere(bad)[0][0])
        if not np.array_equal(s[m], rs[m]):
            g = int(np.argwhere(s[m] != rs[m])[0][0])
            _mismatch(what, "scales", (m, g), s[m, g], rs[m, g])
        j = int(np.argwhere(q[m] != rq[m])[0][0])
        _mismatch(what, "codes", (m, j), q[m, j], rq[m, j])
    fl = np.flatnonzero(flag & ~row_ok)
    if fl.size:
        aq, as_ = apply_rows(fl, other[fl])
        ok = (q[fl] == aq).all(axis=1) & (s[fl] == as_).all(axis=1)
        if not ok.all():
            raise AssertionError(f"{what}: row {int(fl[~ok][0])} (1/rms next to a float32 midpoint) matches "
                                 "neither rounding")
    return int(flag.sum())
