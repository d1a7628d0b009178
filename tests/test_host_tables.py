"""The SiLU-and-mul producer's logistic table (csrc/sigmoid_table.inc): it is
what its generator writes, its entries agree with scipy's float64 logistic
function to within one float64 ulp (mostly exactly), and the two edge
entries follow from bounds checked here.  A CPU check of data the kernel
reads; the kernel's results are compared with the oracle in the GPU tests."""
import math
import os
import re
import subprocess
import sys

import mpmath
import numpy as np
import scipy.special

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "fp8_blockwise_quantized_token_amd", "csrc")


def _table():
    text = open(os.path.join(CSRC, "sigmoid_table.inc")).read()
    body = text[text.index("{"):]
    vals = np.array([float.fromhex(v) for v in re.findall(r"(-?0x[0-9a-f.]+p[-+]?\d+)", body)])
    span = int(re.search(r"kSigmoidSpan = (\d+);", text).group(1))
    base = int(re.search(r"kSigmoidBase = \((\d+) << 7\) - 1;", text).group(1))
    return vals, span, base


def test_table_is_what_the_generator_writes():
    r = subprocess.run([sys.executable, os.path.join(CSRC, "gen_sigmoid_table.py"), "--check"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_table_against_scipy_expit():
    vals, span, e_lo = _table()
    assert vals.size == span == 7810 and e_lo == 74
    bits = np.arange(e_lo << 7, (e_lo << 7) + span - 2, dtype=np.uint32)
    a = (bits << 16).view(np.float32).astype(np.float64)
    got = vals[1:-1]
    # scipy's float64 expit rounds several times (within 2 ulp)
    ref = scipy.special.expit(-a)
    d = np.abs(got.view(np.int64) - ref.view(np.int64))
    assert d.max() <= 2 and np.mean(d == 0) > 0.6
    # the same formula in x87 extended precision (11 more bits): its float64
    # rounding must equal the table wherever the extended value is not
    # within 2^-58 (relative) of a float64 rounding midpoint
    lx = np.longdouble(1) / (np.longdouble(1) + np.exp(a.astype(np.longdouble)))
    ld = lx.astype(np.float64)
    other = np.where(lx > ld.astype(np.longdouble), np.nextafter(ld, np.inf), np.nextafter(ld, -np.inf))
    mid = (ld.astype(np.longdouble) + other.astype(np.longdouble)) / 2
    near = np.abs(lx - mid) <= np.longdouble(2.0 ** -58) * lx
    d2 = np.abs(got.view(np.int64) - ld.view(np.int64))
    assert d2.max() <= 1 and np.all(d2[~near] == 0) and near.mean() < 0.05
    assert np.all(got > 0) and np.all(np.diff(got) <= 0)  # positive, non-increasing in |g|


def test_table_edges_follow_from_the_bounds():
    vals, span, e_lo = _table()
    mpmath.mp.prec = 200
    # every |g| below 2^-53 rounds to 0.5: the largest such bf16 value does,
    # and t is monotonic
    a = mpmath.mpf(255) * mpmath.mpf(2) ** (e_lo - 1 - 127 - 7)
    t = 1 / (1 + mpmath.exp(a))
    assert abs(t - mpmath.mpf(0.5)) < mpmath.mpf(2) ** -55  # closer to 0.5 than half the spacing below it
    assert vals[0] == 0.5
    # |g| >= 256: |g u t(|g|)| <= 256 e^-256 * (largest bf16) < 2^-150, so the
    # float32 result is a signed zero for the true t (|g| t(|g|) decreases for
    # |g| > 1) and for the table's 2^-1022 alike (the largest |g u| times it is
    # far below 2^-150); the entry is positive so that 0 - t < 0
    assert vals[-1] == 2.0 ** -1022
    largest_bf16 = float(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])
    assert 256 * math.exp(-256) * largest_bf16 < 2.0 ** -150
    assert largest_bf16 * largest_bf16 * 2.0 ** -1022 < 2.0 ** -150
    # the first tabled magnitude is 2^-53 itself
    assert (e_lo - 127) == -53
