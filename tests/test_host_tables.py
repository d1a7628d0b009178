"""The SiLU-and-mul producer's sigmoid table (csrc/sigmoid_table.inc): it is
what its generator writes, and its entries agree with scipy's logistic
function (float64, rounded to fp32) to within one fp32 ulp, with the edge
entries exact.  A CPU check of data the kernel reads; the kernel's results
are compared with the oracle in the GPU tests."""
import os
import re
import subprocess
import sys

import numpy as np
import scipy.special

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "fp8_blockwise_quantized_token_amd", "csrc")


def _table():
    text = open(os.path.join(CSRC, "sigmoid_table.inc")).read()
    body = text[text.index("{"):]
    vals = np.array([float.fromhex(v) for v in re.findall(r"(-?0x[0-9a-f.]+p[-+]?\d+)f", body)])
    span = int(re.search(r"kSigmoidSpan = (\d+);", text).group(1))
    base = int(re.search(r"kSigmoidBase = \((\d+) << 7\) - 1;", text).group(1))
    return vals.astype(np.float32), span, base


def test_table_is_what_the_generator_writes():
    r = subprocess.run([sys.executable, os.path.join(CSRC, "gen_sigmoid_table.py"), "--check"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_table_against_scipy_expit():
    vals, span, e_lo = _table()
    assert vals.size == 2 * span and span == 4098 and e_lo == 102
    for sign in (0, 1):
        half = vals[sign * span:(sign + 1) * span]
        assert half[0] == 0.5
        assert half[-1] == (0.0 if sign else 1.0)
        bits = np.arange(e_lo << 7, (e_lo << 7) + span - 2, dtype=np.uint32) | np.uint32(sign << 15)
        g = (bits << 16).view(np.float32).astype(np.float64)
        ref = scipy.special.expit(g).astype(np.float32)
        got = half[1:-1]
        d = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert d.max() <= 1 and np.mean(d == 0) > 0.99


def test_table_edges_follow_from_the_bounds():
    # below 2^-25 the logistic function rounds to 0.5 from either side; at
    # and above 128 it rounds to 1 (g > 0) or 0 (g < 0)
    for g in (2.0 ** -26, -(2.0 ** -26), 2.0 ** -40, -(2.0 ** -100)):
        assert np.float32(scipy.special.expit(g)) == np.float32(0.5)
    assert np.float32(scipy.special.expit(128.0)) == 1.0
    assert np.float32(scipy.special.expit(-128.0)) == 0.0
