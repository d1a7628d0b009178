"""CPU checks of the near-midpoint comparison used by the fused-producer
parity tests (tests/near_midpoint.py): it must flag exactly the float64
values next to a float32 rounding midpoint, accept the oracle's own result,
accept the other rounding at a flagged position only, and reject a changed
code or scale anywhere else (mistakes planted in the oracle's output)."""
import numpy as np
import pytest

import oracle
from fp8_blockwise_quantized_token_amd import synth

from near_midpoint import (SILU_REL, assert_groups_match, assert_rms_rows_match, fp32_alternatives,
                           rms_rel)


def test_flags_exactly_the_values_next_to_a_midpoint():
    a = np.array([1.0, 3.0, 1e-40, -7.5, 2.0 ** -140], np.float32)
    b = np.nextafter(a, np.float32(np.inf))
    mid = (a.astype(np.float64) + b.astype(np.float64)) / 2
    y32, other, flag = fp32_alternatives(mid, SILU_REL)
    assert flag.all()
    assert np.all((y32 == a) | (y32 == b)) and np.all(np.sort([y32, other], axis=0) == np.sort([a, b], axis=0))
    # on a float32 value, or a relative 2^-40 away from the midpoint: not flagged at 2^-48
    _, _, f2 = fp32_alternatives(a.astype(np.float64), SILU_REL)
    assert not f2.any()
    off = mid * (1 + 2.0 ** -40)
    _, _, f3 = fp32_alternatives(off, SILU_REL)
    assert not f3.any()
    _, _, f4 = fp32_alternatives(off, 2.0 ** -38)
    assert f4.all()
    # zeros and signed zeros are never flagged
    _, _, f5 = fp32_alternatives(np.array([0.0, -0.0]), SILU_REL)
    assert not f5.any()


def _silu_case(M=6, I=384, seed=3):
    x = synth.activations_bf16(synth.Case("sweep", "nm", M, 128, 2 * I, "normal_outlier", False, seed))
    return x, oracle.silu_and_mul_values(x)


def test_oracle_result_is_accepted_and_planted_changes_rejected():
    x, y64 = _silu_case()
    q, s = oracle.silu_and_mul_per_block_quant(x)
    assert assert_groups_match(q, s, y64, oracle.group_quant_f32, "self") == 0
    q2 = q.copy()
    q2[2, 200] ^= 1
    with pytest.raises(AssertionError, match="codes"):
        assert_groups_match(q2, s, y64, oracle.group_quant_f32, "planted code")
    s2 = s.copy()
    s2[4, 1] = np.nextafter(s2[4, 1], np.float32(np.inf))
    with pytest.raises(AssertionError, match="scales"):
        assert_groups_match(q, s2, y64, oracle.group_quant_f32, "planted scale")


def _on_midpoint(v):
    a = np.float32(v)
    b = np.nextafter(a, np.float32(np.inf) if a > 0 else np.float32(-np.inf))
    return (np.float64(a) + np.float64(b)) / 2


def test_other_rounding_accepted_only_at_a_flagged_position():
    x, y64 = _silu_case()
    q_ref, s_ref = oracle.group_quant_f32(y64.astype(np.float32))
    # a value whose other rounding changes its group's result: the group
    # maximum (through the scale) of some group
    found = None
    for m in range(y64.shape[0]):
        for g0 in range(0, y64.shape[1], 128):
            j = g0 + int(np.argmax(np.abs(y64[m, g0:g0 + 128])))
            t = y64.copy()
            t[m, j] = _on_midpoint(y64[m, j])
            y32, other, flag = fp32_alternatives(t, SILU_REL)
            alt = y32.copy()
            # the rounding of the midpoint that is not the original value's
            alt[m, j] = other[m, j] if y32[m, j] == np.float32(y64[m, j]) else y32[m, j]
            y32 = y32.copy()
            y32[m, j] = np.float32(y64[m, j])
            qa, sa = oracle.group_quant_f32(alt)
            qn, sn = oracle.group_quant_f32(y32)  # the original rounding
            if not (np.array_equal(qa, qn) and np.array_equal(sa, sn)):
                found = (m, j, t, qa, sa, qn, sn, flag)
                break
        if found:
            break
    assert found, "no group whose maximum changes the result"
    m, j, t, qa, sa, qn, sn, flag = found
    assert flag[m, j] and flag.sum() == 1
    # both roundings of the flagged value are accepted
    assert assert_groups_match(qn, sn, t, oracle.group_quant_f32, "near") == 1
    assert assert_groups_match(qa, sa, t, oracle.group_quant_f32, "other") == 1
    # the same result is refused when the value is not next to a midpoint
    with pytest.raises(AssertionError):
        assert_groups_match(qa, sa, y64, oracle.group_quant_f32, "unflagged")


def test_rms_rows_accept_either_rounding_only_when_flagged():
    M, H = 8, 512
    x = synth.activations_bf16(synth.Case("sweep", "nm", M, 128, H, "normal_outlier", False, 9))
    w = synth.norm_weight_f32(H)
    r64 = oracle.rms_norm_inv_rms(x)

    def apply_rows(rows, r32):
        return oracle.rms_norm_apply(x[rows], w, r32)

    q, s = oracle.rms_norm_per_block_quant(x, w)
    assert assert_rms_rows_match(q, s, r64, apply_rows, "self") == 0
    # the other float32 rounding of row 3's 1/rms: rejected unless flagged
    r32, other, _ = fp32_alternatives(r64, rms_rel(H))
    r_alt = r32.copy()
    r_alt[3] = other[3]
    qa, sa = oracle.rms_norm_apply(x, w, r_alt)
    if not (np.array_equal(qa, q) and np.array_equal(sa, s)):
        with pytest.raises(AssertionError):
            assert_rms_rows_match(qa, sa, r64, apply_rows, "unflagged row")
    # put row 3's 1/rms on a midpoint: then both roundings pass
    r64b = r64.copy()
    r64b[3] = (np.float64(r32[3]) + np.float64(other[3])) / 2
    assert assert_rms_rows_match(qa, sa, r64b, apply_rows, "flagged row") == 1
    assert assert_rms_rows_match(q, s, r64b, apply_rows, "flagged row, oracle side") == 1


def test_oracle_values_round_to_the_oracle_producer_outputs():
    # the float64 values the comparison starts from are the oracle's own:
    # rounded to float32 and group-quantized they give its producer outputs
    x, y64 = _silu_case(M=5, I=256, seed=4)
    q, s = oracle.group_quant_f32(y64.astype(np.float32))
    rq, rs = oracle.silu_and_mul_per_block_quant(x)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    M, H = 5, 640
    xr = synth.activations_bf16(synth.Case("sweep", "nm", M, 128, H, "normal", False, 5))
    w = synth.norm_weight_f32(H)
    q, s = oracle.rms_norm_apply(xr, w, oracle.rms_norm_inv_rms(xr).astype(np.float32))
    rq, rs = oracle.rms_norm_per_block_quant(xr, w)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
