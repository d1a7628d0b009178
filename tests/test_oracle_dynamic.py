"""Pins of the FP8_Dynamic oracle functions (per-token activation scales,
per-channel weight scales, scaled_mm) against special cases that reduce to
the already-pinned group quantizer and block GEMM, closed forms and exact
identities."""
import numpy as np

import oracle
from fp8_blockwise_quantized_token_amd import synth

EPS = np.float32(1e-10)


def _bf16(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _x(M, K, key):
    c = synth.Case("sweep", "dyn", M, 128, K, "student_t3", False, 300 + key)
    return synth.activations_bf16(c)


def test_token_quant_equals_group_quant_when_the_row_is_one_group():
    x = _x(37, 128, 1)
    for ue8m0 in (False, True):
        q1, s1 = oracle.token_quant(x, ue8m0=ue8m0)
        q2, s2 = oracle.group_quant(x, ue8m0=ue8m0)
        assert np.array_equal(q1, q2)
        assert np.array_equal(s1, s2[:, 0])


def test_token_quant_equals_group_quant_when_groups_share_the_row_amax():
    # every 128-group of a row holds the row's amax: all group scales equal the
    # token scale, so the codes must be identical
    x = _x(9, 1024, 2).copy()
    big = _bf16(np.float32(37.5))
    x[:, ::128] = big
    q1, s1 = oracle.token_quant(x)
    q2, s2 = oracle.group_quant(x)
    assert np.all(s2 == s1[:, None])
    assert np.array_equal(q1, q2)


def test_token_quant_hand_worked_rows():
    K = 2048
    zero = np.zeros((1, K), np.uint16)
    q, s = oracle.token_quant(zero)
    assert s[0] == np.float32(EPS) / np.float32(448) and not q.any()
    row = np.full((1, K), _bf16(np.float32(1.0)), np.uint16)
    row[0, 1000] = _bf16(np.float32(448.0))
    q, s = oracle.token_quant(row)
    assert s[0] == np.float32(1.0)
    assert q[0, 1000] == 0x7E and np.all(np.delete(q[0], 1000) == 0x38)
    # the scale is IEEE fp32 amax / 448 over the whole row
    x = _x(5, 640, 3)
    _, s = oracle.token_quant(x)
    amax = np.abs((x.astype(np.uint32) << 16).view(np.float32)).max(axis=1)
    assert np.array_equal(s, (np.maximum(amax, EPS) / np.float32(448)).astype(np.float32))


def test_channel_quant_equals_block_quant_when_each_row_is_a_block_row():
    # one 128x128 block whose 128 rows have equal amax: block scale = channel scale
    rng = synth.generator(301)
    w = rng.uniform(-0.5, 0.5, size=(128, 128)).astype(np.float32)
    w[:, 7] = 0.75
    q1, s1 = oracle.channel_quant(w)
    q2, s2 = oracle.weight_block_quant(w)
    assert np.all(s1 == s2[0, 0]) and np.array_equal(q1, q2)


def test_scaled_mm_equals_block_gemm_for_constant_scales_along_k():
    rng = synth.generator(302)
    M, N, K = 6, 256, 384
    qa = rng.integers(0, 0x7E, size=(M, K), dtype=np.uint8)
    qw = rng.integers(0x80, 0xFE, size=(N, K), dtype=np.uint8)
    sa = (2.0 ** rng.integers(-4, 4, size=M) * rng.uniform(1, 2, M)).astype(np.float32)
    swb = (2.0 ** rng.integers(-4, 4, size=N // 128) * rng.uniform(1, 2, N // 128)).astype(np.float32)
    sw = np.repeat(swb, 128)
    y1 = oracle.scaled_mm(qa, sa, qw, sw)
    y2 = oracle.block_gemm(qa, np.repeat(sa[:, None], K // 128, axis=1), qw,
                           np.repeat(swb[:, None], K // 128, axis=1))
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-12 * np.abs(y2).max())


def test_scaled_mm_identity_weight_pins_per_channel_scales():
    rng = synth.generator(303)
    M, K = 12, 256
    qa = rng.integers(0, 0x7E, size=(M, K), dtype=np.uint8)
    qw = np.zeros((K, K), np.uint8)
    qw[np.arange(K), np.arange(K)] = 0x38
    sa = (2.0 ** rng.integers(-3, 3, size=M)).astype(np.float32)
    sw = (2.0 ** (np.arange(K) % 8)).astype(np.float32)
    y = oracle.scaled_mm(qa, sa, qw, sw)
    exp = oracle.e4m3_decode(qa) * sa[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    assert np.array_equal(y, exp)


def test_scaled_mm_closed_form_and_row_subset():
    M, N, K = 8, 24, 640
    qa = np.full((M, K), 0x38, np.uint8)
    qw = np.full((N, K), 0x38, np.uint8)
    sa = (2.0 ** (np.arange(M) % 4)).astype(np.float32)
    sw = (2.0 ** (np.arange(N) % 3)).astype(np.float32)
    y = oracle.scaled_mm(qa, sa, qw, sw)
    exp = K * np.outer(2.0 ** (np.arange(M) % 4), 2.0 ** (np.arange(N) % 3))
    assert np.array_equal(y, exp)
    rows = np.array([7, 0, 3])
    assert np.array_equal(oracle.scaled_mm(qa, sa, qw, sw, rows=rows), exp[rows])
