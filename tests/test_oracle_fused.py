"""Pins of the fused-producer oracle functions rms_norm_per_block_quant and
silu_and_mul_per_block_quant (German page "Helion-Kernel in vLLM: PyTorch
FP8 ohne CUDA", section "Welche Kernel wurden in vLLM integriert"; RFC page
"[RFC]: Using Helion for Selected vLLM CustomOps", section "Motivation").

Each pin checks the oracle against something other than itself: special
inputs where RMSNorm or SiLU reduce to an exact value that then goes through
the already-pinned per-row quantizer (channel_quant on rows of 128, which is
the group quantizer of fp32 values), power-of-two invariances, closed forms,
and library routines (torch's rms_norm in float64, scipy's expit).
"""
import numpy as np
import scipy.special
import torch

import oracle
from fp8_blockwise_quantized_token_amd import synth

EPS = np.float32(1e-10)


def _bf16(a) -> np.ndarray:
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _val(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _group_quant_f32(y: np.ndarray, ue8m0=False):
    """The per-row quantizer applied to every 128-group of fp32 values."""
    M, H = y.shape
    q, s = oracle.channel_quant(y.reshape(-1, 128), ue8m0=ue8m0)
    return q.reshape(M, H), s.reshape(M, H // 128)


def _signs(shape, key):
    g = synth.generator(41, key)
    return np.where(g.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)


def _weight(H, key):
    # bf16-exact weights, so that x * w is exact in fp32 for x = +-2^k
    g = synth.generator(42, key)
    return _val(_bf16(1.0 + 0.5 * g.standard_normal(H).astype(np.float32)))


def _adjacent_or_equal(q1: np.ndarray, q2: np.ndarray) -> bool:
    same_sign = (q1 & 0x80) == (q2 & 0x80)
    d = np.abs((q1 & 0x7F).astype(np.int32) - (q2 & 0x7F).astype(np.int32))
    return bool(np.all(same_sign & (d <= 1)))


# ----------------------------------------------------------------- RMSNorm


def test_rms_unit_rows_reduce_to_the_group_quantizer_of_the_weight():
    # x = +-1 and eps_norm = 0: mean of squares 1, rms 1, y = +-w exactly
    M, H = 6, 640
    sg = _signs((M, H), 1)
    w = _weight(H, 1)
    for ue8m0 in (False, True):
        q, s = oracle.rms_norm_per_block_quant(_bf16(sg), w, eps_norm=0.0, ue8m0=ue8m0)
        q2, s2 = _group_quant_f32(sg * w[None, :], ue8m0)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_rms_eps_sits_under_the_square_root():
    # x = +-1, eps_norm = 3: rms = sqrt(1 + 3) = 2 and y = +-w / 2 exactly
    M, H = 4, 384
    sg = _signs((M, H), 2)
    w = _weight(H, 2)
    q, s = oracle.rms_norm_per_block_quant(_bf16(sg), w, eps_norm=3.0)
    q2, s2 = _group_quant_f32(sg * w[None, :] * np.float32(0.5))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_rms_divides_by_the_row_length():
    # a row with a single nonzero value v among H: mean of squares v^2 / H,
    # y = v * sqrt(H) / |v| = +-sqrt(H) there (H = 256 -> 16 exactly)
    H = 256
    for v in (3.0, -0.0078125, 96.0):
        x = np.zeros((1, H), np.float32)
        x[0, 200] = v
        q, s = oracle.rms_norm_per_block_quant(_bf16(x), np.ones(H, np.float32), eps_norm=0.0)
        assert s[0, 1] == np.float32(16.0) / np.float32(448.0)
        assert q[0, 200] == (0xFE if v < 0 else 0x7E)
        assert not np.any(np.delete(q[0], 200) & 0x7F)
        assert s[0, 0] == EPS / np.float32(448.0)


def test_rms_is_invariant_to_power_of_two_input_scaling():
    M, H = 5, 1024
    c = synth.Case("sweep", "rms", M, 128, H, "student_t3", False, 401)
    x = synth.activations_bf16(c)
    w = _weight(H, 3)
    q1, s1 = oracle.rms_norm_per_block_quant(x, w, eps_norm=0.0)
    x2 = _bf16(_val(x) * np.float32(32.0))
    q2, s2 = oracle.rms_norm_per_block_quant(x2, w, eps_norm=0.0)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_rms_weight_scales_each_group_exactly():
    # doubling the weight of group g doubles its scale and keeps its codes
    M, H = 3, 512
    c = synth.Case("sweep", "rms", M, 128, H, "normal", False, 402)
    x = synth.activations_bf16(c)
    w = _weight(H, 4)
    q1, s1 = oracle.rms_norm_per_block_quant(x, w)
    w2 = w.copy()
    w2[128:256] *= 2.0
    w2[384:512] *= 0.25
    q2, s2 = oracle.rms_norm_per_block_quant(x, w2)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2[:, 1], s1[:, 1] * 2) and np.array_equal(s2[:, 3], s1[:, 3] / 4)
    assert np.array_equal(s2[:, [0, 2]], s1[:, [0, 2]])


def test_rms_zero_row_and_constant_rows():
    H = 256
    q, s = oracle.rms_norm_per_block_quant(np.zeros((1, H), np.uint16), np.ones(H, np.float32))
    assert not q.any() and np.all(s == EPS / np.float32(448))
    # constant row c: y = c / sqrt(c^2 + eps) in every position -> code 0x7E
    for cval, eps_n in ((2.0 ** -10, 1e-6), (0.75, 1e-6), (-5.0, 1e-2)):
        x = np.full((1, H), _bf16(np.float32(cval)), np.uint16)
        q, s = oracle.rms_norm_per_block_quant(x, np.ones(H, np.float32), eps_norm=eps_n)
        y = abs(cval) / np.sqrt(cval * cval + np.float32(eps_n))
        assert np.all(q == (0xFE if cval < 0 else 0x7E))
        assert np.allclose(s, y / 448.0, rtol=2e-7, atol=0)


def test_rms_matches_torch_rms_norm_in_float64():
    M, H = 24, 2048
    c = synth.Case("sweep", "rms", M, 128, H, "normal_outlier", False, 403)
    x = synth.activations_bf16(c)
    w = synth.generator(43).standard_normal(H).astype(np.float32) * np.float32(0.3) + np.float32(1.0)
    for ue8m0 in (False, True):
        q, s = oracle.rms_norm_per_block_quant(x, w, eps_norm=1e-6, ue8m0=ue8m0)
        y = torch.nn.functional.rms_norm(torch.from_numpy(_val(x)).double(), (H,),
                                         torch.from_numpy(w).double(), eps=float(np.float32(1e-6)))
        q2, s2 = _group_quant_f32(y.float().numpy(), ue8m0)
        # the oracle rounds 1/rms to fp32 before two fp32 products: its y is
        # within ~1.5 ulp of the float64 one, so scales agree to a few ulp
        # and codes differ only next to a rounding midpoint
        assert np.allclose(s, s2, rtol=4 * 2.0 ** -23, atol=0)
        assert np.mean(s == s2) > 0.5
        assert np.mean(q != q2) < 1e-3 and _adjacent_or_equal(q, q2)


# ------------------------------------------------------------ SiLU and mul


def _gate_up(M, I, gate, up):
    x = np.empty((M, 2 * I), np.float32)
    x[:, :I] = gate
    x[:, I:] = up
    return _bf16(x)


def test_silu_of_large_gates_is_the_gate_itself():
    # g >= 32: 1 + exp(-g) rounds to 1 at fp32 precision of the product, so
    # y = g * u exactly (both bf16: the product has <= 16 significant bits)
    M, I = 4, 384
    gen = synth.generator(44)
    g = _val(_bf16(gen.uniform(32.0, 300.0, (M, I)).astype(np.float32)))
    u = _val(_bf16(gen.standard_normal((M, I)).astype(np.float32)))
    for ue8m0 in (False, True):
        q, s = oracle.silu_and_mul_per_block_quant(_gate_up(M, I, g, u), ue8m0=ue8m0)
        q2, s2 = _group_quant_f32(g * u, ue8m0)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_silu_gate_is_the_first_half():
    # swapping the halves must change the result (gate 64, up 1 vs gate 1, up 64)
    M, I = 1, 128
    a = oracle.silu_and_mul_per_block_quant(_gate_up(M, I, 64.0, 1.0))
    b = oracle.silu_and_mul_per_block_quant(_gate_up(M, I, 1.0, 64.0))
    assert a[1][0, 0] == np.float32(64.0) / np.float32(448.0)
    # silu(1) * 64 = 64 / (1 + e^-1)
    assert np.isclose(b[1][0, 0], 64.0 / (1.0 + np.exp(-1.0)) / 448.0, rtol=1e-7)


def test_silu_zero_and_very_negative_gates_give_signed_zero_codes():
    M, I = 2, 256
    gen = synth.generator(45)
    u = _val(_bf16(gen.standard_normal((M, I)).astype(np.float32)))
    for gval in (0.0, -80.0, -3.0e4):
        q, s = oracle.silu_and_mul_per_block_quant(_gate_up(M, I, gval, u))
        # silu(0) = +0 and silu(very negative) is a tiny negative: y has the
        # sign of gate-sign * u, far below the eps-guarded scale
        neg = (u < 0) if gval == 0.0 else (u > 0)
        assert np.all(s == EPS / np.float32(448))
        assert np.array_equal(q, np.where(neg, 0x80, 0x00).astype(np.uint8))


def test_silu_matches_scipy_expit():
    M, I = 16, 1024
    gen = synth.generator(46)
    g = _val(_bf16((2.0 * gen.standard_normal((M, I))).astype(np.float32)))
    u = _val(_bf16(gen.standard_normal((M, I)).astype(np.float32)))
    for ue8m0 in (False, True):
        q, s = oracle.silu_and_mul_per_block_quant(_gate_up(M, I, g, u), ue8m0=ue8m0)
        y = (g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u).astype(np.float32)
        q2, s2 = _group_quant_f32(y, ue8m0)
        assert np.allclose(s, s2, rtol=2 * 2.0 ** -23, atol=0)
        assert np.mean(q != q2) < 1e-4 and _adjacent_or_equal(q, q2)


def test_silu_odd_part_identity():
    # silu(g) - silu(-g) = g: for a group whose gates are +-g pairs with up = 1,
    # the dequantized sum over each pair is g within the quantization error
    I = 128
    gen = synth.generator(47)
    gpos = _val(_bf16(gen.uniform(0.1, 4.0, 64).astype(np.float32)))
    gate = np.concatenate([gpos, -gpos])[None, :]
    q, s = oracle.silu_and_mul_per_block_quant(_gate_up(1, I, gate, 1.0))
    d = oracle.e4m3_decode(q[0]) * s[0, 0]
    # each code is within half a step (2^-4 relative for normal codes) of the value
    assert np.allclose(d[:64] - d[64:], gpos, rtol=0, atol=2.0 ** -3 * np.abs(d).max())
