"""Pins of the oracle's fp64 blockwise-scaled GEMM (CPU only).

Pinned against: numpy's float64 matmul over operands decoded by torch's
float8_e4m3fn conversion (an independent decode), an identity weight, a
closed form, integer-exact inputs, exact power-of-two scaling, and the row
subset path against the full product.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_blockwise_quantized_token_amd import synth

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _torch_dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _reference(qa, sa, qw, sw):
    M, K = qa.shape
    N = qw.shape[0]
    a = _torch_dec(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    w = _torch_dec(qw) * np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)
    return a @ w.T


def test_brute_force_all_codes_4x128x128():
    rng = synth.generator(10)
    qa = rng.permutation(np.resize(FINITE, 4 * 128)).reshape(4, 128).astype(np.uint8)
    qw = rng.permutation(np.resize(FINITE, 128 * 128)).reshape(128, 128).astype(np.uint8)
    # every finite code appears in both operands
    assert set(np.unique(qa)) == set(FINITE) and set(np.unique(qw)) == set(FINITE)
    sa = rng.uniform(0.01, 4, (4, 1)).astype(np.float32)
    sw = rng.uniform(0.01, 4, (1, 1)).astype(np.float32)
    y = oracle.block_gemm(qa, sa, qw, sw)
    ref = _reference(qa, sa, qw, sw)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())


def test_scale_indexing_multi_block():
    """Distinct scales per (m, kb) and (nb, kb): a transposed or shifted index fails."""
    rng = synth.generator(11)
    M, N, K = 4, 256, 512
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    qw = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-6, 6, size=(M, K // 128)) * rng.uniform(1, 2, (M, K // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-6, 6, size=(N // 128, K // 128)) * rng.uniform(1, 2, (N // 128, K // 128))).astype(np.float32)
    y = oracle.block_gemm(qa, sa, qw, sw)
    ref = _reference(qa, sa, qw, sw)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    # the same product with the weight scale grid transposed is different
    bad = _reference(qa, sa, qw, sw[::-1, ::-1].copy())
    assert not np.allclose(y, bad, rtol=1e-3)


def test_identity_weight():
    rng = synth.generator(12)
    M, K = 8, 256
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-4, 4, size=(M, K // 128))).astype(np.float32)
    qw = np.zeros((K, K), dtype=np.uint8)
    qw[np.arange(K), np.arange(K)] = 0x38  # 1.0 on the diagonal
    sw = np.ones((K // 128, K // 128), dtype=np.float32)
    y = oracle.block_gemm(qa, sa, qw, sw)
    exp = oracle.e4m3_decode(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    assert np.array_equal(y, exp)


def test_closed_form_geometric_scales():
    M, N, K = 3, 128, 512
    qa = np.full((M, K), 0x38, dtype=np.uint8)
    qw = np.full((N, K), 0x38, dtype=np.uint8)
    sa = np.tile((2.0 ** np.arange(K // 128)).astype(np.float32), (M, 1))
    sw = np.ones((1, K // 128), dtype=np.float32)
    y = oracle.block_gemm(qa, sa, qw, sw)
    assert np.all(y == 128 * (2.0 ** (K // 128) - 1)) and y[0, 0] == 1920.0


def test_integer_exact():
    rng = synth.generator(13)
    ints = {0x38: 1, 0x40: 2, 0x44: 3, 0x48: 4, 0xB8: -1, 0xC0: -2, 0x00: 0}
    codes = np.array(list(ints), dtype=np.uint8)
    M, N, K = 16, 256, 384
    qa = rng.choice(codes, size=(M, K)).astype(np.uint8)
    qw = rng.choice(codes, size=(N, K)).astype(np.uint8)
    ia = np.vectorize(ints.get)(qa).astype(np.int64)
    iw = np.vectorize(ints.get)(qw).astype(np.int64)
    y = oracle.block_gemm(qa, np.ones((M, 3), np.float32), qw, np.ones((2, 3), np.float32))
    assert np.array_equal(y, (ia @ iw.T).astype(np.float64))


def test_power_of_two_scaling_is_exact():
    rng = synth.generator(14)
    M, N, K = 5, 128, 256
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    qw = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.1, 1, (M, 2)).astype(np.float32)
    sw = rng.uniform(0.1, 1, (1, 2)).astype(np.float32)
    y1 = oracle.block_gemm(qa, sa, qw, sw)
    y2 = oracle.block_gemm(qa, sa * np.float32(2), qw, sw)
    assert np.array_equal(y2, 2 * y1)


def test_row_subset_and_threads():
    rng = synth.generator(15)
    M, N, K = 33, 256, 256
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    qw = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.1, 1, (M, 2)).astype(np.float32)
    sw = rng.uniform(0.1, 1, (2, 2)).astype(np.float32)
    full = oracle.block_gemm(qa, sa, qw, sw, nthreads=1)
    rows = np.array([32, 0, 7, 7, 31])
    sub = oracle.block_gemm(qa, sa, qw, sw, rows=rows, nthreads=3)
    assert np.array_equal(sub, full[rows])
    assert np.array_equal(oracle.block_gemm(qa, sa, qw, sw, nthreads=8), full)
