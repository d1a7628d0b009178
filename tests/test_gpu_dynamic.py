"""GPU parity of the FP8_Dynamic path (per-token activation scales,
per-channel weight scales, scaled_mm) against the CPU oracle.

Quantized bytes and scales must match the oracle bit for bit; the GEMM is
within |y - y_ref| <= 1e-2 |y_ref| + 1e-3 max|y_ref|, and every
configuration gives the same bits on integer-exact inputs.
"""
import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
import oracle
from fp8_blockwise_quantized_token_amd import synth

from gpu_common import assert_close, dev, host, sample_rows, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _x(M, K, dist="normal_outlier", key=0):
    return synth.activations_bf16(synth.Case("sweep", f"dyn{key}", M, 128, K, dist, False, 400 + key))


@pytest.mark.parametrize("M,K,dist", [(1, 4096, "normal_outlier"), (5, 128, "student_t3"),
                                      (64, 12288, "normal_outlier"), (300, 25600, "student_t3"),
                                      (2048, 4096, "normal"), (7, 32768, "student_t3")],
                         ids=lambda v: str(v))
def test_token_quant_bit_exact(M, K, dist):
    x = _x(M, K, dist, key=M)
    for ue8m0 in (False, True):
        say("token quant", M, K, dist, ue8m0)
        q, s = fb.quantize_tokens(to_dev_bf16(x), ue8m0=ue8m0)
        q_ref, s_ref = oracle.token_quant(x, ue8m0=ue8m0)
        assert np.array_equal(host(s), s_ref), "scales differ"
        assert np.array_equal(host(q), q_ref), "codes differ"


def test_token_quant_edges_and_strides():
    import torch
    M, K = 6, 1024
    x = _x(M, K, "student_t3", key=9).copy()
    x[0] = 0                                    # all-zero row: s = eps / 448
    x[1, 5] = np.float32(3.0e38).view(np.uint32) >> 16  # one huge value
    x[2] = 0x8000                               # -0.0 everywhere
    x[3] = np.float32(1e-30).view(np.uint32) >> 16
    big = np.full((M, K + 64), 0x7F7F, np.uint16)  # huge padding: must not be read
    big[:, :K] = x
    xd = to_dev_bf16(big)[:, :K]
    qbig = torch.full((M, K + 32), 0xAB, dtype=torch.uint8, device=dev())
    s = torch.empty((M,), dtype=torch.float32, device=dev())
    say("token quant strided")
    fb.fp8_token_quant(xd, qbig[:, :K], s)
    q_ref, s_ref = oracle.token_quant(x)
    qh = host(qbig)
    assert np.array_equal(qh[:, :K], q_ref) and np.array_equal(host(s), s_ref)
    assert np.all(qh[:, K:] == 0xAB)
    assert np.all(qh[2, :K] == 0x80)


@pytest.mark.parametrize("N,K", [(256, 512), (6144, 4096), (4096, 12288), (5120, 25600)])
def test_channel_quant_bit_exact(N, K):
    w = synth.weights_f32(N, K)
    for ue8m0 in (False, True):
        say("channel quant", N, K, ue8m0)
        q, s = fb.quantize_weight_channels(to_dev(w), ue8m0=ue8m0)
        q_ref, s_ref = oracle.channel_quant(w, ue8m0=ue8m0)
        assert np.array_equal(host(s), s_ref) and np.array_equal(host(q), q_ref)


def _configs(M, N, K):
    kb = K // 128
    out = []
    for tm, tn, ns in ((64, 64, 0), (64, 64, 3), (64, 128, 0), (64, 128, 4), (128, 128, 0), (128, 128, 3),
                       (256, 128, 0), (128, 256, 0), (256, 256, 0)):
        if N % tn:
            continue
        for sk in (1, 3):
            if sk <= kb:
                out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 1, ns))
    for tm, ns in ((64, 4), (128, 0)):  # twice the waves
        for sk in (1, 3):
            if sk <= kb:
                out.append(fb.make_config(fb.STANDARD, tm, 128, sk, 2, ns))
    for tm in (16, 32, 64):
        if M > tm:
            continue
        for tn in (16, 32, 64):
            if tn == 64 and tm == 64:
                continue
            for kw in (1, 4):
                for sk in (1, 2):
                    if sk * kw <= kb:
                        out.append(fb.make_config(fb.SWAPAB, tm, tn, sk, kw))
    return out


def _smm(qa, sa, qw, sw, cfg):
    say("scaled_mm", qa.shape, qw.shape, cfg.as_dict() if cfg is not None else "dispatch")
    return host(fb.scaled_mm(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), cfg)).astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (17, 384, 1152), (64, 256, 640), (300, 768, 896)],
                         ids=lambda v: str(v))
def test_scaled_mm_every_config_against_oracle(M, N, K):
    rng = synth.generator(900, M, N, K)
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    qw = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-8, 4, size=M) * rng.uniform(1, 2, M)).astype(np.float32)
    sw = (2.0 ** rng.integers(-8, 4, size=N) * rng.uniform(1, 2, N)).astype(np.float32)
    ref = oracle.scaled_mm(qa, sa, qw, sw)
    for cfg in _configs(M, N, K) + [None]:
        assert_close(_smm(qa, sa, qw, sw, cfg), ref, str(cfg))


def test_scaled_mm_integer_exact_and_identity():
    ints = {0x38: 1, 0x40: 2, 0x44: 3, 0x48: 4, 0xB8: -1, 0xC0: -2, 0x00: 0, 0x50: 8}
    codes = np.array(list(ints), dtype=np.uint8)
    rng = synth.generator(901)
    M, N, K = 64, 512, 1024
    qa = rng.choice(codes, size=(M, K)).astype(np.uint8)
    qw = rng.choice(codes, size=(N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-3, 4, size=M)).astype(np.float32)
    sw = (2.0 ** rng.integers(-3, 4, size=N)).astype(np.float32)
    ia = np.vectorize(ints.get)(qa).astype(np.int64)
    iw = np.vectorize(ints.get)(qw).astype(np.int64)
    exact = (ia @ iw.T).astype(np.float64) * sa[:, None] * sw[None, :]
    first = None
    for cfg in _configs(M, N, K):
        y = _smm(qa, sa, qw, sw, cfg)
        assert_close(y, exact, str(cfg))
        if first is None:
            first = y
        assert np.array_equal(y, first), str(cfg)
    # identity weight with per-channel scales: y = dec(a) sa sw exactly
    M, K = 48, 512
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    qw = np.zeros((K, K), np.uint8)
    qw[np.arange(K), np.arange(K)] = 0x38
    sa = (2.0 ** rng.integers(-4, 4, size=M)).astype(np.float32)
    sw = (2.0 ** (np.arange(K) % 8 - 4)).astype(np.float32)
    exp = oracle.e4m3_decode(qa) * sa[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    for cfg in _configs(M, K, K):
        assert np.array_equal(_smm(qa, sa, qw, sw, cfg), exp), str(cfg)


DYN_CASES = [c for c in synth.cases("decode_8b") if c.M in (1, 64)] + list(synth.cases("prefill_8b"))


@pytest.mark.parametrize("case", DYN_CASES, ids=lambda c: c.cid)
def test_full_size_dynamic_linear(case):
    """Token quantization (bit-exact) and scaled_mm in the dispatched
    configuration at full size, the GEMM against the oracle on sampled rows."""
    import torch
    x = synth.activations_bf16(case)
    w = synth.weights_f32(case.N, case.K)
    qw_ref, sw_ref = oracle.channel_quant(w)
    say("dynamic linear", case.cid, fb.fp8_block_gemm_select(case.M, case.N, case.K).as_dict())
    qa, sa = fb.quantize_tokens(to_dev_bf16(x))
    y = fb.scaled_mm(qa, sa, to_dev(qw_ref), to_dev(sw_ref))
    torch.cuda.synchronize()
    rows = sample_rows(case.M, 8)
    qa_ref, sa_ref = oracle.token_quant(x[rows])
    assert np.array_equal(host(qa)[rows], qa_ref) and np.array_equal(host(sa)[rows], sa_ref)
    ref = oracle.scaled_mm(qa_ref, sa_ref, qw_ref, sw_ref)
    assert_close(host(y)[rows].astype(np.float64), ref, case.cid)
