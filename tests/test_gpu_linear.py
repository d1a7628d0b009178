"""GPU parity of fp8_linear, the whole layer in one call (activation
quantization fused into the Swap-AB GEMM; quantizer + GEMM otherwise).

fp8_linear must equal fp8_group_quant followed by fp8_block_gemm with the
same configuration bit for bit: the fused quantizer produces the same codes
and scales and the GEMM sums them in the same order.  Against the CPU oracle
(oracle group quantization, then the fp64 oracle GEMM) the bar is the GEMM's:
|y - y_ref| <= 1e-2 |y_ref| + 1e-3 max|y_ref|.
"""
import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
import oracle
from fp8_blockwise_quantized_token_amd import synth

from gpu_common import assert_close, dev, host, oracle_weight, sample_rows, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _x(M, K, dist="normal_outlier", key=0):
    return synth.activations_bf16(synth.Case("decode_8b", f"x{key}", M, 128, K, dist, False, 100 + key))


def _swap_configs(M, K):
    kb = K // 128
    out = []
    for tm in (16, 32, 64):
        if M > tm:
            continue
        for tn in (16, 32, 64):
            if tn == 64 and tm == 64:
                continue
            for kw in (1, 2, 8):
                for sk in (1, 3):
                    if sk * kw <= 2 * kb and sk <= kb:
                        out.append(fb.make_config(fb.SWAPAB, tm, tn, sk, kw))
    return out


def _two_paths(xd, qw, sw, cfg, ue8m0=False):
    """(fp8_linear, fp8_group_quant + fp8_block_gemm) outputs as float64."""
    say("linear", tuple(xd.shape), tuple(qw.shape), cfg.as_dict() if cfg is not None else "dispatch",
        "ue8m0" if ue8m0 else "")
    y1 = fb.linear(xd, qw, sw, ue8m0=ue8m0, cfg=cfg)
    qa, sa = fb.quantize_activations(xd, ue8m0=ue8m0)
    y2 = fb.block_gemm(qa, sa, qw, sw, cfg)
    return host(y1).astype(np.float64), host(y2).astype(np.float64)


SMALL = [(1, 256, 512), (5, 384, 1152), (16, 640, 384), (17, 256, 256), (33, 512, 640),
         (64, 384, 1024), (100, 256, 512), (300, 768, 896)]


@pytest.mark.parametrize("M,N,K", SMALL, ids=lambda v: str(v))
def test_every_config_equals_separate_quant_and_gemm(M, N, K):
    x = _x(M, K, key=M)
    qw, sw = oracle_weight(N, K, False)
    qa_ref, sa_ref = oracle.group_quant(x)
    ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
    xd, qwd, swd = to_dev_bf16(x), to_dev(qw), to_dev(sw)
    cfgs = _swap_configs(M, K) + [fb.make_config(fb.STANDARD, 64, 128, 1),
                                  fb.make_config(fb.STANDARD, 128, 128, 2),
                                  fb.make_config(fb.STANDARD, 64, 64, 1, 2, 3), None]
    for cfg in cfgs:
        y1, y2 = _two_paths(xd, qwd, swd, cfg)
        assert np.array_equal(y1, y2), f"{cfg}: fused differs from quant + GEMM"
        assert_close(y1, ref, str(cfg))


def test_ue8m0_and_distributions():
    N, K = 512, 768
    qw, sw = oracle_weight(N, K, True)
    for M in (3, 12, 24, 40):  # lean fused, full fused (1, 2 and 4 token tiles; tile_n 32 at M = 40: separate)
        tm = 16 if M <= 16 else (32 if M <= 32 else 64)
        for dist in ("normal", "normal_outlier", "student_t3"):
            x = _x(M, K, dist, key=3)
            qa_ref, sa_ref = oracle.group_quant(x, ue8m0=True)
            ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
            for cfg in (fb.make_config(fb.SWAPAB, tm, 16, 1, 2), fb.make_config(fb.SWAPAB, tm, 32, 2, 1)):
                y1, y2 = _two_paths(to_dev_bf16(x), to_dev(qw), to_dev(sw), cfg, ue8m0=True)
                assert np.array_equal(y1, y2), f"M={M} {dist} {cfg}"
                assert_close(y1, ref, f"M={M} {dist} {cfg}")


def test_degenerate_groups():
    """All-zero groups (scale = eps / 448), one huge value per group (the
    rest flush to zero), signed zeros, values at the bf16 extremes."""
    M, N, K = 16, 256, 512
    x = _x(M, K, key=9).copy()
    x[0] = 0                          # all-zero row
    x[1, :128] = 0x8000               # -0.0 group
    x[2, 128:256] = 0
    x[2, 200] = np.float32(3.0e38).view(np.uint32) >> 16  # one huge value
    x[3] = np.float32(1e-30).view(np.uint32) >> 16         # tiny everywhere
    x[4] = 0                          # largest finite bf16 magnitudes in one group
    x[4, 0:128:2] = 0x7F7F            # (one group only, so that y stays finite)
    x[4, 1:128:2] = 0xFF7F
    qw, sw = oracle_weight(N, K, False)
    qa_ref, sa_ref = oracle.group_quant(x)
    ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
    for cfg in (fb.make_config(fb.SWAPAB, 16, 16, 1, 4), fb.make_config(fb.SWAPAB, 16, 64, 2, 2)):
        y1, y2 = _two_paths(to_dev_bf16(x), to_dev(qw), to_dev(sw), cfg)
        assert np.array_equal(y1, y2), str(cfg)
        assert_close(y1, ref, str(cfg))
        assert np.all(y1[0] == 0)


def test_strided_input_and_output():
    """x with a row pitch wider than K and y with a pitch wider than N: the
    padding is neither read into the result nor written."""
    import torch
    M, N, K = 9, 384, 640
    x = _x(M, K, key=11)
    qw, sw = oracle_weight(N, K, False)
    xbig = np.full((M, K + 64), 0x7F7F, np.uint16)  # padding is huge: would wreck the scales
    xbig[:, :K] = x
    xd = to_dev_bf16(xbig)[:, :K]
    ybig = torch.full((M, N + 128), 7.0, dtype=torch.bfloat16, device=dev())
    y = ybig[:, :N]
    qa_ref, sa_ref = oracle.group_quant(x)
    ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
    for cfg in (fb.make_config(fb.SWAPAB, 16, 32, 1, 2), fb.make_config(fb.STANDARD, 64, 128, 1)):
        say("linear strided", cfg.as_dict())
        ws = fb.linear_workspace(M, N, K, cfg, dev())
        fb.fp8_linear(xd, to_dev(qw), to_dev(sw), y, cfg=cfg, workspace=ws)
        yb = host(ybig)
        assert_close(yb[:, :N].astype(np.float64), ref, str(cfg))
        assert np.all(yb[:, N:] == 7.0)


def test_empty_m_is_a_noop():
    import torch
    qw, sw = oracle_weight(256, 256, False)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev())
    y = torch.empty((0, 256), dtype=torch.bfloat16, device=dev())
    fb.fp8_linear(x, to_dev(qw), to_dev(sw), y)
    torch.cuda.synchronize()


DECODE = [c for c in synth.cases("decode_8b")] + [c for c in synth.cases("sweep") if c.M in (2, 16)]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: c.cid)
def test_full_size_decode_dispatched(case):
    """Decode-size layers in the dispatched configuration (fused for Swap-AB),
    against the separate path bitwise and the oracle on sampled rows."""
    x = synth.activations_bf16(case)
    qw, sw = oracle_weight(case.N, case.K, case.ue8m0)
    y1, y2 = _two_paths(to_dev_bf16(x), to_dev(qw), to_dev(sw), None, case.ue8m0)
    assert np.array_equal(y1, y2), case.cid
    rows = sample_rows(case.M, 8)
    qa_ref, sa_ref = oracle.group_quant(x[rows], ue8m0=case.ue8m0)
    ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
    assert_close(y1[rows], ref, case.cid)


def test_graph_replay_of_fused_linear():
    import torch
    case = synth.Case("decode_8b", "x", 8, 24576, 4096, "normal_outlier", False, 0)
    x = to_dev_bf16(synth.activations_bf16(case))
    qw, sw = oracle_weight(24576, 4096, False)
    qw, sw = to_dev(qw), to_dev(sw)
    cfg = fb.make_config(fb.SWAPAB, 16, 32, 2, 4)
    y = torch.empty((8, 24576), dtype=torch.bfloat16, device=dev())
    ws = fb.linear_workspace(8, 24576, 4096, cfg, dev())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fb.fp8_linear(x, qw, sw, y, cfg=cfg, workspace=ws, stream=s)
    s.synchronize()
    eager = host(y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fb.fp8_linear(x, qw, sw, y, cfg=cfg, workspace=ws, stream=s)
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        say("linear graph replay", i)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), eager), f"replay {i}"


@pytest.mark.parametrize("M,N,K", [(96, 1024, 1024), (640, 2048, 1536), (4096, 5120, 2048)])
def test_ue8m0_activations_with_fp32_weight_scales(M, N, K):
    """Power-of-two activation scales with arbitrary fp32 weight scales: the
    dispatched Standard configuration must keep the fp32 scale mode (only the
    caller's FP8BLK_FLAG_WEIGHT_POW2 allows the power-of-two mode), and the
    result must match the oracle.  A power-of-two configuration with the
    UE8M0 flag alone is refused."""
    import torch
    x = _x(M, K, "normal_outlier", key=M % 7)
    qw, sw = oracle_weight(N, K, False)
    assert np.any(sw != pow2_floor(sw)), "weight scales must not all be powers of two here"
    cfg = fb.fp8_block_gemm_select(M, N, K, fb.FLAG_UE8M0)
    assert cfg.variant == fb.STANDARD and cfg.scale_mode == fb.SCALES_FP32, cfg
    say("ue8m0 activations, fp32 weight scales", M, N, K, cfg.as_dict())
    y = fb.linear(to_dev_bf16(x), to_dev(qw), to_dev(sw), ue8m0=True)
    torch.cuda.synchronize()
    rows = sample_rows(M, 16, key=M)
    qa_ref, sa_ref = oracle.group_quant(x[rows], ue8m0=True)
    ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
    assert_close(host(y)[rows].astype(np.float64), ref, "ue8m0 x fp32 weights")
    p2 = fb.fp8_block_gemm_select(M, N, K, fb.FLAG_UE8M0 | fb.FLAG_WEIGHT_POW2)
    assert p2.scale_mode == fb.SCALES_POW2
    with pytest.raises(fb.Fp8BlkError) as e:
        fb.linear(to_dev_bf16(x), to_dev(qw), to_dev(sw), ue8m0=True, cfg=p2)
    assert e.value.status == -6


def pow2_floor(s):
    return (s.view(np.uint32) & np.uint32(0x7F800000)).view(np.float32)
