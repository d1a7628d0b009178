"""GPU parity of the blockwise-scaled FP8 GEMM against the fp64 CPU oracle.

Bar: |y - y_ref| <= 1e-2 |y_ref| + 1e-3 max|y_ref| for every compared output
(max over the compared outputs of the call), for every variant; Standard,
Split-K and Swap-AB agree bit for bit on integer-exact inputs.  GEMM inputs
are oracle-quantized bytes, so quantization error is not part of the check.
"""
import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
import oracle
from fp8_blockwise_quantized_token_amd import synth

from gpu_common import assert_close, dev, host, oracle_weight, sample_rows, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _configs(M, N, K):
    """Every compiled configuration valid for this shape."""
    kb = K // 128
    out = []
    for tm, tn in ((64, 64), (64, 128), (128, 128), (256, 128), (128, 256), (256, 256)):
        if N % tn:
            continue
        for sk in (1, 2, 3):
            if sk <= kb:
                out.append(fb.make_config(fb.STANDARD, tm, tn, sk))
    # deeper LDS pipelines (3 and 4 stages), with and without split-K
    for tm, tn, ns in ((64, 64, 3), (64, 64, 4), (64, 128, 3), (64, 128, 4), (128, 128, 3), (256, 128, 3)):
        if N % tn:
            continue
        for sk in (1, 3):
            if sk <= kb:
                out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 1, ns))
    # twice the waves (each 32 columns wide)
    for tm, tn, ns in ((64, 64, 0), (64, 64, 3), (64, 128, 0), (64, 128, 3), (64, 128, 4), (128, 128, 0),
                       (128, 128, 3)):
        for sk in (1, 2):
            if sk <= kb:
                out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 2, ns))
    for tm in (16, 32, 64):
        if M > tm:
            continue
        for tn in (16, 32, 64):
            if tn == 64 and tm == 64:
                continue
            for kw in (1, 2, 8):
                for sk in (1, 2):
                    if sk <= kb:
                        out.append(fb.make_config(fb.SWAPAB, tm, tn, sk, kw))
    return out


def _run(qa, sa, qw, sw, cfg):
    say("gemm", qa.shape, qw.shape, cfg.as_dict() if cfg is not None else "dispatch")
    y = fb.block_gemm(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), cfg)
    return host(y).astype(np.float64)


def _random_operands(M, N, K, key):
    rng = synth.generator(700, M, N, K, key)
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    qw = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-8, 4, size=(M, K // 128)) * rng.uniform(1, 2, (M, K // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-8, 4, size=(N // 128, K // 128)) * rng.uniform(1, 2, (N // 128, K // 128))).astype(np.float32)
    return qa, sa, qw, sw


SMALL = [(1, 256, 512), (5, 384, 1152), (16, 640, 384), (17, 256, 256), (33, 512, 640),
         (64, 384, 1024), (100, 256, 512), (257, 512, 384), (300, 768, 896)]


@pytest.mark.parametrize("M,N,K", SMALL, ids=lambda v: str(v))
def test_every_config_against_oracle(M, N, K):
    qa, sa, qw, sw = _random_operands(M, N, K, 1)
    ref = oracle.block_gemm(qa, sa, qw, sw)
    for cfg in _configs(M, N, K) + [None]:
        y = _run(qa, sa, qw, sw, cfg)
        assert_close(y, ref, str(cfg))


def test_identity_weight_pins_orientation():
    M, K = 48, 512
    rng = synth.generator(701)
    qa = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-4, 4, size=(M, K // 128))).astype(np.float32)
    qw = np.zeros((K, K), dtype=np.uint8)
    qw[np.arange(K), np.arange(K)] = 0x38
    sw = np.ones((K // 128, K // 128), dtype=np.float32)
    exp = oracle.e4m3_decode(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    for cfg in _configs(M, K, K):
        y = _run(qa, sa, qw, sw, cfg)
        assert np.array_equal(y, exp), str(cfg)


def test_closed_form_geometric_scales():
    M, N, K = 20, 256, 512
    qa = np.full((M, K), 0x38, np.uint8)
    qw = np.full((N, K), 0x38, np.uint8)
    sa = np.tile((2.0 ** np.arange(K // 128)).astype(np.float32), (M, 1))
    sw = np.ones((N // 128, K // 128), np.float32)
    for cfg in _configs(M, N, K):
        y = _run(qa, sa, qw, sw, cfg)
        assert np.all(y == 1920.0), str(cfg)


def test_integer_exact_variants_bitwise_equal():
    ints = {0x38: 1, 0x40: 2, 0x44: 3, 0x48: 4, 0xB8: -1, 0xC0: -2, 0x00: 0, 0x50: 8}
    codes = np.array(list(ints), dtype=np.uint8)
    rng = synth.generator(702)
    M, N, K = 64, 512, 1024
    qa = rng.choice(codes, size=(M, K)).astype(np.uint8)
    qw = rng.choice(codes, size=(N, K)).astype(np.uint8)
    ia = np.vectorize(ints.get)(qa).astype(np.int64)
    iw = np.vectorize(ints.get)(qw).astype(np.int64)
    exact = (ia @ iw.T).astype(np.float64)
    sa = np.ones((M, K // 128), np.float32)
    sw = np.ones((N // 128, K // 128), np.float32)
    # bf16 of an integer below 2^24 is the same for every variant
    first = None
    for cfg in _configs(M, N, K):
        y = _run(qa, sa, qw, sw, cfg)
        assert_close(y, exact, str(cfg))
        if first is None:
            first = y
        assert np.array_equal(y, first), str(cfg)


def test_scaling_activations_by_two_doubles_output():
    qa, sa, qw, sw = _random_operands(40, 256, 384, 3)
    for cfg in [None, fb.make_config(fb.STANDARD, 64, 128, 2), fb.make_config(fb.SWAPAB, 64, 32, 1, 2)]:
        y1 = _run(qa, sa, qw, sw, cfg)
        y2 = _run(qa, sa * np.float32(2), qw, sw, cfg)
        assert np.array_equal(y2, 2 * y1)


def _full_cases():
    """Every case of every workload: C1 single, C2 decode, C3 prefill, C4 the
    UE8M0 32B layers and all 180 cases of the C5 sweep."""
    out = []
    for config in ("single", "decode_8b", "prefill_8b", "ue8m0_32b", "sweep"):
        out += list(synth.cases(config))
    return out


@pytest.mark.parametrize("case", _full_cases(), ids=lambda c: c.cid)
def test_full_size_linear(case):
    """fp8_linear -- the call the benchmark times -- at full size in the
    dispatched configuration (UE8M0 cases with power-of-two activation and
    weight scales, so Standard tiles scale in the matrix core), against the
    oracle (its quantization of the same rows, then the fp64 GEMM) on sampled
    rows: the first and last, one in every 256-row band and up to 254 more."""
    import torch
    x = synth.activations_bf16(case)
    qw, sw = oracle_weight(case.N, case.K, case.ue8m0)
    flags = (fb.FLAG_UE8M0 | fb.FLAG_WEIGHT_POW2) if case.ue8m0 else 0
    say("full", case.cid, fb.fp8_block_gemm_select(case.M, case.N, case.K, flags).as_dict())
    y = fb.linear(to_dev_bf16(x), to_dev(qw), to_dev(sw), ue8m0=case.ue8m0, weight_pow2=case.ue8m0)
    torch.cuda.synchronize()
    rows = sample_rows(case.M, 256, key=case.N)
    qa_ref, sa_ref = oracle.group_quant(x[rows], ue8m0=case.ue8m0)
    ref = oracle.block_gemm(qa_ref, sa_ref, qw, sw)
    yh = host(y)[rows].astype(np.float64)
    del y
    assert_close(yh, ref, case.cid)


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 12288)])
def test_decode_variants_agree(N, K):
    case = synth.Case("decode_8b", "x", 64, N, K, "normal_outlier", False, 0)
    x = synth.activations_bf16(case)
    qa, sa = oracle.group_quant(x)
    qw, sw = oracle_weight(N, K, False)
    cfgs = [fb.make_config(fb.STANDARD, 64, 128, 1), fb.make_config(fb.STANDARD, 64, 128, 8),
            fb.make_config(fb.SWAPAB, 64, 16, 1, 8), fb.make_config(fb.SWAPAB, 64, 32, 4, 4),
            fb.make_config(fb.SWAPAB, 64, 16, 16, 1)]
    ys = [_run(qa, sa, qw, sw, c) for c in cfgs]
    for c, y in zip(cfgs[1:], ys[1:]):
        assert_close(y, ys[0], f"{c} vs standard")
    ref = oracle.block_gemm(qa, sa, qw, sw, rows=np.array([0, 31, 63]))
    assert_close(ys[0][[0, 31, 63]], ref, "standard vs oracle")


def test_hip_graph_replay_matches_eager():
    import torch
    case = synth.Case("decode_8b", "x", 32, 4096, 4096, "normal_outlier", False, 0)
    x = to_dev_bf16(synth.activations_bf16(case))
    qw, sw = oracle_weight(4096, 4096, False)
    qw, sw = to_dev(qw), to_dev(sw)
    cfg = fb.make_config(fb.SWAPAB, 32, 16, 4, 4)  # split-K: two kernels and a workspace
    qa = torch.empty((32, 4096), dtype=torch.uint8, device=dev())
    sa = torch.empty((32, 32), dtype=torch.float32, device=dev())
    y = torch.empty((32, 4096), dtype=torch.bfloat16, device=dev())
    ws = fb.workspace_for(32, 4096, 4096, cfg, dev())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fb.fp8_group_quant(x, qa, sa, stream=s)
        fb.fp8_block_gemm(qa, sa, qw, sw, y, cfg, ws, stream=s)
    s.synchronize()
    eager = host(y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fb.fp8_group_quant(x, qa, sa, stream=s)
        fb.fp8_block_gemm(qa, sa, qw, sw, y, cfg, ws, stream=s)
    for i in range(4):
        y.zero_()
        qa.zero_()
        torch.cuda.synchronize()
        say("graph replay", i)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), eager), f"replay {i}"


def test_hip_graph_replay_of_split_tail():
    """A split-tail launch (unsplit tiles, split tail tiles, the tail sum)
    captured in a graph: every replay equals the eager result."""
    import torch
    M, N, K = 4300, 4096, 640
    qa, sa, qw, sw = (to_dev(a) for a in _random_operands(M, N, K, 32))
    cfg = fb.make_config(fb.STANDARD, 256, 256, 2, split_tail=1)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    ws = fb.workspace_for(M, N, K, cfg, dev())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fb.fp8_block_gemm(qa, sa, qw, sw, y, cfg, ws, stream=s)
    s.synchronize()
    eager = host(y.view(torch.int16)).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fb.fp8_block_gemm(qa, sa, qw, sw, y, cfg, ws, stream=s)
    for i in range(3):
        y.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        say("split tail graph replay", i)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y.view(torch.int16)), eager), f"replay {i}"


def _pow2_configs(N, K):
    kb = K // 128
    out = []
    for tm, tn, ns in ((64, 64, 0), (64, 64, 4), (64, 128, 0), (64, 128, 4), (128, 128, 0), (128, 128, 3),
                       (256, 128, 0), (256, 128, 3), (128, 256, 0), (256, 256, 0)):
        if N % tn:
            continue
        for sk in (1, 2):
            if sk <= kb:
                out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 1, ns, fb.SCALES_POW2))
    return out


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (100, 256, 512), (257, 512, 384), (300, 768, 896)],
                         ids=lambda v: str(v))
def test_power_of_two_scale_mode_against_oracle(M, N, K):
    """UE8M0 inputs (every scale a power of two) through the matrix-core
    scaling path, against the oracle and against the fp32-scale path."""
    x = synth.activations_bf16(synth.Case("ue8m0_32b", "p2", M, N, K, "student_t3", True, 40 + M))
    qa, sa = oracle.group_quant(x, ue8m0=True)
    qw, sw = oracle_weight(N, K, True)
    assert np.all(np.frexp(sa)[0] == 0.5) and np.all(np.frexp(sw)[0] == 0.5)
    ref = oracle.block_gemm(qa, sa, qw, sw)
    base = _run(qa, sa, qw, sw, fb.make_config(fb.STANDARD, 64, 128, 1))
    for cfg in _pow2_configs(N, K):
        y = _run(qa, sa, qw, sw, cfg)
        assert_close(y, ref, str(cfg))
        assert_close(y, base, f"{cfg} vs fp32-scale path")


def test_power_of_two_scale_mode_exact_cases():
    # closed form with geometric activation scales 2^kb: 128 (2^(K/128) - 1)
    M, N, K = 20, 256, 512
    qa = np.full((M, K), 0x38, np.uint8)
    qw = np.full((N, K), 0x38, np.uint8)
    sa = np.tile((2.0 ** np.arange(K // 128)).astype(np.float32), (M, 1))
    sw = np.ones((N // 128, K // 128), np.float32)
    for cfg in _pow2_configs(N, K):
        assert np.all(_run(qa, sa, qw, sw, cfg) == 1920.0), str(cfg)
    # integer-exact operands: every path gives the same bits
    ints = {0x38: 1, 0x40: 2, 0x44: 3, 0x48: 4, 0xB8: -1, 0xC0: -2, 0x00: 0, 0x50: 8}
    codes = np.array(list(ints), dtype=np.uint8)
    rng = synth.generator(703)
    M, N, K = 64, 512, 1024
    qa = rng.choice(codes, size=(M, K)).astype(np.uint8)
    qw = rng.choice(codes, size=(N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-3, 4, size=(M, K // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-3, 4, size=(N // 128, K // 128))).astype(np.float32)
    first = _run(qa, sa, qw, sw, fb.make_config(fb.STANDARD, 64, 128, 1))
    for cfg in _pow2_configs(N, K):
        assert np.array_equal(_run(qa, sa, qw, sw, cfg), first), str(cfg)


def test_largest_operand_pitches():
    # Row pitches just below 2^24 bytes (the largest accepted): a 256-row tile
    # then spans almost 2^32 bytes, the range of the Standard kernel's 32-bit
    # load offsets.  A and W live in 4 GiB buffers; the scale arrays get
    # pitches just below 2^22 floats in a second pass.
    import torch
    M, N, K = 256, 256, 512
    qa, sa, qw, sw = _random_operands(M, N, K, 9)
    ref = oracle.block_gemm(qa, sa, qw, sw)
    big = (1 << 24) - 16
    cfgs = [fb.make_config(fb.STANDARD, 256, 256), fb.make_config(fb.STANDARD, 128, 128, 2),
            fb.make_config(fb.STANDARD, 64, 128, 1, 2, 4), fb.make_config(fb.STANDARD, 256, 128, 1, 1, 3)]
    say("gemm largest pitches: A and W")
    abuf = torch.zeros((M, big), dtype=torch.uint8, device=dev())
    wbuf = torch.zeros((N, big), dtype=torch.uint8, device=dev())
    abuf[:, :K] = to_dev(qa)
    wbuf[:, :K] = to_dev(qw)
    a, w = abuf[:, :K], wbuf[:, :K]
    sad, swd = to_dev(sa), to_dev(sw)
    for cfg in cfgs:
        say("  ", cfg.as_dict())
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        ws = torch.empty((fb.fp8_block_gemm_workspace_size(M, N, K, cfg) // 4 + 4,), dtype=torch.float32,
                         device=dev())
        fb.fp8_block_gemm(a, sad, w, swd, y, cfg, ws)
        assert_close(host(y).astype(np.float64), ref, ("pitch A/W", cfg.as_dict()))
    del abuf, wbuf, a, w
    torch.cuda.empty_cache()
    say("gemm largest pitches: scales")
    sbig = (1 << 22) - 4
    sabuf = torch.zeros((M, sbig), dtype=torch.float32, device=dev())
    swbuf = torch.zeros((N // 128, sbig), dtype=torch.float32, device=dev())
    sabuf[:, : K // 128] = sad
    swbuf[:, : K // 128] = swd
    for cfg in cfgs:
        say("  ", cfg.as_dict())
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        ws = torch.empty((fb.fp8_block_gemm_workspace_size(M, N, K, cfg) // 4 + 4,), dtype=torch.float32,
                         device=dev())
        fb.fp8_block_gemm(to_dev(qa), sabuf[:, : K // 128], to_dev(qw), swbuf[:, : K // 128], y, cfg, ws)
        assert_close(host(y).astype(np.float64), ref, ("pitch scales", cfg.as_dict()))
    del sabuf, swbuf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kb", [1, 2, 3, 4, 5, 7, 9])
def test_k_loop_depths_splits_and_stages(kb):
    # The K loop consumes NS blocks per trip and fills each stage during the
    # block after the one that consumed it; its tail handles the last
    # kb mod NS blocks, and split-K can leave uneven or empty trailing
    # splits.  Every depth 1..9 blocks against every stage count and split.
    M, N, K = 70, 256, 128 * kb
    qa, sa, qw, sw = _random_operands(M, N, K, 100 + kb)
    ref = oracle.block_gemm(qa, sa, qw, sw)
    # power-of-two scale mode: the same operands with sa, sw rounded to 2^e
    sa2 = np.exp2(np.round(np.log2(sa))).astype(np.float32)
    sw2 = np.exp2(np.round(np.log2(sw))).astype(np.float32)
    ref2 = oracle.block_gemm(qa, sa2, qw, sw2)
    for (tm, tn, kw, stages) in ((64, 64, 1, 0), (64, 64, 2, 3), (64, 128, 1, 0), (64, 128, 1, 3),
                                 (64, 128, 1, 4), (64, 128, 2, 4), (128, 128, 1, 3), (128, 128, 2, 3),
                                 (256, 256, 1, 0), (256, 128, 1, 3)):
        for sk in (1, 2, 3, 4, 6):
            if sk > kb:
                continue
            cfg = fb.make_config(fb.STANDARD, tm, tn, sk, kw, stages)
            assert_close(_run(qa, sa, qw, sw, cfg), ref, ("fp32", kb, cfg.as_dict()))
            cfg.scale_mode = fb.SCALES_POW2
            assert_close(_run(qa, sa2, qw, sw2, cfg), ref2, ("pow2", kb, cfg.as_dict()))


def test_bf16_output_rounding_ties_and_subnormals():
    # y[m][n] = sa[m] exactly (one K block, a single 1.0 x 1.0 product per
    # output, sw = 1), so the output bits are the bf16 rounding of sa[m]
    # alone: ties go to the even neighbour, subnormals are kept.  Expected
    # bits worked out by hand; every Standard tile and Swap-AB configuration.
    targets = [
        (1.0 + 2.0 ** -8, 0x3F80),                  # tie between 1 and 1 + 2^-7 -> even (1)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),              # tie between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),     # just above the tie -> up
        (-(1.0 + 2.0 ** -8), 0xBF80),
        (2.0 ** -130, 0x0008),                      # bf16 subnormal 8 * 2^-133
        (1.5 * 2.0 ** -133, 0x0002),                # tie between 1 and 2 units of 2^-133 -> even (2)
        (0.5 * 2.0 ** -133, 0x0000),                # tie between 0 and 2^-133 -> even (0)
        (3.0, 0x4040),
    ]
    M, N, K = 16, 256, 128
    sa = np.ones((M, 1), np.float32)
    for i, (v, _) in enumerate(targets):
        sa[i, 0] = np.float32(v)
        assert float(sa[i, 0]) == v                 # exact in fp32
    qa = np.zeros((M, K), np.uint8)
    qa[:, 0] = 0x38                                 # e4m3 1.0
    qw = np.zeros((N, K), np.uint8)
    qw[:, 0] = 0x38
    sw = np.ones((N // 128, 1), np.float32)
    expect = np.full((M, N), 0x3F80, np.uint16)     # rows past the targets: sa = 1
    for i, (_, bits) in enumerate(targets):
        expect[i, :] = bits
    cfgs = [fb.make_config(fb.STANDARD, tm, tn) for tm, tn in ((64, 64), (64, 128), (128, 128), (256, 128),
                                                                (128, 256), (256, 256))]
    cfgs += [fb.make_config(fb.STANDARD, 64, 128, 1, 2), fb.make_config(fb.STANDARD, 128, 128, 1, 2, 3),
             fb.make_config(fb.STANDARD, 64, 64, 1, 2)]
    cfgs += [fb.make_config(fb.SWAPAB, tm, tn, 1, kw) for tm in (16, 32, 64) for tn in (16, 32, 64)
             for kw in (1, 2) if not (tm == 64 and tn == 64)]
    for cfg in cfgs:
        say("bf16 rounding", cfg.as_dict())
        import torch
        y = fb.block_gemm(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), cfg)
        got = host(y.view(torch.int16)).view(np.uint16)
        if not np.array_equal(got, expect):
            bad = np.argwhere(got != expect)[:4]
            raise AssertionError((cfg.as_dict(), [(tuple(b), hex(got[tuple(b)]), hex(expect[tuple(b)])) for b in bad]))


def _walk(tiles_m, tiles_n):
    """(tile row, tile column) of each tile in the Standard kernel's walk
    order: column groups of 8 tile-rows, column by column inside a group."""
    out = []
    for t in range(tiles_m * tiles_n):
        first = t // (8 * tiles_n) * 8
        gm = min(8, tiles_m - first)
        out.append((first + t % (8 * tiles_n) % gm, t % (8 * tiles_n) // gm))
    return out


_TAIL_CASES = [(256, 256, 1, 0, "block"), (128, 256, 1, 0, "block"), (256, 128, 1, 3, "block"),
               (128, 128, 1, 0, "block"), (128, 128, 2, 3, "block"), (64, 128, 1, 4, "block"),
               (256, 256, 1, 0, "pow2"), (128, 128, 2, 0, "pow2"), (256, 256, 1, 0, "dynamic"),
               (64, 128, 2, 3, "dynamic"), (64, 64, 1, 3, "block"), (64, 64, 2, 0, "dynamic")]


@pytest.mark.parametrize("tm,tn,kw,ns,mode", _TAIL_CASES, ids=lambda v: str(v))
def test_split_tail_takes_each_tile_from_the_unsplit_or_the_split_run(tm, tn, kw, ns, mode):
    """Split tail: the tiles of the whole rounds of resident workgroups run
    unsplit, the rest split.  More tiles than any round (M = 4300, a ragged
    last tile row), K = 640 (5 blocks: the splits are 3 + 2 and 2 + 2 + 1).
    In the kernel's walk order, the tiles before some multiple d of the CU
    count (d < tiles) must equal, bit for bit, the unsplit run's and the
    tiles from d on the plain Split-K run's; both runs must differ from the
    result somewhere; sampled rows match the oracle."""
    import torch
    M, N, K = 4300, 4096, 640
    qa, sa, qw, sw = _random_operands(M, N, K, 31)
    rows = sample_rows(M, 8, 3)
    if mode == "pow2":      # every scale a power of two, applied by the matrix core
        sa, sw = (np.exp2(np.round(np.log2(v))).astype(np.float32) for v in (sa, sw))
    if mode == "dynamic":   # per-token / per-channel scales (scaled_mm)
        sa, sw = np.ascontiguousarray(sa[:, 0]), np.repeat(sw[:, 0], 128).astype(np.float32)
        ref = oracle.scaled_mm(qa, sa, qw, sw, rows=rows)
        run = fb.scaled_mm
    else:
        ref = oracle.block_gemm(qa, sa, qw, sw, rows=rows)
        run = fb.block_gemm
    sm = fb.SCALES_POW2 if mode == "pow2" else fb.SCALES_FP32
    args = [to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw)]
    walk = _walk(-(-M // tm), N // tn)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for sk in (2, 3):
        say("split tail", tm, tn, kw, ns, mode, sk)
        y1 = host(run(*args, fb.make_config(fb.STANDARD, tm, tn, 1, kw, ns, sm)).view(torch.int16))
        ys = host(run(*args, fb.make_config(fb.STANDARD, tm, tn, sk, kw, ns, sm)).view(torch.int16))
        yt_dev = run(*args, fb.make_config(fb.STANDARD, tm, tn, sk, kw, ns, sm, split_tail=1))
        yt = host(yt_dev.view(torch.int16))
        tile = lambda a, r, c: a[r * tm:(r + 1) * tm, c * tn:(c + 1) * tn]
        eq_u = np.array([np.array_equal(tile(yt, r, c), tile(y1, r, c)) for r, c in walk])
        eq_s = np.array([np.array_equal(tile(yt, r, c), tile(ys, r, c)) for r, c in walk])
        ok = [d for d in range(cus, len(walk), cus) if eq_u[:d].all() and eq_s[d:].all()]
        assert ok, (tm, tn, sk, np.flatnonzero(~eq_u)[:8], np.flatnonzero(~eq_s)[:8])
        assert not eq_u.all() and not eq_s.all(), (tm, tn, sk)
        assert_close(host(yt_dev)[rows].astype(np.float64), ref, f"split tail {tm}x{tn} {mode} sk{sk}")


def _run_mn(qa, sa, qw, sw, cfg):
    """The same GEMM with the activation scales token-contiguous: sa^T stored
    [K/128][M + 8] (a padded pitch), configuration bit FP8BLK_SCALES_SA_MN_MAJOR."""
    M, G = sa.shape
    st = np.full((G, M + 8), np.nan, np.float32)
    st[:, :M] = sa.T
    c = fb.make_config(cfg.variant, cfg.tile_m, cfg.tile_n, cfg.split_k, cfg.kwaves, cfg.stages,
                       cfg.scale_mode | fb.SCALES_SA_MN_MAJOR, cfg.split_tail)
    say("gemm mn-major scales", qa.shape, qw.shape, c.as_dict())
    y = fb.block_gemm(to_dev(qa), to_dev(st)[:, :M], to_dev(qw), to_dev(sw), c)
    return host(y).astype(np.float64)


@pytest.mark.parametrize("M,N,K", SMALL, ids=lambda v: str(v))
def test_token_contiguous_scales_equal_row_major(M, N, K):
    """Every configuration reads token-contiguous activation scales to the
    same result, bit for bit, as row-major ones (only the scale addresses
    differ), and that result is within the oracle's tolerance."""
    qa, sa, qw, sw = _random_operands(M, N, K, 2)
    ref = oracle.block_gemm(qa, sa, qw, sw)
    for cfg in _configs(M, N, K):
        y = _run(qa, sa, qw, sw, cfg)
        ym = _run_mn(qa, sa, qw, sw, cfg)
        assert np.array_equal(y, ym), str(cfg)
        assert_close(ym, ref, str(cfg))


def test_token_contiguous_power_of_two_scales():
    M, N, K = 300, 768, 896
    x = synth.activations_bf16(synth.Case("ue8m0_32b", "p2", M, N, K, "student_t3", True, 41))
    qa, sa = oracle.group_quant(x, ue8m0=True)
    qw, sw = oracle_weight(N, K, True)
    ref = oracle.block_gemm(qa, sa, qw, sw)
    for cfg in _pow2_configs(N, K):
        y = _run(qa, sa, qw, sw, cfg)
        ym = _run_mn(qa, sa, qw, sw, cfg)
        assert np.array_equal(y, ym), str(cfg)
        assert_close(ym, ref, str(cfg))
