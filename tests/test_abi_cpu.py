"""C ABI checks that need no GPU: the library loads, exports every function
include/fp8blk.h declares, and rejects every invalid argument with its status
code before any HIP call (the fake device addresses used here are never
dereferenced).  Also the per-shape dispatcher, which is host-only.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
from fp8_blockwise_quantized_token_amd import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp8blk.h")

OK, NULL, SHAPE, MISAL, STRIDE, WS, CFG = 0, -1, -2, -3, -4, -5, -6
A = 0x10000  # fake 16-byte aligned device addresses
B = 0x20000
C = 0x30000
D = 0x40000
E = 0x50000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"fp8_group_quant", "fp8_block_gemm", "fp8_block_gemm_select"} <= set(names)
    L = fb.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert fb.fp8_abi_version() == fb.ABI_VERSION == 6
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert fb.fp8_status_string(st) != "unknown status"
    assert fb.fp8_status_string(-99) == "unknown status"


def _gq(x=A, M=4, K=256, ldx=256, q=B, ldq=256, s=C, lds=2, group=128, eps=1e-10, flags=0):
    return fb.lib().fp8_group_quant(x, M, K, ldx, q, ldq, s, lds, group, eps, flags, None)


def test_group_quant_argument_errors():
    assert _gq(x=None) == NULL
    assert _gq(q=None) == NULL
    assert _gq(s=None) == NULL
    assert _gq(K=200, ldx=200, ldq=200) == SHAPE
    assert _gq(M=-1) == SHAPE
    assert _gq(group=64) == SHAPE
    assert _gq(eps=0.0) == SHAPE
    assert _gq(eps=float("inf")) == SHAPE
    # eps below the floor 2^-80 is rejected; the floor itself is accepted
    assert _gq(eps=2.0 ** -81) == SHAPE and _gq(eps=1e-38) == SHAPE
    assert _gq(eps=2.0 ** -80, M=0) == OK
    assert _gq(flags=2) == CFG
    assert _gq(ldx=128) == STRIDE
    assert _gq(ldq=128) == STRIDE
    assert _gq(lds=1) == STRIDE
    assert _gq(x=A + 2) == MISAL
    assert _gq(q=B + 8) == MISAL
    assert _gq(s=C + 2) == MISAL
    assert _gq(ldx=260, ldq=256) == MISAL
    assert _gq(ldq=264) == MISAL
    # M == 0 is a no-op, no pointer is needed
    assert _gq(M=0, x=None, q=None, s=None) == OK


def _wq(w=A, N=256, K=256, ldw=256, q=B, ldq=256, s=C, lds=2, eps=1e-10, flags=0):
    return fb.lib().fp8_weight_block_quant(w, N, K, ldw, q, ldq, s, lds, eps, flags, None)


def test_weight_quant_argument_errors():
    assert _wq(w=None) == NULL
    assert _wq(N=200) == SHAPE
    assert _wq(K=200, ldw=200, ldq=200) == SHAPE
    assert _wq(ldw=128) == STRIDE
    assert _wq(eps=2.0 ** -81) == SHAPE and _wq(eps=0.0) == SHAPE
    assert _wq(w=A + 4) == MISAL
    assert _wq(ldw=257) == MISAL
    assert _wq(flags=4) == CFG
    assert _wq(N=0, w=None, q=None, s=None) == OK


def test_encode_argument_errors():
    L = fb.lib()
    assert L.fp8_e4m3_encode(None, B, 16, None) == NULL
    assert L.fp8_e4m3_encode(A, None, 16, None) == NULL
    assert L.fp8_e4m3_encode(A + 4, B, 16, None) == MISAL
    assert L.fp8_e4m3_encode(A, B, -1, None) == SHAPE
    assert L.fp8_e4m3_encode(None, None, 0, None) == OK


def _gemm(a=A, sa=B, lda=256, ldsa=2, w=C, sw=D, ldw=256, ldsw=2, y=E, ldy=256, M=8, N=256, K=256,
          cfg=None, ws=None, ws_bytes=0):
    return fb.lib().fp8_block_gemm(a, sa, lda, ldsa, w, sw, ldw, ldsw, y, ldy, M, N, K,
                                   ctypes.byref(cfg) if cfg is not None else None, ws, ws_bytes, None)


def test_gemm_argument_errors():
    std = fb.make_config(fb.STANDARD, 128, 128)
    assert _gemm(a=None, cfg=std) == NULL
    assert _gemm(sa=None, cfg=std) == NULL
    assert _gemm(w=None, cfg=std) == NULL
    assert _gemm(sw=None, cfg=std) == NULL
    assert _gemm(y=None, cfg=std) == NULL
    assert _gemm(K=200, lda=256, ldw=256, cfg=std) == SHAPE
    assert _gemm(N=200, ldy=256, cfg=std) == SHAPE
    assert _gemm(M=-1, cfg=std) == SHAPE
    assert _gemm(lda=128, cfg=std) == STRIDE
    assert _gemm(ldw=128, cfg=std) == STRIDE
    assert _gemm(ldy=128, cfg=std) == STRIDE
    assert _gemm(ldsa=1, cfg=std) == STRIDE
    assert _gemm(ldsw=1, cfg=std) == STRIDE
    # operand row pitches below 2^24 bytes (a 256-row tile spans < 2^32 bytes)
    big = 1 << 24
    assert _gemm(lda=big, cfg=std) == STRIDE and _gemm(lda=big - 16, M=0, cfg=std) == OK
    assert _gemm(ldw=big, cfg=std) == STRIDE and _gemm(ldw=big, cfg=None) == STRIDE
    assert _gemm(ldsa=big // 4, cfg=std) == STRIDE and _gemm(ldsw=big // 4, cfg=std) == STRIDE
    assert _gemm(a=A + 1, cfg=std) == MISAL
    assert _gemm(w=C + 8, cfg=std) == MISAL
    assert _gemm(y=E + 2, cfg=std) == MISAL
    assert _gemm(lda=264, cfg=std) == MISAL
    assert _gemm(ldy=260, cfg=std) == MISAL
    assert _gemm(sa=B + 1, cfg=std) == MISAL
    # configurations
    assert _gemm(cfg=fb.make_config(7, 128, 128)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 96, 128)) == CFG
    assert _gemm(N=384, ldy=384, cfg=fb.make_config(fb.STANDARD, 128, 256)) == CFG  # N % tile_n
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, split_k=0)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, split_k=4)) == CFG  # K/128 = 2 blocks
    assert _gemm(cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 3)) == CFG         # kwaves
    assert _gemm(M=40, cfg=fb.make_config(fb.SWAPAB, 32, 16, 1, 4)) == CFG   # M > tile_m
    # split tail: 0 or 1, Standard only
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, split_tail=5)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, split_tail=-1)) == CFG
    assert _gemm(cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2, split_tail=1)) == CFG
    # scale modes: fp32 or power-of-two (Standard only), each optionally with
    # token-contiguous activation scales
    for bad in (4, 3 | 4, 8, -1):
        assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, scale_mode=bad)) == CFG, bad
    assert _gemm(cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2, scale_mode=fb.SCALES_POW2)) == CFG
    assert _gemm(cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2, scale_mode=fb.SCALES_POW2 | 2)) == CFG
    # token-contiguous activation scales: [K/128][ldsa] needs ldsa >= M, and a
    # K block's offset (K/128) ldsa 4 below 2^31 bytes
    for mode in (fb.SCALES_SA_MN_MAJOR, fb.SCALES_POW2 | fb.SCALES_SA_MN_MAJOR):
        mn = fb.make_config(fb.STANDARD, 128, 128, scale_mode=mode)
        assert _gemm(cfg=mn, ldsa=2) == STRIDE          # 2 < M = 8
        assert _gemm(cfg=mn, ldsa=8, M=0) == OK
        assert _gemm(cfg=mn, ldsa=8, sa=None) == NULL   # accepted up to the pointer check
        assert _gemm(cfg=mn, ldsa=1 << 21, M=8, K=128 * 256, lda=128 * 256, ldw=128 * 256, ldsw=256) == STRIDE
    swmn = fb.make_config(fb.SWAPAB, 16, 16, 1, 2, scale_mode=fb.SCALES_SA_MN_MAJOR)
    assert _gemm(cfg=swmn, ldsa=2) == STRIDE and _gemm(cfg=swmn, ldsa=8, sa=None) == NULL
    # LDS pipeline depth: compiled per tile; Swap-AB takes none
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 256, 256, stages=3)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, stages=4)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 64, 128, stages=5)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 64, 128, stages=1)) == CFG
    # twice the waves: 64x128 and 128x128 only, at most 4 / 3 stages; kwaves 1 or 2
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 256, 256, kwaves=2)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, kwaves=2, stages=4)) == CFG
    assert _gemm(cfg=fb.make_config(fb.STANDARD, 128, 128, kwaves=3)) == CFG
    assert _gemm(M=0, a=None, sa=None, w=None, sw=None, y=None, cfg=fb.make_config(fb.STANDARD, 64, 128, kwaves=2, stages=4)) == OK
    assert _gemm(cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2, stages=2)) == CFG
    # split-K needs a workspace of split * M * N * 4 bytes
    sk = fb.make_config(fb.STANDARD, 128, 128, split_k=2)
    assert fb.fp8_block_gemm_workspace_size(8, 256, 256, sk) == 2 * 8 * 256 * 4
    assert _gemm(cfg=sk) == WS
    assert _gemm(cfg=sk, ws=0x60000, ws_bytes=2 * 8 * 256 * 4 - 1) == WS
    assert _gemm(cfg=sk, ws=0x60004, ws_bytes=2 * 8 * 256 * 4) == MISAL
    # M == 0 is a no-op
    assert _gemm(M=0, a=None, sa=None, w=None, sw=None, y=None, cfg=std) == OK


def test_select_and_workspace_queries():
    L = fb.lib()
    assert L.fp8_block_gemm_select(1, 4096, 4096, 0, None) == NULL
    assert L.fp8_block_gemm_workspace_size(1, 100, 4096, None) == SHAPE
    for config in ("single", "decode_8b", "prefill_8b", "ue8m0_32b", "sweep"):
        for case in synth.cases(config):
            c = fb.fp8_block_gemm_select(case.M, case.N, case.K)
            # every dispatched configuration is one the library accepts
            n = fb.fp8_block_gemm_workspace_size(case.M, case.N, case.K, c)
            assert n == (c.split_k * case.M * case.N * 4 if c.split_k > 1 else 0)
            assert n == fb.fp8_block_gemm_workspace_size(case.M, case.N, case.K, None)
            if c.variant == fb.SWAPAB:
                assert case.M <= c.tile_m
            assert 1 <= c.split_k <= case.K // 128


def test_select_power_of_two_mode_needs_both_flags():
    both = fb.FLAG_UE8M0 | fb.FLAG_WEIGHT_POW2
    for config in ("prefill_8b", "ue8m0_32b", "decode_8b"):
        for case in synth.cases(config):
            plain = fb.fp8_block_gemm_select(case.M, case.N, case.K, 0)
            p2 = fb.fp8_block_gemm_select(case.M, case.N, case.K, both)
            assert plain.scale_mode == fb.SCALES_FP32
            want = fb.SCALES_POW2 if plain.variant == fb.STANDARD else fb.SCALES_FP32
            assert p2.scale_mode == want
            # one of the two alone: power-of-two activations with fp32 weight
            # scales (or the converse) keep the fp32 mode
            for one in (fb.FLAG_UE8M0, fb.FLAG_WEIGHT_POW2):
                assert fb.fp8_block_gemm_select(case.M, case.N, case.K, one).scale_mode == fb.SCALES_FP32
            d1, d2 = plain.as_dict(), p2.as_dict()
            d1.pop("scale_mode"), d2.pop("scale_mode")
            assert d1 == d2


def test_select_rejects_unknown_flags():
    c = fb.GemmConfig()
    for flags in (2, 4, 16, 1 << 31):
        assert fb.lib().fp8_block_gemm_select(64, 4096, 4096, flags, ctypes.byref(c)) == CFG


def test_linear_power_of_two_config_needs_both_flags():
    # the matrix core keeps only the exponent bits of every scale: a caller's
    # power-of-two configuration is refused unless the activation scales
    # (FP8BLK_FLAG_UE8M0) and the weight scales (FP8BLK_FLAG_WEIGHT_POW2) are
    # both powers of two; nothing is launched
    p2 = fb.make_config(fb.STANDARD, 128, 128, scale_mode=fb.SCALES_POW2)
    n = fb.fp8_linear_workspace_size(8, 256, 256, p2)
    for flags in (0, fb.FLAG_UE8M0, fb.FLAG_WEIGHT_POW2):
        assert _lin(flags=flags, cfg=p2, ws=0x70000, ws_bytes=n) == CFG, flags
    # unknown flag bits are refused too
    assert _lin(flags=16, cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2)) == CFG
    assert _lin(flags=fb.FLAG_UE8M0 | 2, cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2)) == CFG


def test_select_is_deterministic_and_swaps_small_m():
    a = fb.fp8_block_gemm_select(8, 24576, 4096).as_dict()
    b = fb.fp8_block_gemm_select(8, 24576, 4096).as_dict()
    assert a == b
    assert fb.fp8_block_gemm_select(1, 4096, 4096).variant == fb.SWAPAB
    assert fb.fp8_block_gemm_select(8192, 4096, 4096).variant == fb.STANDARD
    # a shape no table holds still gets a valid configuration
    c = fb.fp8_block_gemm_select(777, 384, 1152)
    assert fb.fp8_block_gemm_workspace_size(777, 384, 1152, c) >= 0


def test_select_splits_the_tail_round_of_untabled_shapes():
    # N = 512, K = 1024 is far from every tabled shape (the heuristic decides):
    # 256x256 tiles, 2 per tile row
    for M, sk, tail in ((130 * 256, 4, 1), (150 * 256 - 100, 4, 1), (190 * 256, 2, 1), (200 * 256, 1, 0),
                        (256 * 256, 1, 0)):  # the last: whole rounds only
        c = fb.fp8_block_gemm_select(M, 512, 1024)
        assert (c.tile_m, c.tile_n, c.split_k, c.split_tail) == (256, 256, sk, tail), (M, c.as_dict())
        if tail:
            assert fb.fp8_block_gemm_workspace_size(M, 512, 1024, c) == sk * M * 512 * 4
    # too few K blocks to split: no tail split
    c = fb.fp8_block_gemm_select(130 * 256, 512, 384)
    assert c.split_tail == 0 and c.split_k == 1


def test_select_takes_the_nearest_tabled_shape():
    # Llama-like layers next to tabled Qwen3 ones get their neighbour's configuration
    for (n, k), (tn, tk) in (((28672, 4096), (24576, 4096)), ((4096, 14336), (4096, 12288)),
                             ((57344, 8192), (51200, 5120)), ((8192, 28672), (5120, 25600))):
        for M in (1, 8, 32, 64, 256, 1024, 8192):
            a = fb.fp8_block_gemm_select(M, n, k).as_dict()
            b = fb.fp8_block_gemm_select(M, tn, tk).as_dict()
            assert a == b, (M, n, k, a, b)


def test_selected_configs_are_valid_for_any_shape():
    rng = np.random.default_rng(5)
    for _ in range(3000):
        M = int(rng.integers(1, 20000))
        N = 128 * int(rng.integers(1, 600))
        K = 128 * int(rng.integers(1, 300))
        for flags in (0, fb.FLAG_UE8M0, fb.FLAG_UE8M0 | fb.FLAG_WEIGHT_POW2):
            c = fb.fp8_block_gemm_select(M, N, K, flags)
            assert fb.fp8_block_gemm_workspace_size(M, N, K, c) >= 0, (M, N, K, flags, c.as_dict())
            assert fb.fp8_linear_workspace_size(M, N, K, c) >= 0, (M, N, K, flags, c.as_dict())


def _lin(x=A, ldx=256, w=C, sw=D, ldw=256, ldsw=2, y=E, ldy=256, M=8, N=256, K=256, eps=1e-10,
         flags=0, cfg=None, ws=None, ws_bytes=0):
    return fb.lib().fp8_linear(x, ldx, w, sw, ldw, ldsw, y, ldy, M, N, K, eps, flags,
                               ctypes.byref(cfg) if cfg is not None else None, ws, ws_bytes, None)


def test_linear_argument_errors():
    sw1 = fb.make_config(fb.SWAPAB, 16, 16, 1, 2)
    std = fb.make_config(fb.STANDARD, 128, 128)
    assert _lin(x=None, cfg=sw1) == NULL
    assert _lin(w=None, cfg=sw1) == NULL
    assert _lin(sw=None, cfg=sw1) == NULL
    assert _lin(y=None, cfg=sw1) == NULL
    assert _lin(K=200, cfg=sw1) == SHAPE
    assert _lin(N=200, cfg=sw1) == SHAPE
    assert _lin(M=-1, cfg=sw1) == SHAPE
    assert _lin(K=(1 << 22) + 128, ldx=(1 << 22) + 128, ldw=(1 << 22) + 128, ldsw=1 << 16,
                cfg=sw1) == SHAPE
    assert _lin(eps=0.0, cfg=sw1) == SHAPE and _lin(eps=2.0 ** -81, cfg=sw1) == SHAPE
    assert _lin(eps=float("nan"), cfg=sw1) == SHAPE
    assert _lin(flags=2, cfg=sw1) == CFG
    assert _lin(ldx=128, cfg=sw1) == STRIDE
    assert _lin(ldw=128, cfg=sw1) == STRIDE
    assert _lin(ldy=128, cfg=sw1) == STRIDE
    assert _lin(ldsw=1, cfg=sw1) == STRIDE
    assert _lin(ldw=1 << 24, cfg=sw1) == STRIDE and _lin(ldsw=1 << 22, cfg=sw1) == STRIDE
    assert _lin(x=A + 2, cfg=sw1) == MISAL
    assert _lin(ldx=260, cfg=sw1) == MISAL
    assert _lin(M=40, cfg=sw1) == CFG  # Swap-AB tile_m < M
    # Swap-AB with one token tile quantizes in the GEMM: workspace only for split-K partials
    assert fb.fp8_linear_workspace_size(8, 256, 256, sw1) == 0
    # two token tiles, and four with 16 weight rows, quantize in the GEMM too
    assert fb.fp8_linear_workspace_size(20, 256, 256, fb.make_config(fb.SWAPAB, 32, 16, 1, 2)) == 0
    assert fb.fp8_linear_workspace_size(40, 256, 256, fb.make_config(fb.SWAPAB, 64, 16, 1, 2)) == 0
    # four token tiles with 32 weight rows quantize first: q [M][K] and s [M][K/128], each padded to 256 bytes
    assert fb.fp8_linear_workspace_size(40, 256, 256, fb.make_config(fb.SWAPAB, 64, 32, 1, 2)) == 40 * 256 + 512
    sk = fb.make_config(fb.SWAPAB, 16, 16, 2, 1)
    assert fb.fp8_linear_workspace_size(8, 256, 256, sk) == 2 * 8 * 256 * 4
    assert _lin(cfg=sk) == WS
    # Standard: q [M][K] bytes and s [M][K/128] floats first, each padded to 256 bytes
    n = fb.fp8_linear_workspace_size(8, 256, 256, std)
    assert n == 8 * 256 + 256
    assert _lin(cfg=std) == WS
    assert _lin(cfg=std, ws=0x60000, ws_bytes=n - 1) == WS
    assert _lin(cfg=std, ws=0x60008, ws_bytes=n) == MISAL
    stdk = fb.make_config(fb.STANDARD, 64, 128, 2)
    assert fb.fp8_linear_workspace_size(300, 256, 256, stdk) == 300 * 256 + 2560 + 2 * 300 * 256 * 4
    assert _lin(M=0, x=None, w=None, sw=None, y=None, cfg=std) == OK
    # the dispatched configuration is the GEMM's
    for config in ("decode_8b", "prefill_8b"):
        for case in synth.cases(config):
            assert fb.fp8_linear_workspace_size(case.M, case.N, case.K) == \
                fb.fp8_linear_workspace_size(case.M, case.N, case.K,
                                             fb.fp8_block_gemm_select(case.M, case.N, case.K))


def test_dynamic_entry_argument_errors():
    L = fb.lib()
    tq = lambda x=A, M=4, K=256, ldx=256, q=B, ldq=256, s=C, eps=1e-10, flags=0: \
        L.fp8_token_quant(x, M, K, ldx, q, ldq, s, eps, flags, None)
    assert tq(x=None) == NULL and tq(q=None) == NULL and tq(s=None) == NULL
    assert tq(K=200, ldx=256, ldq=256) == SHAPE
    assert tq(K=32768 + 128, ldx=40000, ldq=40000) == SHAPE
    assert tq(M=-1) == SHAPE and tq(eps=0.0) == SHAPE and tq(flags=2) == CFG
    assert tq(eps=2.0 ** -81) == SHAPE
    assert tq(ldx=128) == STRIDE and tq(ldq=128) == STRIDE
    assert tq(x=A + 2) == MISAL and tq(ldx=260) == MISAL and tq(s=C + 2) == MISAL
    assert tq(M=0, x=None, q=None, s=None) == OK
    cq = lambda w=A, N=128, K=256, ldw=256, q=B, ldq=256, s=C, eps=1e-10, flags=0: \
        L.fp8_weight_channel_quant(w, N, K, ldw, q, ldq, s, eps, flags, None)
    assert cq(w=None) == NULL and cq(K=100, ldw=256, ldq=256) == SHAPE and cq(ldw=200) == STRIDE
    assert cq(ldw=258) == MISAL and cq(N=0, w=None, q=None, s=None) == OK
    assert cq(eps=2.0 ** -81) == SHAPE
    sm = lambda a=A, sa=B, lda=256, w=C, sw=D, ldw=256, y=E, ldy=256, M=8, N=256, K=256, cfg=None, ws=None, n=0: \
        L.fp8_scaled_mm(a, sa, lda, w, sw, ldw, y, ldy, M, N, K,
                        ctypes.byref(cfg) if cfg is not None else None, ws, n, None)
    std = fb.make_config(fb.STANDARD, 128, 128)
    assert sm(a=None, cfg=std) == NULL and sm(sa=None, cfg=std) == NULL and sm(sw=None, cfg=std) == NULL
    assert sm(K=200, cfg=std) == SHAPE and sm(N=200, cfg=std) == SHAPE
    assert sm(lda=128, cfg=std) == STRIDE and sm(ldy=128, cfg=std) == STRIDE
    assert sm(lda=1 << 24, cfg=std) == STRIDE and sm(ldw=1 << 24, cfg=std) == STRIDE
    assert sm(sa=B + 2, cfg=std) == MISAL and sm(a=A + 1, cfg=std) == MISAL
    assert sm(cfg=fb.make_config(fb.STANDARD, 128, 128, scale_mode=fb.SCALES_POW2)) == CFG
    assert sm(cfg=fb.make_config(fb.STANDARD, 128, 128, split_k=2)) == WS
    assert sm(M=0, a=None, sa=None, w=None, sw=None, y=None, cfg=std) == OK


def test_group_quant_scale_format_flags():
    # E8M0 bytes hold powers of two only; MN-major needs lds >= M; unknown bits rejected
    assert _gq(flags=2) == CFG
    assert _gq(flags=8) == CFG
    assert _gq(M=4, flags=4, lds=3) == STRIDE
    assert _gq(M=0, flags=1 | 2 | 4, x=None, q=None, s=None, lds=0) == OK


def test_header_abi_version_matches_the_binding():
    m = re.search(r"#define\s+FP8BLK_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == fb.ABI_VERSION


def test_fused_producer_argument_errors():
    L = fb.lib()
    rq = lambda x=A, M=4, H=256, ldx=256, w=D, en=1e-6, q=B, ldq=256, s=C, lds=2, eps=1e-10, flags=0: \
        L.fp8_rms_norm_per_block_quant(x, M, H, ldx, w, en, q, ldq, s, lds, eps, flags, None)
    assert rq(x=None) == NULL and rq(w=None) == NULL and rq(q=None) == NULL and rq(s=None) == NULL
    assert rq(H=200, ldx=256, ldq=256) == SHAPE and rq(H=0) == SHAPE and rq(M=-1) == SHAPE
    assert rq(H=32768 + 128, ldx=40000, ldq=40000, lds=300) == SHAPE
    assert rq(eps=0.0) == SHAPE and rq(en=-1.0) == SHAPE and rq(en=float("inf")) == SHAPE
    assert rq(eps=2.0 ** -81) == SHAPE
    assert rq(en=float("nan")) == SHAPE
    assert rq(ldx=128) == STRIDE and rq(ldq=128) == STRIDE and rq(lds=1) == STRIDE
    assert rq(flags=2) == CFG and rq(flags=8) == CFG and rq(flags=4, lds=3) == STRIDE
    assert rq(x=A + 2) == MISAL and rq(w=D + 4) == MISAL and rq(q=B + 8) == MISAL
    assert rq(s=C + 2) == MISAL and rq(ldx=260) == MISAL and rq(ldq=264) == MISAL
    assert rq(M=0, x=None, w=None, q=None, s=None) == OK
    sq = lambda x=A, M=4, I=256, ldx=512, q=B, ldq=256, s=C, lds=2, eps=1e-10, flags=0: \
        L.fp8_silu_and_mul_per_block_quant(x, M, I, ldx, q, ldq, s, lds, eps, flags, None)
    assert sq(x=None) == NULL and sq(q=None) == NULL and sq(s=None) == NULL
    assert sq(I=200, ldx=512, ldq=256) == SHAPE and sq(I=0) == SHAPE and sq(M=-1) == SHAPE
    assert sq(eps=0.0) == SHAPE and sq(flags=2) == CFG and sq(flags=16) == CFG
    assert sq(eps=2.0 ** -81) == SHAPE
    assert sq(ldx=511) == STRIDE and sq(ldx=256) == STRIDE and sq(ldq=128) == STRIDE
    assert sq(lds=1) == STRIDE and sq(flags=4, lds=3) == STRIDE
    assert sq(x=A + 2) == MISAL and sq(ldx=516) == MISAL and sq(s=C + 2) == MISAL
    assert sq(M=0, x=None, q=None, s=None) == OK


def test_linear_noalloc_argument_errors():
    # every argument error, and a workspace need beyond the library's scratch
    # array, is reported before the array is looked up or anything launched
    L = fb.lib()

    def f(M=8, N=256, K=256, ldx=None, cfg=None, flags=0):
        ldx = K if ldx is None else ldx
        return L.fp8_linear_noalloc(A, ldx, C, D, K, K // 128, E, N, M, N, K, 1e-10, flags,
                                    ctypes.byref(cfg) if cfg is not None else None, None)
    assert f(K=200) == SHAPE and f(N=200) == SHAPE and f(M=-1) == SHAPE
    assert f(ldx=128) == STRIDE
    assert f(flags=16) == CFG
    assert f(cfg=fb.make_config(fb.STANDARD, 128, 128, scale_mode=fb.SCALES_POW2), flags=fb.FLAG_UE8M0) == CFG
    assert f(cfg=fb.make_config(fb.SWAPAB, 16, 16, 1, 2), M=17) == CFG
    M, N, K = 16384, 4096, 12288
    assert fb.fp8_linear_workspace_size(M, N, K, None) > fb.NOALLOC_SCRATCH_BYTES
    assert f(M=M, N=N, K=K) == WS
    big = fb.make_config(fb.STANDARD, 64, 128, split_k=8)
    assert fb.fp8_linear_workspace_size(4096, 4096, 4096, big) > fb.NOALLOC_SCRATCH_BYTES
    assert f(M=4096, N=4096, K=4096, cfg=big) == WS
